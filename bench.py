#!/usr/bin/env python3
"""Benchmark of the QK-Normed MLA absorbed-latent decode step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
query absorption, cache append of the s_q new tokens, split-KV decode over the
paged latent cache, and the log-sum-exp combine.  The cache and every input are
resident in HBM before the timed region starts.  Steps rotate over several
replicas of the cache so that consecutive steps never re-read a cache that
could still sit in the 256 MB last-level cache (at least 512 MB is touched
between two reads of a replica).

Prints one JSON line.  ``value`` is the latent-cache read rate of the step:
algorithmic cache bytes (every visible token's latent + RoPE key + alpha^k,
once) divided by the step time.  ``roofline`` rates the decode kernel alone
(HIP events on its stream) against the 8 TB/s HBM peak; ``cpu_baseline`` is
the float64 CPU oracle timed on a bounded sample on the host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]
"""
from __future__ import annotations

import argparse
import hashlib
import heapq
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
MIN_ROTATION_BYTES = 512 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def split_len(T, P):
    """Tokens per split of a sequence of T tokens over P splits (whole pages)."""
    return 64 * math.ceil(math.ceil(T / P) / 64)


def default_splits(wl, seq_lens, cus=256):
    """Split count with the smallest estimated decode + combine time.

    Cost model, in units of one 32-token stage of one workgroup (about 2 us on
    MI355X for 128 query rows): a workgroup costs WG_FIXED (its prologue, which
    loads q~ and the first stages, and its epilogue, which writes the
    partials) plus its stage count.  The decode kernel deals work item w =
    (b P + p) R + r (R row blocks) to XCD w / ceil(n / 8), and each XCD's 32
    CUs take their items in order as they free up (one workgroup per CU); the
    combine costs its partial bytes, written and read back, at about 6 TB/s.
    With WG_FIXED = 8 this reproduces the measured decode times of the
    workloads within a few percent.  Equal lengths then get the count that
    fills the CUs once; a ragged batch (a few long sequences) gets more."""
    WG_FIXED, STAGE_US = 8.0, 2.0
    R = math.ceil(wl.s_q * wl.heads / 128)
    rows = wl.batch * wl.s_q * wl.heads
    best = None
    for P in range(1, min(512, max(1, 8 * cus // (wl.batch * R))) + 1):
        items = []
        for T in seq_lens:
            T = int(T)
            L = split_len(max(T, 1), P)
            for p in range(P):
                n = min(T, (p + 1) * L) - p * L
                items += [WG_FIXED + math.ceil(n / 32) if n > 0 else 1.0] * R
        per_xcd = math.ceil(len(items) / 8)
        makespan = 0.0
        for x in range(8):
            loads = [0.0] * (cus // 8)
            for c in items[x * per_xcd:(x + 1) * per_xcd]:
                heapq.heappush(loads, heapq.heappop(loads) + c)
            makespan = max(makespan, max(loads))
        t = makespan * STAGE_US + rows * P * wl.rank * 2 * 2 / 6e12 * 1e6
        if best is None or t < best[0] - 1e-9:
            best = (t, P)
    return best[1]


def kernel_source_sha():
    path = os.path.join(ROOT, "qk_normed_mla_amd", "csrc", "qkn_decode_mfma.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload):
    """HBM traffic of the decode kernel from committed rocprofv3 counter runs,
    only if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(wl, inp, target_s=12.0):
    """The oracle's decode over the stored state, timed on the host's cores on a
    sample of whole sequences (each with all its heads), scaled to cache GB/s.
    Building each sequence's stored state is set-up and is not timed."""
    from oracle import qkn_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    qi = O.query_image(wl, inp)
    offs = inp["tok_offsets"]
    nseq = len(inp["seq_lens"])
    prepared = []  # (wl, query image, cache image, block table, seq_lens, bytes) per sequence
    for b in range(min(nseq, 4)):
        T = int(inp["seq_lens"][b])
        pages = -(-T // 64)
        one = dict(inp)
        one.update(seq_lens=inp["seq_lens"][b:b + 1], tok_offsets=[0, T],
                   c=inp["c"][offs[b]:offs[b + 1]], k_rope=inp["k_rope"][offs[b]:offs[b + 1]],
                   block_table=np.arange(pages, dtype=np.int32)[None, :], num_pages=pages)
        one_wl = wl.replace(batch=1, seq_len=T, seq_len_range=None)
        img = O.full_cache_image(one_wl, one)
        prepared.append((one_wl, {k: v[b:b + 1] for k, v in qi.items()}, img,
                         one["block_table"], one["seq_lens"],
                         T * (2 * (wl.rank + wl.rope_dim) + 4 * wl.groups)))
    done, t_spent, nbytes = 0, 0.0, 0
    while t_spent < target_s:
        one_wl, q1, img, bt, sl, nb = prepared[done % len(prepared)]
        t0 = time.perf_counter()
        O.decode_on_image(one_wl, q1, img["kv"], img["alpha_k"], bt, sl, wl.num_splits)
        t_spent += time.perf_counter() - t0
        nbytes += nb
        done += 1
    return {"value": round(nbytes / t_spent / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} single-sequence decodes cycling over the first "
                      f"{len(prepared)} of {nseq} sequences (each {int(inp['seq_lens'][0])} "
                      f"tokens mean, all {wl.heads} heads), float64 NumPy decode over the "
                      f"stored bf16 cache, {t_spent:.1f} s of host time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--splits", type=int, default=0, help="split-KV partitions (0 = default)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-overhead", action="store_true", help="skip the alpha-free timing")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path "
                                   "is not sharded across GPUs (--gpus must be 1)"}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 4}), flush=True)
        return

    import qk_normed_mla_amd as Q
    import workloads as W
    from qk_normed_mla_amd.runner import DecodeRunner

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[args.workload]
    log(f"workload {wl.name}: generating inputs")
    inp = W.make_inputs(wl, seed=0)
    splits = args.splits or default_splits(wl, inp["seq_lens"])
    wl = wl.replace(num_splits=splits)
    flops, nbytes = W.flops_and_bytes(wl, inp["seq_lens"], 2 if wl.cache_dtype == "bf16" else 4)
    kind = Q.decode_kernel_kind(Q.dims_for(wl, inp["num_pages"]), splits)
    log(f"B={wl.batch} s_q={wl.s_q} H={wl.heads} G={wl.groups} T~{int(np.mean(inp['seq_lens']))} "
        f"splits={splits} kernel={'mfma' if kind == 1 else 'generic'} cache bytes={nbytes / 1e6:.1f} MB")

    r = DecodeRunner(wl, inp, num_splits=splits)
    log("filling the cache")
    r.fill_history()
    r.append_new()
    torch.cuda.synchronize()
    # bulk append: up to 2^18 history tokens in one qkn_mla_append call, inputs in
    # HBM (rewrites the same slots with the same values)
    hist = r.history_inputs()
    n_fill = int(hist[0].shape[0])
    fill = None
    if n_fill:
        r.append_tokens(*hist)
        fe = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            r.append_tokens(*hist)
            b.record()
            fe.append((a, b))
        torch.cuda.synchronize()
        fill_ms = min(a.elapsed_time(b) for a, b in fe)
        fill = {"tokens": n_fill, "ms": round(fill_ms, 3),
                "mtok_per_s": round(n_fill / fill_ms / 1e3, 2)}
        log(f"bulk append of {n_fill} tokens: {fill_ms:.3f} ms")
    del hist
    cache_bytes = r.kv.numel() * r.kv.element_size() + r.alpha_k.numel() * 4
    n_rep = max(2, math.ceil(MIN_ROTATION_BYTES / cache_bytes) + 1)
    kvs = [r.kv] + [r.kv.clone() for _ in range(n_rep - 1)]
    aks = [r.alpha_k] + [r.alpha_k.clone() for _ in range(n_rep - 1)]
    log(f"{n_rep} cache replicas of {cache_bytes / 1e6:.1f} MB rotate across steps")

    def step(k, flags=0):
        r.kv, r.alpha_k = kvs[k % n_rep], aks[k % n_rep]
        r.step(flags)

    def attn(k, flags=0):
        r.kv, r.alpha_k = kvs[k % n_rep], aks[k % n_rep]
        r.decode(flags)
        r.combine()

    def dec(k, flags=0):
        r.kv, r.alpha_k = kvs[k % n_rep], aks[k % n_rep]
        r.decode(flags)

    def attn_proj(k, flags=0):
        r.kv, r.alpha_k = kvs[k % n_rep], aks[k % n_rep]
        r.decode(flags)
        r.combine_project()

    # eager warm-up (also the reference for the graph check below)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    ref = r.o_latent.clone()

    def capture(fn, n, flags=0):
        """A HIP graph of n calls fn(k, flags), k = 0 .. n-1 (launch overhead of
        the Python binding stays outside the timed region)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for k in range(n):
                    fn(k, flags)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    def warm(g, seconds=0.25):
        """Untimed replays of g for about `seconds` of wall time: the GPU's
        clocks ramp up over the first milliseconds of sustained work, and the
        timings below are of the steady state."""
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()

    def timed(graphs, reps=5):
        """Per graph, the median over reps of one replay in ms.  The replays
        of all graphs are interleaved back to back (no host sync between
        them, so the GPU stays busy), each bracketed by HIP events on the
        replay stream, after two untimed rounds."""
        stream = torch.cuda.current_stream()
        for _ in range(2):
            for g in graphs:
                g.replay()
        ev = []
        for _ in range(reps):
            for g in graphs:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                ev.append((a, b))
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev]).reshape(reps, len(graphs))
        return [float(np.median(t[:, j])) for j in range(len(graphs))]

    # the timed region: exactly K steps, one graph replay, barrier + sync on both sides
    g_steps = capture(step, args.steps)
    g_steps.replay()                      # untimed replay
    torch.cuda.synchronize()
    # all replicas hold the same cache and the step is deterministic, so every
    # replayed step must leave exactly the eager result
    if not torch.equal(r.o_latent, ref):
        raise RuntimeError("graph replay differs from the eager step")
    warm(g_steps)
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    g_steps.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    if not torch.equal(r.o_latent, ref):
        raise RuntimeError("graph replay differs from the eager step")

    # the decode kernel alone, and decode + combine: back-to-back launches over
    # the rotating replicas.  QK-norm overhead: the decode kernel with and
    # without the inverse-RMS factors, the graphs' replays interleaved
    n_dec = max(40, 4 * n_rep)
    graphs = [capture(dec, n_dec), capture(attn, n_dec)]
    if not args.no_overhead:
        graphs.append(capture(dec, n_dec, Q.QKN_DECODE_NO_ALPHA))
    # decode + the combine with the value up-projection (qkn_mla_combine_project)
    graphs.append(capture(attn_proj, n_dec))
    warm(graphs[0])
    times = [t / n_dec for t in timed(graphs, reps=15)]
    dec_ms, attn_ms, proj_ms = times[0], times[1], times[-1]
    log(f"step {ms_per_step * 1e3:.1f} us, decode kernel {dec_ms * 1e3:.1f} us, "
        f"decode+combine {attn_ms * 1e3:.1f} us, decode+combine_project {proj_ms * 1e3:.1f} us")
    overhead = None
    if not args.no_overhead:
        overhead = round((dec_ms / times[2] - 1.0) * 100.0, 2)
        log(f"decode kernel {dec_ms * 1e3:.1f} us with alpha, {times[2] * 1e3:.1f} us without "
            f"({overhead:+.2f}%)")

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (dec_ms * 1e-3) / 1e9
    ai = flops / nbytes
    bound = "hbm" if ai < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.name)}
    else:
        tf = flops / (dec_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "traffic": load_traffic(wl.name)}
    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(wl, inp)
    out = {
        "metric": "MLA decode-attn latent-cache GB/s (% HBM peak) and us/step, h=128 r=512",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_combine_us": round(attn_ms * 1e3, 2),
        "decode_combine_project_us": round(proj_ms * 1e3, 2),
        "history_fill": fill,
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "qknorm_overhead_pct": overhead,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cache_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "s_q": wl.s_q, "heads": wl.heads,
                   "kv_groups": wl.groups, "rank": wl.rank, "rope_dim": wl.rope_dim,
                   "seq_len": int(np.mean(inp["seq_lens"])), "num_splits": splits,
                   "cache": wl.cache_dtype, "cache_bytes": nbytes, "flops": flops,
                   "kernel": "mfma" if kind == 1 else "generic"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
