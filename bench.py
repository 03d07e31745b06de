#!/usr/bin/env python3
"""Benchmark of the QK-Normed MLA absorbed-latent decode step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
query absorption, cache append of the s_q new tokens, split-KV decode over the
paged latent cache, and the log-sum-exp combine.  The cache and every input are
resident in HBM before the timed region starts.  Steps rotate over several
replicas of the cache so that consecutive steps never re-read a cache that
could still sit in the 256 MB last-level cache (at least 512 MB is touched
between two reads of a replica).

Prints one JSON line.  The headline workload (default ``mtp``: 64 sequences of
1024-16384 tokens, 4 query tokens per step, the largest configuration) sets
``value``: the latent-cache read rate of the step, algorithmic cache bytes
(every visible token's latent + RoPE key + alpha^k, once) divided by the step
time of exactly K timed steps.  ``roofline`` rates its decode kernel alone (HIP
events on its stream) against the peak of its bound: bf16 matrix-core FLOP/s
when the workload's arithmetic intensity is past the ridge, else 8 TB/s of HBM.
``workloads`` carries the same figures for the other bf16 workloads (dsv3,
grouped, long); ``sparse`` the selected-token decode (2048 listed tokens per
query out of 16384, its listed rows as the algorithmic bytes); ``prefill`` the
chunked prefill on the explicit path (a 512-token chunk over 8192 tokens);
``qknorm_sweep`` the cost of the inverse-RMS factors over a
batch-1 context sweep from 4k to 256k tokens; ``hbm_read_stream`` the HBM read
rate a plain read-only stream reaches on this GPU (each workload's decode rate
is also given as a fraction of it); ``cpu_baseline`` the float64 CPU
oracle timed on a bounded sample on the host's cores (and on one core).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mtp]
                    [--only] [--no-cpu] [--no-sweep]
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


def hbm_read_stream(Q, torch, timer, gib=2, launches=4):
    """The achievable HBM read rate on this GPU: qkn_mla_stream_read (every
    16-byte word of a 2 GiB buffer read once, non-temporal, as the decode reads
    the cache) captured `launches` times in a graph and timed like the
    kernels.  Also checks the XOR it returns against the buffer's."""
    import ctypes
    n = gib << 30
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib = Q.library()

    def call(_k=0):
        st = lib.qkn_mla_stream_read(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"qkn_mla_stream_read failed: {st}")

    call()
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32)))
    got = int(sink.cpu().numpy().view(np.uint32)[0])
    if got != want:
        raise RuntimeError(f"qkn_mla_stream_read: XOR {got:#x}, expected {want:#x}")
    g = timer.capture(call, launches)
    timer.warm(g)
    ms = timer.timed([g], reps=7)[0] / launches
    gbs = n / (ms * 1e-3) / 1e9
    log(f"HBM read stream: {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of {HBM_PEAK_GBS:.0f})")
    del buf
    return {"kernel": "qkn_mla_stream_read", "bytes_per_launch": n, "gbs": round(gbs, 1),
            "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4)}


def split_len(T, P):
    """Tokens per split of a sequence of T tokens over P splits (whole pages)."""
    return 64 * math.ceil(math.ceil(T / P) / 64)


def default_splits(wl, seq_lens, cus=256):
    """Split count with the smallest estimated decode + combine time.

    Cost model, in units of one 32-token stage of one workgroup (about 2 us on
    MI355X for 128 query rows): a workgroup costs WG_FIXED (its prologue, which
    loads q~ and the first stages, and its epilogue, which writes the
    partials) plus its stage count.  The decode kernel deals its items the
    way the kernel does: equal lengths (or more than 64 sequences) in index
    order, XCD x taking the x-th eighth of the items; a ragged batch of up to
    64 sequences longest sequence first, its (sequence, split) pairs dealt
    round-robin over the XCDs, the row blocks of a pair together.  Each XCD's
    32 CUs take their items in order as they free up (one workgroup per CU);
    the combine costs its partial bytes, written and read back, at about
    6 TB/s.  Equal lengths then get the count that fills the CUs once; a
    ragged batch gets the count that best evens out its long sequences."""
    WG_FIXED, STAGE_US = 8.0, 2.0
    R = math.ceil(wl.s_q * wl.heads / 128)
    rows = wl.batch * wl.s_q * wl.heads
    lens = [int(T) for T in seq_lens]
    ragged = len(lens) <= 64 and len(set(lens)) > 1
    order = sorted(range(len(lens)), key=lambda b: (-lens[b], b)) if ragged else range(len(lens))
    best = None
    for P in range(1, min(512, max(1, 8 * cus // (wl.batch * R))) + 1):
        queues = [[] for _ in range(8)]
        items = []
        for b in order:
            T = lens[b]
            L = split_len(max(T, 1), P)
            for p in range(P):
                n = min(T, (p + 1) * L) - p * L
                items.append([WG_FIXED + math.ceil(n / 32) if n > 0 else 1.0] * R)
        if ragged:
            for k, its in enumerate(items):
                queues[k % 8] += its
        else:
            flat = [c for its in items for c in its]
            per_xcd = math.ceil(len(flat) / 8)
            queues = [flat[x * per_xcd:(x + 1) * per_xcd] for x in range(8)]
        makespan = 0.0
        for q in queues:
            loads = [0.0] * (cus // 8)
            for c in q:
                heapq.heappush(loads, heapq.heappop(loads) + c)
            makespan = max(makespan, max(loads))
        t = makespan * STAGE_US + rows * P * wl.rank * 2 * 2 / 6e12 * 1e6
        if best is None or t < best[0] - 1e-9:
            best = (t, P)
    return best[1]


def gqa_splits(wl, seq_lens, cus=256):
    """Split count of the GQA-path attention with the smallest estimated
    attention + combine time.  Cost model, in units of one 32-key tile of one
    workgroup: a workgroup costs GQA_WG_FIXED (loading its queries, writing its
    output) plus its tiles; the workgroups are dealt to the 8 XCDs as the
    kernel numbers them (ragged batches of up to 64: the (sequence, split)
    pairs, longest sequence first, round robin over the XCDs, the token and
    head blocks of a pair together; otherwise XCD x takes the x-th eighth in
    order), and each XCD's workgroups go in order to the least-loaded of its 32 CUs; a
    CU holding two or more runs them at PAIR_GAIN times the throughput of one
    (two waves per SIMD).  The combine costs its half partials, written and
    read back, at about 3 TB/s, or the latency of walking a row's partials
    (four at a time in each of 1 or 4 lane groups) when that is longer.  At
    most 256 splits.  The constants are fitted to measured attention times of
    the mtp, dsv3, grouped and long workloads at several split counts."""
    GQA_WG_FIXED, TILE_US, PAIR_GAIN = 8.0, 1.24, 1.2
    tpw = 4
    while tpw > 1 and tpw // 2 >= wl.s_q and (wl.heads // wl.groups // 32) % (8 // tpw) == 0:
        tpw //= 2
    per_pair = math.ceil(wl.s_q / tpw) * (wl.heads // 32 // (4 // tpw))
    rows = wl.batch * wl.s_q * wl.heads
    lens = [int(T) for T in seq_lens]
    ragged = len(lens) <= 64 and len(set(lens)) > 1
    order = sorted(range(len(lens)), key=lambda b: (-lens[b], b)) if ragged else range(len(lens))
    best = None
    for P in range(1, max(1, min(256, 8 * cus // (wl.batch * per_pair))) + 1):
        pairs = []
        for b in order:
            T = lens[b]
            L = split_len(max(T, 1), P)
            for p in range(P):
                n = min(T, (p + 1) * L) - p * L
                pairs.append([GQA_WG_FIXED + math.ceil(n / 32) if n > 0 else 1.0] * per_pair)
        if ragged:
            xcd_items = [sum(pairs[x::8], []) for x in range(8)]
        else:
            flat = sum(pairs, [])
            per_xcd = math.ceil(len(flat) / 8)
            xcd_items = [flat[x * per_xcd:(x + 1) * per_xcd] for x in range(8)]
        makespan = 0.0
        for items in xcd_items:
            loads = [(0.0, 0, c) for c in range(cus // 8)]  # (work, items, cu)
            heapq.heapify(loads)
            for c in items:
                w, k, cu = heapq.heappop(loads)
                heapq.heappush(loads, (w + c, k + 1, cu))
            makespan = max(makespan, max(w / (PAIR_GAIN if k >= 2 else 1.0) for w, k, _ in loads))
        walk = P / 16 if P >= 32 else P / 4  # rounds of partial loads per lane group
        comb = max(rows * P * wl.head_dim * 2 * 2 / 3e12 * 1e6, walk * 0.35) if P > 1 else 0.0
        t = makespan * TILE_US + comb
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, target_s=12.0, one_core_s=5.0):
    """The oracle's decode over the stored state, timed on the host's cores on a
    sample of whole sequences (each with all its heads), scaled to cache GB/s;
    then the same on one core.  Building each sequence's stored state is
    set-up and is not timed."""
    from oracle import qkn_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
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

    def run(seconds):
        done, t_spent, nbytes = 0, 0.0, 0
        while t_spent < seconds:
            one_wl, q1, img, bt, sl, nb = prepared[done % len(prepared)]
            t0 = time.perf_counter()
            O.decode_on_image(one_wl, q1, img["kv"], img["alpha_k"], bt, sl, wl.num_splits)
            t_spent += time.perf_counter() - t0
            nbytes += nb
            done += 1
        return done, t_spent, nbytes

    done, t_spent, nbytes = run(target_s)
    with threadpool_limits(limits=1):
        done1, t1, nbytes1 = run(one_core_s)
    lens = [int(x) for x in inp["seq_lens"][:len(prepared)]]
    return {"value": round(nbytes / t_spent / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(),
            "one_core": {"value": round(nbytes1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "sample": f"{done1} decodes, {t1:.1f} s"},
            "sample": f"{done} single-sequence decodes cycling over the first "
                      f"{len(prepared)} of {nseq} sequences (lengths {lens}, all {wl.heads} "
                      f"heads, {wl.s_q} query tokens each), float64 NumPy decode over the "
                      f"stored bf16 cache, {t_spent:.1f} s of host time"}


class Timer:
    """HIP graphs of back-to-back launches and their steady-state timing."""

    def __init__(self, torch):
        self.torch = torch

    def capture(self, fn, n):
        """A HIP graph of n calls fn(k), k = 0 .. n-1 (launch overhead of the
        Python binding stays outside the timed region)."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for k in range(n):
                    fn(k)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    def warm(self, g, seconds=0.25):
        """Untimed replays of g for about `seconds` of wall time: the GPU's
        clocks ramp up over the first milliseconds of sustained work, and the
        timings below are of the steady state."""
        torch = self.torch
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()

    def timed(self, graphs, reps=5):
        """Per graph, the median over reps of one replay in ms.  The replays
        of all graphs are interleaved back to back (no host sync between
        them, so the GPU stays busy), each bracketed by HIP events on the
        replay stream, after two untimed rounds."""
        torch = self.torch
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


def roofline_of(flops, nbytes, seconds, traffic):
    """The decode kernel against the peak of its bound (matrix-core FLOP/s past
    the ridge, HBM bandwidth below it)."""
    ai = flops / nbytes
    if ai < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        a = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic}
    a = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(a / BF16_PEAK_TFLOPS, 4), "traffic": traffic}


def measure(Q, W, torch, timer, wl, inp, splits, *, steps, warmup, overhead=True,
            history_fill=False):
    """Every figure of one workload: the step (exactly `steps` timed steps in
    one graph replay), the decode kernel alone, decode + combine, decode +
    combine with the value up-projection, and the decode kernel without the
    inverse-RMS factors."""
    from qk_normed_mla_amd.runner import DecodeRunner

    flops, nbytes = W.flops_and_bytes(wl, inp["seq_lens"], 2 if wl.cache_dtype == "bf16" else 4)
    kind = Q.decode_kernel_kind(Q.dims_for(wl, inp["num_pages"]), splits)
    log(f"{wl.name}: B={wl.batch} s_q={wl.s_q} H={wl.heads} G={wl.groups} "
        f"T~{int(np.mean(inp['seq_lens']))} splits={splits} kernel={'mfma' if kind == 1 else 'generic'} "
        f"cache bytes={nbytes / 1e6:.1f} MB")
    r = DecodeRunner(wl, inp, num_splits=splits)
    r.fill_history()
    r.prepare()                           # the query side and the new tokens
    torch.cuda.synchronize()
    fill = None
    if history_fill:
        # bulk append: up to 2^18 history tokens in one qkn_mla_append call,
        # inputs in HBM (rewrites the same slots with the same values)
        hist = r.history_inputs()
        n_fill = int(hist[0].shape[0])
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
            fill = {"workload": wl.name, "tokens": n_fill, "ms": round(fill_ms, 3),
                    "mtok_per_s": round(n_fill / fill_ms / 1e3, 2)}
            log(f"bulk append of {n_fill} tokens: {fill_ms:.3f} ms")
        del hist
    cache_bytes = r.kv.numel() * r.kv.element_size() + r.alpha_k.numel() * 4
    n_rep = max(2, math.ceil(MIN_ROTATION_BYTES / cache_bytes) + 1)
    kvs = [r.kv] + [r.kv.clone() for _ in range(n_rep - 1)]
    aks = [r.alpha_k] + [r.alpha_k.clone() for _ in range(n_rep - 1)]
    log(f"{n_rep} cache replicas of {cache_bytes / 1e6:.1f} MB rotate across launches")

    def use(k):
        r.kv, r.alpha_k = kvs[k % n_rep], aks[k % n_rep]

    # restarts of the exact fixed-reference softmax, with and without the factors
    restarted = {}
    for name, fl in (("alpha", 0), ("no_alpha", Q.QKN_DECODE_NO_ALPHA)):
        r.err_flag.zero_()
        r.decode(fl)
        torch.cuda.synchronize()
        restarted[name] = bool(int(r.err_flag.item()) & Q.QKN_FLAG_RESTART)
    r.err_flag.zero_()

    # eager warm-up (also the reference for the graph check below)
    for k in range(warmup):
        use(k)
        r.step()
    torch.cuda.synchronize()
    ref = r.o_latent.clone()

    def step(k):
        use(k)
        r.step()

    g_steps = timer.capture(step, steps)
    g_steps.replay()                      # untimed replay
    torch.cuda.synchronize()
    # all replicas hold the same cache and the step is deterministic, so every
    # replayed step must leave exactly the eager result
    if not torch.equal(r.o_latent, ref):
        raise RuntimeError("graph replay differs from the eager step")
    timer.warm(g_steps)
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    g_steps.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / steps
    if not torch.equal(r.o_latent, ref):
        raise RuntimeError("graph replay differs from the eager step")

    # back-to-back launches over the rotating replicas: the decode kernel
    # alone, decode + combine, decode + combine_project; the decode kernel
    # without the factors; the graphs' replays interleaved
    n_dec = max(40, 4 * n_rep)

    def dec(k):
        use(k)
        r.decode()

    def attn(k):
        use(k)
        r.decode()
        r.combine()

    def attn_proj(k):
        use(k)
        r.decode()
        r.combine_project()

    def dec_plain(k):
        use(k)
        r.decode(Q.QKN_DECODE_NO_ALPHA)

    fns = [dec, attn, attn_proj] + ([dec_plain] if overhead else [])
    graphs = [timer.capture(f, n_dec) for f in fns]
    timer.warm(graphs[0])
    times = [t / n_dec for t in timer.timed(graphs, reps=15)]
    dec_ms, attn_ms, proj_ms = times[0], times[1], times[2]
    log(f"{wl.name}: step {ms_per_step * 1e3:.1f} us, decode kernel {dec_ms * 1e3:.1f} us, "
        f"decode+combine {attn_ms * 1e3:.1f} us, decode+combine_project {proj_ms * 1e3:.1f} us")
    ov = None
    if overhead:
        ov = round((dec_ms / times[3] - 1.0) * 100.0, 2)
        log(f"{wl.name}: decode kernel {dec_ms * 1e3:.1f} us with alpha, {times[3] * 1e3:.1f} us "
            f"without ({ov:+.2f}%)" + ("; the alpha-free kernel restarted" if restarted["no_alpha"] else ""))
    out = {
        "workload": wl.name, "batch": wl.batch, "s_q": wl.s_q, "heads": wl.heads,
        "kv_groups": wl.groups, "rank": wl.rank, "rope_dim": wl.rope_dim,
        "seq_len": int(np.mean(inp["seq_lens"])), "num_splits": splits,
        "kernel": "mfma" if kind == 1 else "generic",
        "cache_bytes": nbytes, "flops": flops,
        "us_per_step": round(ms_per_step * 1e3, 2),
        "step_cache_gbs": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "decode_combine_us": round(attn_ms * 1e3, 2),
        "decode_combine_project_us": round(proj_ms * 1e3, 2),
        "decode_hbm_frac": round(nbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_mfma_frac": round(flops / (dec_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "decode_combine_hbm_frac": round(nbytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "qknorm_overhead_pct": None if (ov is None or restarted["no_alpha"]) else ov,
        "restarted": restarted,
        # HBM bytes per decode launch from the committed counter runs (null
        # when they were taken on another kernel source)
        "decode_hbm_traffic": load_traffic(wl.name),
    }
    if ov is not None and restarted["no_alpha"]:
        out["qknorm_overhead_note"] = ("not comparable: without the inverse-RMS factors the "
                                       "logits outgrow the fixed softmax reference and the "
                                       f"kernel takes the exact restart ({ov:+.2f}% measured)")
    res = {"summary": out, "ms_per_step": ms_per_step, "dec_ms": dec_ms, "flops": flops,
           "nbytes": nbytes, "fill": fill}
    del graphs, g_steps, kvs, aks, r
    torch.cuda.empty_cache()
    return res


def measure_sparse(Q, W, torch, timer, splits=8):
    """Selected-token decode: 32 sequences of 16384 tokens (shuffled pages),
    each query listing 2048 of its tokens at random; the decode kernel alone
    and decode + combine, over rotating cache replicas.  Algorithmic bytes:
    the listed rows (latent, RoPE key and alpha^k of each)."""
    from qk_normed_mla_amd.runner import DecodeRunner

    wl = W.WORKLOADS["sparse"].replace(num_splits=splits)
    log("sparse: generating inputs")
    inp = W.make_inputs(wl, seed=0)
    K = W.SPARSE_LIST_LEN
    sel = W.make_selection(wl, inp["seq_lens"], K, seed=1)
    n_listed = int(np.sum(sel >= 0))
    row_bytes = (wl.rank + wl.rope_dim) * 2 + 4 * wl.groups
    nbytes = n_listed * row_bytes
    flops = n_listed * wl.heads * (4 * wl.rank + 2 * wl.rope_dim)
    r = DecodeRunner(wl, inp, num_splits=splits)
    r.fill_history()
    r.prepare()
    idx = torch.from_numpy(sel).to("cuda")
    torch.cuda.synchronize()
    cache_bytes = r.kv.numel() * r.kv.element_size() + r.alpha_k.numel() * 4
    n_rep = max(2, math.ceil(MIN_ROTATION_BYTES / cache_bytes) + 1)
    kvs = [r.kv] + [r.kv.clone() for _ in range(n_rep - 1)]
    aks = [r.alpha_k] + [r.alpha_k.clone() for _ in range(n_rep - 1)]

    def dec(k):
        Q.qkn_mla_decode_sparse(r.dims, r.q_tilde, r.alpha_q, r.q_rope_normed, kvs[k % n_rep],
                                aks[k % n_rep], r.block_table, r.seq_lens, idx, splits, 0,
                                r.o_partial, r.lse_partial, r.err_flag)

    def attn(k):
        dec(k)
        r.combine()

    r.err_flag.zero_()
    attn(0)
    torch.cuda.synchronize()
    if int(r.err_flag.item()) != 0:
        raise RuntimeError("the sparse decode flagged its inputs")
    n_dec = max(40, 4 * n_rep)
    graphs = [timer.capture(f, n_dec) for f in (dec, attn)]
    timer.warm(graphs[0])
    dec_ms, attn_ms = [t / n_dec for t in timer.timed(graphs, reps=15)]
    log(f"sparse: B={wl.batch} T={wl.seq_len} K={K} splits={splits} listed bytes "
        f"{nbytes / 1e6:.1f} MB: decode kernel {dec_ms * 1e3:.1f} us, decode+combine "
        f"{attn_ms * 1e3:.1f} us")
    return {"workload": "sparse", "batch": wl.batch, "heads": wl.heads, "seq_len": wl.seq_len,
            "list_len": K, "num_splits": splits, "listed_bytes": nbytes, "flops": flops,
            "decode_kernel_us": round(dec_ms * 1e3, 2),
            "decode_combine_us": round(attn_ms * 1e3, 2),
            "decode_gbs": round(nbytes / (dec_ms * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(nbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def measure_prefill(Q, W, torch, timer, cpu=False):
    """Chunked prefill on the explicit path: 2 sequences of 8192 tokens whose
    last 512 are the chunk; the query side, the materialised keys and values of
    the whole cache, and the causal attention, each timed back to back.  FLOPs:
    the attention's q^.k^ + q^R.k^R and P.V products over each query's visible
    keys, and the expansion's two products over every cached token."""
    from qk_normed_mla_amd.runner import DecodeRunner

    wl = W.WORKLOADS["prefill"]
    log("prefill: generating inputs")
    inp = W.make_inputs(wl, seed=0)
    r = DecodeRunner(wl, inp)
    r.fill_history()
    r.append_new()
    r.alloc_prefill()
    torch.cuda.synchronize()
    vis = sum(int(T) - wl.s_q + i + 1 for T in inp["seq_lens"] for i in range(wl.s_q))
    att_flops = vis * wl.heads * 2 * (2 * wl.head_dim + wl.rope_dim)
    exp_flops = int(np.sum(inp["seq_lens"])) * wl.groups * 2 * (2 * wl.rank * wl.head_dim)
    n = 20
    graphs = [timer.capture(lambda k: r.prefill_query(), n),
              timer.capture(lambda k: r.prefill_expand(), n),
              timer.capture(lambda k: r.prefill_attend(), n)]
    timer.warm(graphs[2])
    q_ms, e_ms, a_ms = [t / n for t in timer.timed(graphs, reps=9)]
    log(f"prefill: B={wl.batch} chunk={wl.s_q} T={wl.seq_len}: query {q_ms * 1e3:.1f} us, "
        f"expand {e_ms * 1e3:.1f} us, attend {a_ms * 1e3:.1f} us "
        f"({att_flops / (a_ms * 1e-3) / 1e12:.0f} TFLOP/s)")
    return {"workload": "prefill", "batch": wl.batch, "chunk": wl.s_q, "seq_len": wl.seq_len,
            "heads": wl.heads, "query_us": round(q_ms * 1e3, 2), "expand_us": round(e_ms * 1e3, 2),
            "attend_us": round(a_ms * 1e3, 2), "attend_flops": att_flops,
            "attend_tflops": round(att_flops / (a_ms * 1e-3) / 1e12, 1),
            "attend_mfma_frac": round(att_flops / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "expand_flops": exp_flops,
            "expand_tflops": round(exp_flops / (e_ms * 1e-3) / 1e12, 1),
            "cpu_oracle": cpu_oracle_sample("prefill", wl, inp) if cpu else None}


def _one_sequence(wl, inp, b):
    """Workload and inputs of sequence b alone, its pages renumbered 0 .. n-1."""
    offs = inp["tok_offsets"]
    T = int(inp["seq_lens"][b])
    pages = -(-T // 64)
    one = dict(inp)
    one.update(seq_lens=inp["seq_lens"][b:b + 1], tok_offsets=np.array([0, T]),
               c=inp["c"][offs[b]:offs[b + 1]], k_rope=inp["k_rope"][offs[b]:offs[b + 1]],
               q=inp["q"][b:b + 1], q_rope=inp["q_rope"][b:b + 1],
               block_table=np.arange(pages, dtype=np.int32)[None, :], num_pages=pages)
    return wl.replace(batch=1, seq_len=T, seq_len_range=None), one


def cpu_oracle_sample(kind, wl, inp, seconds=3.0):
    """The oracle's attention of the GQA path (kind "gqa") or of the chunked
    prefill ("prefill") on the host cores, on a sample: the first sequence,
    every head of its last query token, repeated for about `seconds`.  The
    stored images are built first and not timed.  FLOPs as the GPU figure
    counts them (q^.k^ + q^R.k^R and P.V over the visible keys)."""
    from oracle import qkn_oracle as O
    from threadpoolctl import threadpool_info
    cores = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    one_wl, one = _one_sequence(wl, inp, 0)
    T = int(one["seq_lens"][0])
    rows = [(0, wl.s_q - 1, h) for h in range(wl.heads)]
    qi = O.prefill_query_image(one_wl, one)
    if kind == "gqa":
        img = O.gqa_full_image(one_wl, one)["kvg"]
        run = lambda: O.gqa_decode_on_image(one_wl, qi, img, one["block_table"], one["seq_lens"], 1,  # noqa: E731
                                            rows=rows)
    else:
        cache = O.full_cache_image(one_wl, one)
        e = O.expand_image(one_wl, cache["kv"], cache["alpha_k"], one["block_table"], one["seq_lens"],
                           one["w_k"], one["w_v"], one["gamma_k"], -(-T // 64) * 64)
        run = lambda: O.prefill_on_images(one_wl, qi, e, cache["kv"], one["block_table"],  # noqa: E731
                                          one["seq_lens"], rows=rows)
    done, spent = 0, 0.0
    while spent < seconds:
        t0 = time.perf_counter()
        run()
        spent += time.perf_counter() - t0
        done += 1
    flops = done * wl.heads * T * 2 * (2 * wl.head_dim + wl.rope_dim)
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "sample": f"{done} attentions of the last query token of one {T}-token "
                                        f"sequence, all {wl.heads} heads, float64 NumPy over the stored "
                                        f"images, {spent:.1f} s of host time"}


def measure_gqa(Q, W, torch, timer, name, absorbed_step_us=None, sweep=(), cpu=False):
    """The GQA path on one workload: the step (query side, GQA append of the
    s_q new tokens, attention over the per-group cache with its combine) and
    the attention call alone, over rotating cache replicas.  FLOPs: the
    q^.k^ + q^R.k^R and P.V products over each query's visible keys; bytes: the
    cache rows read (2 G d half + d_R bf16 per token).  ``sweep``: split
    counts to time the attention call at as well (logged)."""
    from qk_normed_mla_amd.runner import DecodeRunner

    wl = W.WORKLOADS[name]
    log(f"gqa {name}: generating inputs")
    inp = W.make_inputs(wl, seed=0)
    splits = gqa_splits(wl, inp["seq_lens"])
    r = DecodeRunner(wl, inp)
    r.alloc_gqa(splits)
    r.err_flag.zero_()
    r.gqa_fill_history()
    r.gqa_step()
    torch.cuda.synchronize()
    if int(r.err_flag.item()) != 0:
        raise RuntimeError("the GQA path flagged its inputs")
    del r.kv, r.alpha_k  # the latent cache is not used on this path
    torch.cuda.empty_cache()
    lens = [int(T) for T in inp["seq_lens"]]
    vis = sum(T - wl.s_q + i + 1 for T in lens for i in range(wl.s_q))
    flops = vis * wl.heads * 2 * (2 * wl.head_dim + wl.rope_dim)
    nbytes = sum(lens) * Q.gqa_row_words(r.dims) * 2
    cache_bytes = r.kvg.numel() * 2
    n_rep = max(2, math.ceil(MIN_ROTATION_BYTES / cache_bytes) + 1)
    kvgs = [r.kvg] + [r.kvg.clone() for _ in range(n_rep - 1)]
    n = max(20, 4 * n_rep)

    def attend_graph():
        return timer.capture(lambda k: r.gqa_attend(kvg=kvgs[k % n_rep]), n)

    out_sweep = []
    for P_ in sweep:
        r.set_gqa_splits(P_)
        g = attend_graph()
        timer.warm(g)
        t = timer.timed([g], reps=9)[0] / n
        out_sweep.append({"splits": P_, "attend_us": round(t * 1e3, 2)})
        log(f"gqa {name}: splits {P_}: attend {t * 1e3:.1f} us")
        del g
    r.set_gqa_splits(splits)
    graphs = [timer.capture(lambda k: r.gqa_step(kvg=kvgs[k % n_rep]), n), attend_graph()]
    timer.warm(graphs[1])
    step_ms, att_ms = [t / n for t in timer.timed(graphs, reps=15)]
    tf = flops / (att_ms * 1e-3) / 1e12
    log(f"gqa {name}: B={wl.batch} s_q={wl.s_q} G={wl.groups} splits={splits}: step "
        f"{step_ms * 1e3:.1f} us, attention+combine {att_ms * 1e3:.1f} us ({tf:.0f} TFLOP/s, "
        f"{nbytes / (att_ms * 1e-3) / 1e9:.0f} GB/s of cache rows)")
    res = {"workload": name, "batch": wl.batch, "s_q": wl.s_q, "heads": wl.heads,
           "kv_groups": wl.groups, "num_splits": splits, "cache_row_bytes": Q.gqa_row_words(r.dims) * 2,
           "flops": flops, "cache_bytes": nbytes, "step_us": round(step_ms * 1e3, 2),
           "attend_us": round(att_ms * 1e3, 2), "attend_tflops": round(tf, 1),
           "attend_mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
           "attend_gbs": round(nbytes / (att_ms * 1e-3) / 1e9, 1),
           "attend_hbm_frac": round(nbytes / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if absorbed_step_us:
        res["absorbed_step_us"] = absorbed_step_us
        res["speedup_vs_absorbed"] = round(absorbed_step_us / (step_ms * 1e3), 3)
    if out_sweep:
        res["split_sweep"] = out_sweep
    if cpu:
        log(f"gqa {name}: timing the CPU oracle on a sample")
        res["cpu_oracle"] = cpu_oracle_sample("gqa", wl, inp)
    del kvgs, graphs, r
    torch.cuda.empty_cache()
    return res


def qknorm_sweep(Q, W, torch, timer, lengths=(4096, 8192, 16384, 32768, 65536, 131072, 262144)):
    """Batch-1 decode + combine (128 heads, r = 512, d_R = 64, latent scales
    log-normal sigma 0.5) with and without the inverse-RMS factors over a
    context sweep.  One 262144-token cache is drawn; three copies of it are
    resident, and each launch reads a different window of pages (a block table
    per window), so that at least 512 MB are read between two reads of one
    window and none is served from the last-level cache."""
    from qk_normed_mla_amd.runner import DecodeRunner

    T_max = max(lengths)
    wl = W.WORKLOADS["long"].replace(name="sweep", seq_len=T_max, latent_log_sigma=0.5)
    inp = W.make_inputs(wl, seed=1)
    r = DecodeRunner(wl, inp, num_splits=1)
    r.fill_history()
    r.append_new()
    torch.cuda.synchronize()
    copies = 3
    pages = int(inp["num_pages"])
    kv = torch.cat([r.kv] * copies, dim=0)
    ak = torch.cat([r.alpha_k] * copies, dim=0)
    del r
    torch.cuda.empty_cache()
    out = []
    for T in lengths:
        wlT = wl.replace(seq_len=T)
        P = default_splits(wlT, [T])
        ppw = -(-T // 64)                        # pages per window
        n_win = (pages * copies) // ppw
        bytes_T = T * (2 * (wl.rank + wl.rope_dim) + 4 * wl.groups)
        need = min(n_win, math.ceil(MIN_ROTATION_BYTES / bytes_T) + 1)
        n_launch = max(24, need)
        tables = [torch.arange(w * ppw, (w + 1) * ppw, dtype=torch.int32, device="cuda")[None, :]
                  for w in range(need)]
        dims = Q.dims_for(wlT, pages * copies)
        inpT = dict(inp, seq_lens=np.array([T], np.int32))
        rT = DecodeRunner(wlT, dict(inpT, num_pages=1, block_table=np.zeros((1, ppw), np.int32),
                                    c=inp["c"][:T], k_rope=inp["k_rope"][:T],
                                    tok_offsets=np.array([0, T])), num_splits=P)
        rT.absorb()
        ws = Q.alloc_decode_workspace(dims, P)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")

        def attend(k, flags, rT=rT, dims=dims, tables=tables, ws=ws, P=P, err=err):
            Q.qkn_mla_decode_attend(dims, rT.q_tilde, rT.alpha_q, rT.q_rope_normed, kv, ak,
                                    tables[k % len(tables)], rT.seq_lens, P, flags, ws,
                                    rT.o_latent, rT.lse, err)

        restarted = {}
        for name, fl in (("alpha", 0), ("no_alpha", Q.QKN_DECODE_NO_ALPHA)):
            err.zero_()
            for k in range(len(tables)):
                attend(k, fl)
            torch.cuda.synchronize()
            restarted[name] = bool(int(err.item()) & Q.QKN_FLAG_RESTART)
        graphs = [timer.capture(lambda k: attend(k, 0), n_launch),
                  timer.capture(lambda k: attend(k, Q.QKN_DECODE_NO_ALPHA), n_launch)]
        timer.warm(graphs[0], 0.15)
        t_a, t_n = [t / n_launch for t in timer.timed(graphs, reps=11)]
        ov = (t_a / t_n - 1.0) * 100.0
        rec = {"seq_len": T, "num_splits": P, "decode_combine_us": round(t_a * 1e3, 2),
               "no_alpha_us": round(t_n * 1e3, 2),
               "cache_gbs": round(bytes_T / (t_a * 1e-3) / 1e9, 1),
               "overhead_pct": None if restarted["no_alpha"] else round(ov, 2),
               "restarted": restarted}
        log(f"sweep T={T}: {t_a * 1e3:.1f} us with alpha, {t_n * 1e3:.1f} us without "
            f"({ov:+.2f}%), splits {P}, windows {len(tables)}")
        out.append(rec)
        del graphs, rT, ws
        torch.cuda.empty_cache()
    del kv, ak
    torch.cuda.empty_cache()
    return out


def profile_run(Q, W, torch, name, launches):
    """Only `launches` eager decode + combine calls of one workload over its
    rotating cache replicas, after one warm-up call: the program the
    rocprofv3 counter and trace summaries are taken from."""
    from qk_normed_mla_amd.runner import DecodeRunner

    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)
    splits = default_splits(wl, inp["seq_lens"])
    r = DecodeRunner(wl, inp, num_splits=splits)
    r.fill_history()
    r.prepare()
    cache_bytes = r.kv.numel() * r.kv.element_size() + r.alpha_k.numel() * 4
    n_rep = max(2, math.ceil(MIN_ROTATION_BYTES / cache_bytes) + 1)
    kvs = [r.kv] + [r.kv.clone() for _ in range(n_rep - 1)]
    aks = [r.alpha_k] + [r.alpha_k.clone() for _ in range(n_rep - 1)]
    torch.cuda.synchronize()
    for k in range(launches + 1):
        r.kv, r.alpha_k = kvs[k % n_rep], aks[k % n_rep]
        r.decode()
        r.combine()
    torch.cuda.synchronize()
    print(json.dumps({"profiled": name, "num_splits": splits, "launches": launches + 1,
                      "replicas": n_rep}), flush=True)


def profile_gqa_run(Q, W, torch, name, launches):
    """Only `launches` eager GQA-path steps (query side, append of the new
    tokens, attention and combine) of one workload over rotating replicas of
    its cache, after one warm-up step."""
    from qk_normed_mla_amd.runner import DecodeRunner

    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)
    splits = gqa_splits(wl, inp["seq_lens"])
    r = DecodeRunner(wl, inp)
    r.alloc_gqa(splits)
    r.gqa_fill_history()
    del r.kv, r.alpha_k
    n_rep = max(2, math.ceil(MIN_ROTATION_BYTES / (r.kvg.numel() * 2)) + 1)
    kvgs = [r.kvg] + [r.kvg.clone() for _ in range(n_rep - 1)]
    torch.cuda.synchronize()
    for k in range(launches + 1):
        r.gqa_step(kvg=kvgs[k % n_rep])
    torch.cuda.synchronize()
    print(json.dumps({"profiled": f"gqa {name}", "num_splits": splits, "launches": launches + 1,
                      "replicas": n_rep}), flush=True)


def profile_prefill_run(Q, W, torch, launches):
    """Only `launches` eager prefill passes (query side, expansion, attention)
    of the chunked-prefill workload, after one warm-up pass."""
    from qk_normed_mla_amd.runner import DecodeRunner

    wl = W.WORKLOADS["prefill"]
    inp = W.make_inputs(wl, seed=0)
    r = DecodeRunner(wl, inp)
    r.fill_history()
    r.append_new()
    r.alloc_prefill()
    torch.cuda.synchronize()
    for _ in range(launches + 1):
        r.prefill_query()
        r.prefill_expand()
        r.prefill_attend()
    torch.cuda.synchronize()
    print(json.dumps({"profiled": "prefill", "launches": launches + 1}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mtp", help="the headline workload")
    ap.add_argument("--splits", type=int, default=0, help="split-KV partitions (0 = default)")
    ap.add_argument("--only", action="store_true", help="the headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-sweep", action="store_true", help="skip the batch-1 QK-norm sweep")
    ap.add_argument("--no-overhead", action="store_true", help="skip the alpha-free timings")
    ap.add_argument("--profile", type=int, default=0, metavar="N",
                    help="only run N + 1 eager decode + combine calls of --workload (the "
                         "program rocprofv3 profiles) and exit")
    ap.add_argument("--profile-path", default="decode", choices=("decode", "gqa", "prefill"),
                    help="what --profile runs: the latent decode + combine, the GQA-path step "
                         "or the chunked prefill")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path "
                                   "is not sharded across GPUs (--gpus must be 1)"}))
        sys.exit(2)

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

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    Q.library()
    if args.profile:
        if args.profile_path == "gqa":
            profile_gqa_run(Q, W, torch, args.workload, args.profile)
        elif args.profile_path == "prefill":
            profile_prefill_run(Q, W, torch, args.profile)
        else:
            profile_run(Q, W, torch, args.workload, args.profile)
        return
    timer = Timer(torch)

    def run(name, headline):
        wl = W.WORKLOADS[name]
        log(f"workload {name}: generating inputs")
        inp = W.make_inputs(wl, seed=0)
        splits = (args.splits if headline and args.splits else 0) or default_splits(wl, inp["seq_lens"])
        wl = wl.replace(num_splits=splits)
        res = measure(Q, W, torch, timer, wl, inp, splits,
                      steps=args.steps if headline else 10,
                      warmup=args.warmup if headline else 3,
                      overhead=not args.no_overhead, history_fill=headline)
        return wl, inp, res

    wl, inp, head = run(args.workload, True)
    others = []
    if not args.only:
        for name in ("dsv3", "grouped", "long", "mtp"):
            if name != args.workload:
                others.append(run(name, False)[2]["summary"])
    sparse = prefill = None
    gqa = []
    if not args.only:
        sparse = measure_sparse(Q, W, torch, timer)
        prefill = measure_prefill(Q, W, torch, timer, cpu=not args.no_cpu)
        absorbed = {w["workload"]: w.get("us_per_step") for w in [head["summary"]] + others}
        for name in ("mtp", "dsv3", "grouped", "long"):
            gqa.append(measure_gqa(Q, W, torch, timer, name, absorbed.get(name),
                                   cpu=name == "mtp" and not args.no_cpu))
    sweep = None
    if not args.only and not args.no_sweep:
        log("batch-1 QK-norm overhead sweep")
        sweep = qknorm_sweep(Q, W, torch, timer)

    stream = None
    if not args.only:
        stream = hbm_read_stream(Q, torch, timer)
        # each HBM-bound figure also against the measured read rate
        for w in [head["summary"]] + others:
            if w.get("decode_kernel_us"):
                w["decode_frac_of_stream"] = round(
                    w["cache_bytes"] / (w["decode_kernel_us"] * 1e-6) / 1e9 / stream["gbs"], 4)

    hs = head["summary"]
    roof = roofline_of(head["flops"], head["nbytes"], head["dec_ms"] * 1e-3, load_traffic(wl.name))
    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(wl, inp)
    value = head["nbytes"] / (head["ms_per_step"] * 1e-3) / 1e9
    out = {
        "metric": "MLA decode-attn latent-cache GB/s (% HBM peak) and us/step, h=128 r=512",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "us_per_step": round(head["ms_per_step"] * 1e3, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_kernel_us": hs["decode_kernel_us"],
        "decode_combine_us": hs["decode_combine_us"],
        "decode_combine_project_us": hs["decode_combine_project_us"],
        "qknorm_overhead_pct": hs["qknorm_overhead_pct"],
        "history_fill": head["fill"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cache_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {k: v for k, v in hs.items()
                   if k in ("workload", "batch", "s_q", "heads", "kv_groups", "rank", "rope_dim",
                            "seq_len", "num_splits", "kernel", "cache_bytes", "flops")}
                  | {"cache": wl.cache_dtype},
        "roofline": roof,
        "workloads": [hs] + others,
        "sparse": sparse,
        "prefill": prefill,
        "gqa_path": gqa or None,
        "qknorm_sweep": sweep,
        "hbm_read_stream": stream,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
