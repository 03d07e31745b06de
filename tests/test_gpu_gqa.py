"""GPU parity of the GQA path of GQLA under QK-norm (qkn_mla_gqa_append,
qkn_mla_gqa_attend; the query side is qkn_mla_prefill_query) against the CPU
oracle.

The append is held to the oracle's cache image word by word (keys and values
to a bound derived from exact products with float32 sums and the half
rounding, RoPE keys within one bf16 step, untouched slots unchanged); the
attention, on the oracle's own images, to the decode's derived bound with half
probabilities and half split partials; the whole step from float32 inputs to
the explicit float64 path at the 1e-2 bar of a bf16 cache; and a full-size
ragged multi-token batch, in the benchmark's launch configuration, on sampled
rows.  Every GPU step is announced (case name, seed, shape) first.
"""
import numpy as np
import pytest
import torch

import bench  # the benchmark's split rule for the GQA path
import oracle_pins as P
import qk_normed_mla_amd as Q
import workloads as W
from gpu_helpers import (TOL_E2E, announce, gamma_k, kernel_elementwise_bound, kernel_lse_bound,
                         require_gpu, row_err, ulp_distance_bf16)
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner

pytestmark = pytest.mark.gpu

CASES = [
    # (name, overrides, split counts)
    ("dsv3", dict(batch=2, seq_len=200), (1, 3)),            # s_q = 1: one token x 128 heads per workgroup
    ("mtp", dict(batch=3, s_q=4), (1, 3)),                   # ragged lengths, shuffled pages
    ("grouped", dict(batch=2, seq_len=150, s_q=2), (1, 4)),  # G = 4: 32 heads per group
    ("long", dict(seq_len=1000), (7, 40)),                   # 32 key tiles; 40 splits: the wide combine, 24 empty
    ("mtp", dict(batch=2, s_q=2, seq_len_range=(40, 300)), (1, 2)),  # s_q = 2: 2 tokens x 64 heads per workgroup
    ("mtp", dict(batch=3, s_q=4, seq_len_range=(4, 6)), (1, 2)),     # sequences of 4 to 6 tokens: T = s_q included
]
APPEND_CASES = [(n, kw) for n, kw, _ in CASES] + [
    ("grouped", dict(batch=2, seq_len=90, rank=256, heads=64, groups=2)),  # r = 256, G = 2
    ("grouped", dict(batch=2, seq_len=400)),  # G = 4, a history of 798 tokens: the matrix-core route
    ("dsv3", dict(batch=3, seq_len=52)),   # a history of 153 tokens: two per block, a ragged last block
    ("dsv3", dict(batch=3, seq_len=110)),  # 327 tokens: four per block, a ragged last block
]
SENTINEL = 0x7E01


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _runner(wl, inp, splits=1):
    r = DecodeRunner(wl, inp)
    r.alloc_gqa(splits, fill_word=SENTINEL)
    return r


def _token_slots(wl, inp):
    seq = np.repeat(np.arange(wl.batch), inp["seq_lens"])
    pos = np.concatenate([np.arange(int(T)) for T in inp["seq_lens"]])
    return inp["block_table"][seq, pos // 64], pos % 64


@pytest.mark.parametrize("name,kw", APPEND_CASES)
def test_gqa_append_image(name, kw):
    """History in bulk (more than 512 tokens in one call take the matrix-core
    route, fewer blocks of 1, 2 or 4 tokens), then the s_q new tokens: every written
    key and value
    within 2^-11 |x| + 2^-25 (half rounding) of exact, plus the float32 sum's
    gamma_{3r+2} sum_m |c_m W_mj| (times gamma_k alpha for a key, plus the
    key's share of the inverse RMS's own error); RoPE keys within one bf16 step
    (or 2^-20 of the row's largest entry at a zero crossing); every other word
    unchanged."""
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=61)
    announce(f"gqa append {name} {kw}")
    r = _runner(wl, inp)
    r.err_flag.zero_()
    r.gqa_fill_history()
    r.gqa_append_new()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    got = r.words(r.kvg)
    img = O.gqa_full_image(wl, inp, O.gqa_empty_image(wl, int(inp["num_pages"]), SENTINEL))
    page, slot = _token_slots(wl, inp)
    written = np.zeros(got.shape[:2], dtype=bool)
    written[page, slot] = True
    assert np.array_equal(got[~written], img["kvg"][~written])
    d, G, r_ = wl.head_dim, wl.groups, wl.rank
    rows = got[page, slot]
    C = np.abs(O.stored_value(np.asarray(inp["c"], dtype=np.float64), "bf16").astype(np.float64))
    g_s = gamma_k(3 * r_ + 2) * 1.01
    for g in range(G):
        K = O.stored_value(np.asarray(inp["c"], np.float64), "bf16").astype(np.float64) \
            @ inp["w_k"][g].astype(np.float64)
        dK = g_s * (C @ np.abs(inp["w_k"][g].astype(np.float64)))
        dV = g_s * (C @ np.abs(inp["w_v"][g].astype(np.float64)))
        alpha = 1.0 / np.sqrt(np.mean(K * K, axis=1) + wl.eps)
        rel_a = np.sum(np.abs(K) * dK, axis=1) / np.sum(K * K, axis=1) + gamma_k(d + 8)
        k_ex, v_ex = img["k_hat"][:, g], img["v"][:, g]
        gk = np.abs(inp["gamma_k"][g]).astype(np.float64)
        k_got = O.words_to_f64(rows[:, 2 * d * g:2 * d * g + d], "f16")
        v_got = O.words_to_f64(rows[:, 2 * d * g + d:2 * d * (g + 1)], "f16")
        tol_k = (2.0 ** -11 * np.abs(k_ex) + 2.0 ** -25 + gk * alpha[:, None] * dK
                 + np.abs(k_ex) * rel_a[:, None]) * 1.01
        tol_v = (2.0 ** -11 * np.abs(v_ex) + 2.0 ** -25 + dV) * 1.01
        assert np.all(np.abs(k_got - k_ex) <= tol_k), (g, float(np.max(np.abs(k_got - k_ex) - tol_k)))
        assert np.all(np.abs(v_got - v_ex) <= tol_v), (g, float(np.max(np.abs(v_got - v_ex) - tol_v)))
    got_r, want_r = rows[:, 2 * d * G:], img["kvg"][page, slot, 2 * d * G:]
    u = ulp_distance_bf16(got_r, want_r)
    gf, wf = O.words_to_f64(got_r, "bf16"), O.words_to_f64(want_r, "bf16")
    near = np.abs(gf - wf) <= 2.0 ** -20 * np.max(np.abs(wf), axis=-1, keepdims=True)
    assert np.all((u <= 1) | near)


def test_gqa_append_skips_bad_tokens():
    """Tokens naming a sequence, position or page out of range are skipped and
    flagged; the good tokens of the same call are written."""
    wl = P.small("dsv3", batch=2, seq_len=200)
    inp = W.make_inputs(wl, seed=62)
    announce("gqa append with bad tokens")
    r = _runner(wl, inp)
    bt = inp["block_table"].copy()
    bt[1, 1] = -1                                     # sequence 1's second page unmapped
    r.block_table.copy_(torch.from_numpy(bt))
    n = 40
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32)
    seq[3], seq[5], pos[7] = 5, -1, 10 ** 6           # bad sequences, a bad position
    seq[9], pos[9] = 1, 70                            # on the unmapped page
    dev = r.device
    c = torch.from_numpy(np.ascontiguousarray(inp["c"][:n])).to(dev)
    kr = torch.from_numpy(np.ascontiguousarray(inp["k_rope"][:n])).to(dev)
    r.err_flag.zero_()
    r.gqa_append_tokens(c, kr, torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev))
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) & Q.QKN_FLAG_INDEX
    got = r.words(r.kvg)
    good = [k for k in range(n) if k not in (3, 5, 7, 9)]
    pg = bt[0, pos[good] // 64]
    assert not np.any(got[pg, pos[good] % 64] == SENTINEL)
    rest = np.ones(got.shape[:2], dtype=bool)
    rest[pg, pos[good] % 64] = False
    assert np.all(got[rest] == SENTINEL)


def _attend_bound_check(wl, inp, o, lse, q_img, kvg, splits):
    """o, lse against the oracle's GQA decode on the same images, element by
    element: the decode's derived bound with half probabilities (plus 2^-25
    each below half's normal range), float32 logits over d + d_R terms and,
    for several splits, the half step of the stored partials; and 1e-2."""
    res = O.gqa_decode_on_image(wl, q_img, kvg, inp["block_table"], inp["seq_lens"], splits)
    d, G = wl.head_dim, wl.groups
    qh = O.words_to_f64(q_img["q_hat"], "f16")
    qr = O.words_to_f64(q_img["qr_hat"], "bf16")
    worst = 0.0
    for b, T in enumerate(inp["seq_lens"]):
        t = np.arange(int(T))
        rows = kvg[inp["block_table"][b, t // 64], t % 64]
        KR = O.words_to_f64(rows[:, 2 * d * G:], "bf16")
        for i in range(wl.s_q):
            n = O.visible_count(int(T), wl.s_q, i)
            for h in range(wl.heads):
                g = int(O.group_of(h, wl.heads, G))
                K = O.words_to_f64(rows[:n, 2 * d * g:2 * d * g + d], "f16")
                V = O.words_to_f64(rows[:n, 2 * d * g + d:2 * d * (g + 1)], "f16")
                v = res[(b, i, h)]
                logits = wl.softmax_scale * (K @ qh[b, i, h] + KR[:n] @ qr[b, i, h])
                w = np.exp(logits - logits.max())
                w /= w.sum()
                mag = np.abs(K) @ np.abs(qh[b, i, h]) + np.abs(KR[:n]) @ np.abs(qr[b, i, h])
                D = wl.softmax_scale * gamma_k(d + wl.rope_dim) * float(np.max(mag)) * 1.01 + 1e-5
                sub = 2.0 * n * 2.0 ** -25 * float(np.max(np.abs(V)))
                tol = kernel_elementwise_bound(2, "bf16" if splits > 1 else "f32", w, V, v["o"], D, n,
                                               False) + sub
                err = np.abs(o[b, i, h] - v["o"])
                assert np.all(err <= tol), (b, i, h, float(np.max(err - tol)))
                rel = row_err(o[b, i, h], v["o"])
                worst = max(worst, rel)
                assert rel <= TOL_E2E["bf16"], (b, i, h, rel)
                assert abs(lse[b, i, h] - v["lse"]) <= kernel_lse_bound(2, D, n) + n * 2.0 ** -24, \
                    (b, i, h)
    return worst


@pytest.mark.parametrize("name,kw,splits", CASES)
def test_gqa_attend_on_oracle_images(name, kw, splits):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=63)
    img = O.gqa_full_image(wl, inp, O.gqa_empty_image(wl, int(inp["num_pages"]), 0))
    qi = O.prefill_query_image(wl, inp)
    r = _runner(wl, inp)
    r.kvg.copy_(torch.from_numpy(img["kvg"].view(np.int16)))
    r.q_hat.copy_(torch.from_numpy(qi["q_hat"].view(np.int16)).view(torch.float16))
    r.q_rope_normed.copy_(torch.from_numpy(qi["qr_hat"].view(np.int16)).view(torch.bfloat16))
    for P_ in splits:
        announce(f"gqa attend on the oracle's images {name} {kw} splits={P_}")
        r.set_gqa_splits(P_)
        r.err_flag.zero_()
        r.gqa_attend()
        torch.cuda.synchronize()
        assert int(r.err_flag.item()) == 0
        worst = _attend_bound_check(wl, inp, r.o_gqa.cpu().numpy(), r.lse_gqa.cpu().numpy(), qi,
                                    img["kvg"], P_)
        print(f"  splits {P_}: worst row error {worst:.2e}", flush=True)


@pytest.mark.parametrize("name,kw,splits", CASES)
def test_gqa_end_to_end(name, kw, splits):
    """History appended, then one GQA step (query side, append of the new
    tokens, attention) from float32 inputs against the explicit float64 path."""
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=64)
    for P_ in splits:
        announce(f"gqa end to end {name} {kw} splits={P_}")
        r = _runner(wl, inp, P_)
        r.err_flag.zero_()
        r.gqa_fill_history()
        r.gqa_step()
        torch.cuda.synchronize()
        assert int(r.err_flag.item()) == 0
        o, lse = r.o_gqa.cpu().numpy(), r.lse_gqa.cpu().numpy()
        worst = 0.0
        for b in range(wl.batch):
            for i in range(wl.s_q):
                ex = O.explicit_rows(wl, inp, b, i)
                for h in range(wl.heads):
                    rel = row_err(o[b, i, h], ex["o"][h])
                    worst = max(worst, rel)
                    assert rel <= TOL_E2E["bf16"], (b, i, h, rel)
                assert np.max(np.abs(lse[b, i] - ex["lse"])) <= TOL_E2E["bf16"]
        print(f"  splits {P_}: worst row error {worst:.2e}", flush=True)


def test_gqa_attend_flags_bad_sequences():
    """A sequence shorter than s_q, and one whose page entry is unmapped, are
    flagged; the other sequences' rows are unchanged."""
    wl = P.small("mtp", batch=3, s_q=4)
    inp = W.make_inputs(wl, seed=65)
    announce("gqa attend with a short sequence and an unmapped page")
    r = _runner(wl, inp, 3)
    r.gqa_fill_history()
    r.gqa_step()
    torch.cuda.synchronize()
    good = r.o_gqa[2].clone()
    r.seq_lens[0] = 2
    r.err_flag.zero_()
    r.gqa_attend()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) & Q.QKN_FLAG_INDEX
    assert torch.equal(r.o_gqa[2], good)
    r.seq_lens[0] = int(inp["seq_lens"][0])
    r.block_table[1, 0] = -1
    r.err_flag.zero_()
    r.gqa_attend()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) & Q.QKN_FLAG_INDEX
    assert torch.equal(r.o_gqa[2], good)


def test_gqa_full_size_mtp_sampled_rows():
    """The ragged multi-token workload (64 sequences of 1024-16384 tokens, 4
    query tokens, shuffled pages) at full size in the benchmark's launch
    configuration: sampled rows against the explicit path."""
    wl = W.WORKLOADS["mtp"]
    inp = W.make_inputs(wl, seed=0)
    splits = bench.gqa_splits(wl, inp["seq_lens"])
    announce(f"gqa full-size mtp B={wl.batch} s_q={wl.s_q} H={wl.heads} splits={splits} seed=0")
    r = DecodeRunner(wl, inp)
    r.alloc_gqa(splits)
    r.gqa_fill_history()
    r.gqa_step()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    o, lse = r.o_gqa.cpu().numpy(), r.lse_gqa.cpu().numpy()
    del r
    torch.cuda.empty_cache()
    heads = np.array([0, 31, 32, 63, 64, 95, 96, 127])
    worst, worst_lse = 0.0, 0.0
    for b in sorted({0, wl.batch // 2, wl.batch - 1, int(np.argmax(inp["seq_lens"]))}):
        for i in (0, wl.s_q - 1):
            e = O.explicit_rows(wl, inp, b, i, heads=heads)
            for k, h in enumerate(heads):
                worst = max(worst, row_err(o[b, i, h], e["o"][k]))
                worst_lse = max(worst_lse, abs(float(lse[b, i, h]) - float(e["lse"][k])))
    print(f"  row err {worst:.2e}, lse err {worst_lse:.2e}", flush=True)
    assert worst <= TOL_E2E["bf16"] and worst_lse <= TOL_E2E["bf16"]
