"""GPU parity of the chunked prefill on the explicit path (qkn_mla_prefill_query,
qkn_mla_prefill_expand, qkn_mla_prefill_attend) against the CPU oracle.

Each call is held on the oracle's own images (query, expanded keys and values,
cache) to a bound derived from its arithmetic, and the three calls end to end
(float32 inputs -> GPU) to the 1e-2 bar of a bf16 cache against the explicit
float64 path.  Every GPU step is announced (case name, seed, shape) first.
"""
import numpy as np
import pytest
import torch

import oracle_pins as P
import qk_normed_mla_amd as Q
import workloads as W
from gpu_helpers import (TOL_E2E, announce, gamma_k, kernel_elementwise_bound, kernel_lse_bound,
                         require_gpu, row_err, ulp_distance_bf16, upload_words)
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner

pytestmark = pytest.mark.gpu

CASES = [
    # (name, overrides): the chunk is s_q new tokens per sequence
    ("dsv3", dict(batch=2, seq_len=200, s_q=8)),
    ("mtp", dict(batch=3, s_q=4)),                        # ragged lengths, shuffled pages
    ("grouped", dict(batch=2, seq_len=150, s_q=5)),       # G = 4; the last token group half idle
    ("long", dict(seq_len=1000, s_q=33)),                 # 32 key tiles
    ("dsv3", dict(batch=2, seq_len=70, s_q=70)),          # the chunk is the whole sequence: T = s_q
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _runner(wl, inp):
    r = DecodeRunner(wl, inp)
    r.fill_history()
    r.append_new()
    r.alloc_prefill()
    return r


@pytest.mark.parametrize("name,kw", CASES)
def test_prefill_query(name, kw):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=52)
    announce(f"prefill query {name} {kw}")
    r = _runner(wl, inp)
    r.prefill_query()
    torch.cuda.synchronize()
    ref = O.prefill_query_image(wl, inp)
    # q^ = gamma q / RMS(q) rounded once from float32: within one half step
    assert r.q_hat.dtype == torch.float16
    assert ulp_distance_bf16(r.words(r.q_hat), ref["q_hat"]).max() <= 1
    # the rotation x1 cos - x2 sin can cancel: within one step, or within 2^-20
    # of the row's largest entry
    got_r, want_r = r.words(r.q_rope_normed), ref["qr_hat"]
    d = ulp_distance_bf16(got_r, want_r)
    gf, wf = O.words_to_f64(got_r, "bf16"), O.words_to_f64(want_r, "bf16")
    near = np.abs(gf - wf) <= 2.0 ** -20 * np.max(np.abs(wf), axis=-1, keepdims=True)
    assert np.all((d <= 1) | near)


@pytest.mark.parametrize("name,kw", CASES)
def test_prefill_expand(name, kw):
    """Keys and values against the oracle's exact values: the float32 sums
    (every product exact) are within gamma_{r+2} sum_m |c_m W_mj| (times
    |gamma_k alpha^k| for a key) of exact, and the half rounding within 2^-11
    relative (2^-25 absolute below the normal range); rows past each sequence
    are zero."""
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=53)
    announce(f"prefill expand {name} {kw}")
    r = _runner(wl, inp)
    r.err_flag.zero_()
    r.prefill_expand()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    img = O.full_cache_image(wl, inp)
    max_T = r.k_hat.shape[1]
    e = O.expand_image(wl, img["kv"], img["alpha_k"], inp["block_table"], inp["seq_lens"],
                       inp["w_k"], inp["w_v"], inp["gamma_k"], max_T)
    pd = O.prefill_dtype(wl)
    got_k = O.words_to_f64(r.words(r.k_hat), pd)
    got_v = O.words_to_f64(r.words(r.v_exp), pd)
    g_r = gamma_k(wl.rank + 2)
    for b, T in enumerate(inp["seq_lens"]):
        T = int(T)
        t = np.arange(T)
        page, sl = inp["block_table"][b, t // 64], t % 64
        C = np.abs(O.words_to_f64(img["kv"][page, sl, :wl.rank], "bf16"))
        AK = img["alpha_k"][page, sl, :].astype(np.float64)
        for g in range(wl.groups):
            sk = (C @ np.abs(inp["w_k"][g].astype(np.float64))) * np.abs(inp["gamma_k"][g])[None, :] \
                * AK[:, g:g + 1]
            sv = C @ np.abs(inp["w_v"][g].astype(np.float64))
            for got, want, s in ((got_k, e["k_hat"], sk), (got_v, e["v"], sv)):
                err = np.abs(got[b, :T, g] - want[b, :T, g])
                tol = 2.0 ** -11 * np.abs(want[b, :T, g]) + 2.0 ** -25 + g_r * s * 1.01
                assert np.all(err <= tol), (b, g, float(np.max(err - tol)))
        assert not np.any(got_k[b, T:]) and not np.any(got_v[b, T:])


def _attend_bound_check(wl, inp, r, img, qi, e):
    """o and lse of the attend call against the oracle on the same images,
    element by element to the bound of the decode kernel's arithmetic with
    half probabilities into the P.V product (2^-11 relative, plus 2^-25
    absolute each below half's normal range), float32 logits over d + d_R
    terms, the values as the rows and no split partials; and row-relative
    1e-2."""
    res = O.prefill_on_images(wl, qi, e, img["kv"], inp["block_table"], inp["seq_lens"])
    o = r.o_prefill.cpu().numpy()
    lse = r.lse_prefill.cpu().numpy()
    pd = O.prefill_dtype(wl)
    qh = O.words_to_f64(qi["q_hat"], pd)
    qr = O.words_to_f64(qi["qr_hat"], "bf16")
    kh = O.words_to_f64(e["k_hat_words"], pd)
    vv = O.words_to_f64(e["v_words"], pd)
    worst = 0.0
    for b, T in enumerate(inp["seq_lens"]):
        for i in range(wl.s_q):
            n = O.visible_count(int(T), wl.s_q, i)
            t = np.arange(n)
            KR = O.words_to_f64(img["kv"][inp["block_table"][b, t // 64], t % 64, wl.rank:], "bf16")
            for h in range(wl.heads):
                g = int(O.group_of(h, wl.heads, wl.groups))
                v = res[(b, i, h)]
                logits = wl.softmax_scale * (kh[b, :n, g] @ qh[b, i, h] + KR @ qr[b, i, h])
                w = np.exp(logits - logits.max())
                w /= w.sum()
                mag = np.abs(kh[b, :n, g]) @ np.abs(qh[b, i, h]) + np.abs(KR) @ np.abs(qr[b, i, h])
                D = wl.softmax_scale * gamma_k(wl.head_dim + wl.rope_dim) * float(np.max(mag)) \
                    * 1.01 + 1e-5
                # every subnormal probability's absolute error (<= 2^-25, the
                # sum of the kernel's weights >= 1) moves o by at most twice it
                sub = 2.0 * n * 2.0 ** -25 * float(np.max(np.abs(vv[b, :n, g])))
                tol = kernel_elementwise_bound(2, "f32", w, vv[b, :n, g], v["o"], D, n, False) \
                    + sub
                err = np.abs(o[b, i, h] - v["o"])
                assert np.all(err <= tol), (b, i, h, float(np.max(err - tol)))
                rel = row_err(o[b, i, h], v["o"])
                worst = max(worst, rel)
                assert rel <= TOL_E2E["bf16"], (b, i, h, rel)
                assert abs(lse[b, i, h] - v["lse"]) <= kernel_lse_bound(2, D, n) \
                    + n * 2.0 ** -24, (b, i, h)
    return worst


@pytest.mark.parametrize("name,kw", CASES)
def test_prefill_attend_on_oracle_images(name, kw):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=54)
    announce(f"prefill attend on the oracle's images {name} {kw}")
    r = _runner(wl, inp)
    img = O.full_cache_image(wl, inp)
    qi = O.prefill_query_image(wl, inp)
    max_T = r.k_hat.shape[1]
    e = O.expand_image(wl, img["kv"], img["alpha_k"], inp["block_table"], inp["seq_lens"],
                       inp["w_k"], inp["w_v"], inp["gamma_k"], max_T)
    r.kv.copy_(upload_words(img["kv"], r.kv))
    r.q_hat.copy_(upload_words(qi["q_hat"], r.q_hat))
    r.q_rope_normed.copy_(upload_words(qi["qr_hat"], r.q_rope_normed))
    r.k_hat.copy_(upload_words(e["k_hat_words"], r.k_hat))
    r.v_exp.copy_(upload_words(e["v_words"], r.v_exp))
    r.err_flag.zero_()
    r.prefill_attend()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    worst = _attend_bound_check(wl, inp, r, img, qi, e)
    print(f"  worst row error {worst:.2e}", flush=True)


@pytest.mark.parametrize("name,kw", CASES)
def test_prefill_end_to_end(name, kw):
    """The three calls from float32 inputs against the explicit float64 path."""
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=55)
    announce(f"prefill end to end {name} {kw}")
    r = _runner(wl, inp)
    r.err_flag.zero_()
    r.prefill_query()
    r.prefill_expand()
    r.prefill_attend()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    o = r.o_prefill.cpu().numpy()
    lse = r.lse_prefill.cpu().numpy()
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            ex = O.explicit_rows(wl, inp, b, i)
            for h in range(wl.heads):
                rel = row_err(o[b, i, h], ex["o"][h])
                worst = max(worst, rel)
                assert rel <= TOL_E2E["bf16"], (b, i, h, rel)
            assert np.max(np.abs(lse[b, i] - ex["lse"])) <= TOL_E2E["bf16"]
    print(f"  worst row error {worst:.2e}", flush=True)


def test_prefill_flags_short_sequences():
    """A sequence shorter than the chunk is flagged; the others are unaffected."""
    wl = P.small("dsv3", batch=2, seq_len=200, s_q=8)
    inp = W.make_inputs(wl, seed=56)
    announce("prefill short sequence flagged")
    r = _runner(wl, inp)
    r.prefill_query()
    r.prefill_expand()
    r.prefill_attend()
    torch.cuda.synchronize()
    good = r.o_prefill[1].clone()
    r.seq_lens[0] = 3
    r.err_flag.zero_()
    r.prefill_attend()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) & Q.QKN_FLAG_INDEX
    assert torch.equal(r.o_prefill[1], good)
