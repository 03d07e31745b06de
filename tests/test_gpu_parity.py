"""GPU parity: every library call against the CPU oracle, element by element.

Sizes keep the float64 oracle to seconds while spanning several 64-token tiles
and a ragged tail.  Every GPU step is announced (case name, seed, shape) on
stdout before it runs.
"""
import numpy as np
import pytest
import torch

import oracle_pins as P
import qk_normed_mla_amd as Q
import workloads as W
from gpu_helpers import (TOL_E2E, TOL_KERNEL_GENERIC, U_PART, U_PROB, announce,
                         kernel_elementwise_bound, kernel_lse_bound, logit_error_bound,
                         require_gpu, row_err, ulp_distance_bf16, upload_words, run_e2e)
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner

pytestmark = pytest.mark.gpu
NAMES = ["tiny", "dsv3", "grouped", "long", "mtp"]
SENTINEL_BF16 = 0x7FC1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _oracle_decode_all(wl, inp, qi, img, num_splits, use_alpha=True):
    return O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                             inp["seq_lens"], num_splits, use_alpha=use_alpha)


# ---------------------------------------------------------------------------
# append: the cache image
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", NAMES)
def test_append_cache_image(name):
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=21, extra_pages=2)
    announce(f"append {name} B={wl.batch} T={list(inp['seq_lens'])[:4]} pages={inp['num_pages']}")
    _check_append_image(wl, inp)


# per-step appends at other shapes: head dims 32, 64 and 256, ranks 128 to
# 384, up to 80 tokens in one call and KV groups
APPEND_SHAPES = [("dsv3", dict(head_dim=32, rank=128)), ("dsv3", dict(head_dim=64, rank=256)),
                 ("grouped", dict(rank=384)), ("mtp", dict(batch=20)),
                 ("grouped", dict(batch=40, seq_len=100)),
                 ("dsv3", dict(head_dim=256, rank=256))]


@pytest.mark.parametrize("name,kw", APPEND_SHAPES)
def test_append_cache_image_shapes(name, kw):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=26, extra_pages=2)
    announce(f"append {name} {kw} tokens={wl.batch * wl.s_q}")
    _check_append_image(wl, inp)


# thousands of tokens in one call: alpha^k as one matrix product per group
BULK = [("dsv3", dict(batch=8, seq_len=600)), ("grouped", dict(batch=4, seq_len=1100)),
        ("mtp", dict(batch=12, seq_len=500, seq_len_range=(300, 500))),
        # every head dim the matrix-core route takes (its chunk rows and steps
        # per chunk differ with d): 32, 64 and 256, at ranks 256 and 384
        ("dsv3", dict(batch=8, seq_len=600, head_dim=32, rank=256)),
        ("grouped", dict(batch=4, seq_len=1100, head_dim=64, rank=384)),
        ("dsv3", dict(batch=8, seq_len=600, head_dim=256, rank=256)),
        ("grouped", dict(batch=4, seq_len=1100, head_dim=256, rank=384))]


@pytest.mark.parametrize("name,kw", BULK)
def test_append_cache_image_bulk(name, kw):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=25, extra_pages=2)
    n_hist = int(np.sum(inp["seq_lens"])) - wl.batch * wl.s_q
    assert n_hist >= 4096  # the bulk path's threshold
    announce(f"append bulk {name} {n_hist} tokens G={wl.groups} d={wl.head_dim} r={wl.rank}")
    _check_append_image(wl, inp)


def _check_append_image(wl, inp):
    fill = SENTINEL_BF16 if wl.cache_dtype == "bf16" else float("nan")
    r = DecodeRunner(wl, inp, kv_fill_word=fill)
    r.fill_history()
    r.append_new()
    torch.cuda.synchronize()
    _verify_append_image(wl, inp, r)


def _verify_append_image(wl, inp, r):
    """The runner's cache image against the oracle's (every token appended)."""
    assert int(r.err_flag.item()) == 0
    got = r.kv_words()
    ak = r.alpha_k.cpu().numpy()
    kv0, ak0 = O.empty_images(wl, inp["num_pages"])
    img = O.full_cache_image(wl, inp, kv0, ak0)
    rk = wl.rank
    written = np.zeros(got.shape[:2], bool)
    bt = inp["block_table"]
    for b, T in enumerate(inp["seq_lens"]):
        t = np.arange(int(T))
        written[bt[b, t // 64], t % 64] = True
    # latent and slot indexing: bit-exact; untouched slots keep the sentinel
    if wl.cache_dtype == "bf16":
        assert np.array_equal(got[..., :rk], img["kv"][..., :rk])
        assert np.all(got[~written] == SENTINEL_BF16)
        # RoPE key: the float32 rotation x1 cos - x2 sin is off by ~2^-24 of its
        # terms, which near a zero crossing is several bf16 steps of a tiny result;
        # so within 1 step, or within 2^-20 of the row's largest entry
        gw, iw = got[written][:, rk:], img["kv"][written][:, rk:]
        d = ulp_distance_bf16(gw, iw)
        gf, rf = O.words_to_f64(gw, "bf16"), O.words_to_f64(iw, "bf16")
        near = np.abs(gf - rf) <= 2.0 ** -20 * np.max(np.abs(rf), axis=1, keepdims=True)
        assert np.all((d <= 1) | near), f"RoPE key off by {d[~near].max()} bf16 steps"
    else:
        assert np.array_equal(got[..., :rk][written], img["kv"][..., :rk][written])
        assert np.all(np.isnan(got[~written]))
        assert np.allclose(got[written][:, rk:], img["kv"][written][:, rk:], rtol=1e-5, atol=1e-6)
    assert np.all(np.isnan(ak[~written]))
    rel = np.abs(ak[written] / img["alpha_k"][written] - 1.0)
    assert rel.max() < 1e-5, rel.max()


@pytest.mark.parametrize("n_bad_seq", [1, 5000])  # 5000: the bulk path
def test_append_rejects_bad_slots(n_bad_seq):
    """Out-of-range sequence, position or page entries are skipped and flagged."""
    wl = P.small("dsv3", batch=2, seq_len=130)
    inp = W.make_inputs(wl, seed=22)
    inp["block_table"] = inp["block_table"].copy()
    inp["block_table"][1, 1] = -1            # page entry out of range
    announce(f"append bad slots dsv3 ({n_bad_seq} tokens of a bad sequence)")
    r = DecodeRunner(wl, inp, kv_fill_word=SENTINEL_BF16)
    before = r.kv_words().copy()
    ak_before = r.alpha_k.cpu().numpy().copy()
    # tokens: one valid, one in the bad page, one past max pages, bad sequences
    seq = torch.tensor([0, 1, 0] + [5] * n_bad_seq, dtype=torch.int32, device="cuda")
    pos = torch.tensor([3, 70, 64 * wl.max_pages_per_seq + 1] + [0] * n_bad_seq,
                       dtype=torch.int32, device="cuda")
    n = 3 + n_bad_seq
    c = torch.randn(n, wl.rank, device="cuda")
    kr = torch.randn(n, wl.rope_dim, device="cuda")
    r.err_flag.zero_()
    Q.qkn_mla_append(r.dims, c, kr, seq, pos, r.block_table, r.w_k, r.gamma_kr, r.kv, r.alpha_k,
                     r.err_flag)
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 1
    after = r.kv_words()
    changed = np.any(after != before, axis=-1)
    pg = inp["block_table"][0, 0]
    assert changed[pg, 3] and changed.sum() == 1
    ak = r.alpha_k.cpu().numpy()
    ak_changed = ~((ak == ak_before) | (np.isnan(ak) & np.isnan(ak_before)))
    assert ak_changed[pg, 3].all() and ak_changed.sum() == wl.groups


# ---------------------------------------------------------------------------
# absorb_query
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", NAMES)
def test_absorb_query(name):
    _check_absorb(P.small(name), f"absorb {name}")


# bf16 shapes with fewer column blocks per row tile (rank <= 384: each block
# forms alpha^q and the RoPE query of more than one batch of rows) and a head
# dim spanning two staging steps
ABSORB_SHAPES = [("dsv3", dict(rank=128)), ("dsv3", dict(rank=256, heads=64)),
                 ("grouped", dict(rank=384)), ("dsv3", dict(head_dim=256, rank=64)),
                 # from 16384 query rows (x 4 column blocks) the wave-tile kernel:
                 # whole tiles, a ragged last tile with tiles spanning two query
                 # tokens (100 heads), and four groups
                 ("mtp", dict(batch=32)), ("mtp", dict(batch=41, heads=100)),
                 ("grouped", dict(batch=130)),
                 # every RoPE width it takes (1 to 4 pairs per lane), and no rotation
                 ("mtp", dict(batch=32, rope_dim=32)), ("mtp", dict(batch=32, rope_dim=96)),
                 ("mtp", dict(batch=32, rope_dim=128)), ("mtp", dict(batch=32, rope_theta=0.0)),
                 # two column blocks (16 RoPE rows each, in two chunks) and G = 8 (16 heads
                 # per group: two query tokens per tile)
                 ("grouped", dict(batch=260, groups=8, rank=256))]


@pytest.mark.parametrize("name,kw", ABSORB_SHAPES)
def test_absorb_query_shapes(name, kw):
    _check_absorb(P.small(name, **kw), f"absorb {name} {kw}")


def _check_absorb(wl, case):
    inp = W.make_inputs(wl, seed=23)
    announce(case)
    r = DecodeRunner(wl, inp)
    r.absorb()
    torch.cuda.synchronize()
    _verify_absorb(wl, inp, r)


def _verify_absorb(wl, inp, r):
    """The runner's query side against the oracle's."""
    ref = O.query_image(wl, inp)
    aq = r.alpha_q.cpu().numpy()
    assert np.max(np.abs(aq / ref["alpha_q"] - 1)) < 1e-5
    qt, qr = r.words(r.q_tilde), r.words(r.q_rope_normed)
    if wl.cache_dtype == "bf16":
        # q~ is a dot product of length d that can cancel, so a per-element ulp
        # bound is wrong near zero: hold each row to half a bf16 step of its
        # largest entry (the storage rounding, 2^-8 relative) against the exact
        # float64 value, and require almost every word to be bit-equal.
        exact = O.absorb_query(wl, inp["q"], inp["q_rope"], inp["w_k"], inp["gamma_q"],
                               inp["gamma_k"], inp["gamma_qr"], r.q_pos.cpu().numpy())
        got = O.bf16_bits_to_f32(qt).astype(np.float64)
        assert row_err(got, exact["q_tilde"]) <= 2.0 ** -8 * 1.01
        assert np.mean(qt == ref["q_tilde"]) > 0.99
        # The RoPE query word is x1 cos - x2 sin (and x2 cos + x1 sin) formed in
        # float32 and rounded to bf16.  Its terms are as large as the row, so
        # the float32 evaluation (the norm, the products, the sine and cosine
        # of the angle rounded to float) is good to ~2^-21 of the row's
        # largest entry, and a word near zero may be several bf16 steps off
        # while still that close.  So each word is within one bf16 step of the
        # oracle's word, or within 2^-20 of its row's largest entry of the
        # exact float64 value.
        d = ulp_distance_bf16(qr, ref["qr_hat"])
        got_r = O.bf16_bits_to_f32(qr).astype(np.float64)
        ex_r = exact["qr_hat"]
        near = np.abs(got_r - ex_r) <= 2.0 ** -20 * np.max(np.abs(ex_r), axis=-1, keepdims=True)
        assert np.all((d <= 1) | near), (int(d.max()), int(np.sum(d > 1)))
        assert np.mean(d == 0) > 0.99
    else:
        assert row_err(qt, ref["q_tilde"]) < 1e-5
        assert row_err(qr, ref["qr_hat"]) < 1e-5


# ---------------------------------------------------------------------------
# decode + combine on the oracle's own stored state
# ---------------------------------------------------------------------------

def _decode_on_image(wl, inp, num_splits, flags=0):
    """Run decode + combine on the oracle's stored state; returns the runner,
    the oracle's result and, per (b, i), what the error bounds need."""
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    r = DecodeRunner(wl, inp, num_splits=num_splits)
    r.kv.copy_(upload_words(img["kv"], r.kv))
    r.alpha_k.copy_(torch.from_numpy(img["alpha_k"]).to("cuda"))
    r.q_tilde.copy_(upload_words(qi["q_tilde"], r.q_tilde))
    r.alpha_q.copy_(torch.from_numpy(qi["alpha_q"]).to("cuda"))
    r.q_rope_normed.copy_(upload_words(qi["qr_hat"], r.q_rope_normed))
    r.decode(flags)
    r.combine()
    torch.cuda.synchronize()
    use_alpha = not (flags & Q.QKN_DECODE_NO_ALPHA)
    ref = _oracle_decode_all(wl, inp, qi, img, num_splits, use_alpha=use_alpha)
    return r, ref, _row_context(wl, inp, img, qi, use_alpha=use_alpha)


def _row_context(wl, inp, img, qi, use_alpha=True):
    """Per (b, i): the stored latents the query sees C [n, r], the oracle's
    float64 logits over them [H, n] (to form its weights), per head the bound D
    on the float32 error of the kernel's logits over the same tokens (plus 1e-5
    for the exponent's own rounding), and the sequence length."""
    out = {}
    for b, T in enumerate(inp["seq_lens"]):
        t = np.arange(int(T))
        pg, sl = inp["block_table"][b, t // 64], t % 64
        C = O.words_to_f64(img["kv"][pg, sl, :wl.rank], wl.cache_dtype)
        KR = O.words_to_f64(img["kv"][pg, sl, wl.rank:], wl.cache_dtype)
        AK = img["alpha_k"][pg, sl, :].astype(np.float64)
        if not use_alpha:
            AK = np.ones_like(AK)
        for i in range(wl.s_q):
            n = int(T) - wl.s_q + i + 1
            hs = np.arange(wl.heads)
            g = O.group_of(hs, wl.heads, wl.groups)
            qt = O.words_to_f64(qi["q_tilde"][b, i], wl.cache_dtype)
            qr = O.words_to_f64(qi["qr_hat"][b, i], wl.cache_dtype)
            aq = qi["alpha_q"][b, i].astype(np.float64) if use_alpha else np.ones(wl.heads)
            D = np.zeros(wl.heads)
            logits = np.zeros((wl.heads, n))
            for gg in range(wl.groups):
                sel = g == gg
                D[sel] = logit_error_bound(wl.softmax_scale, qt[sel], aq[sel], qr[sel],
                                           C[:n], AK[:n, gg], KR[:n]) + 1e-5
                logits[sel] = O.absorbed_logits(wl, qt[sel], aq[sel], qr[sel], C[:n], AK[:n],
                                                KR[:n], gg)
            out[(b, i)] = (C[:n], logits, D, int(T))
    return out


def _compare_decode(wl, r, ref, kind, ctx):
    """Partials and the merged result against the oracle: every row within the
    row-relative bar of its cache dtype (1e-2 bf16, 1e-4 float32; 1e-5 for the
    vector-ALU kernel on a float32 cache), and every element within the bound
    derived from the kernel's arithmetic with the oracle's own weights (see
    gpu_helpers).  Returns (worst row-relative error, worst ratio of the
    elementwise bound to the row's largest entry)."""
    o_part = r.o_partial.float().cpu().numpy()
    lse_part = r.lse_partial.cpu().numpy()
    o_lat = r.o_latent.cpu().numpy()
    lse = r.lse.cpu().numpy()
    bar = TOL_E2E[wl.cache_dtype] if kind == 1 or wl.cache_dtype == "bf16" else TOL_KERNEL_GENERIC
    num_splits = o_part.shape[3]
    worst_rel, worst_bound = 0.0, 0.0
    for (b, i, h), v in ref.items():
        C, logits, D, T = ctx[(b, i)]
        n = C.shape[0]
        empty = np.isneginf(v["lse_part"])
        assert np.all(np.isneginf(lse_part[b, i, h][empty]))
        assert not np.any(o_part[b, i, h][empty])
        # (got, exact, got lse, exact lse, token range, is a stored partial)
        cases = [(o_lat[b, i, h], v["o_lat"], lse[b, i, h], v["lse"], (0, n), False)]
        bounds = O.split_bounds(T, num_splits)
        for p in np.nonzero(~empty)[0]:
            lo, hi = bounds[p]
            cases.append((o_part[b, i, h, p], v["o_part"][p], lse_part[b, i, h, p],
                          v["lse_part"][p], (lo, min(hi, n)), True))
        for got, want, lg, lw, (lo, hi), partial in cases:
            w = np.exp(logits[h, lo:hi] - lw)
            err = np.abs(got - want)
            scale = max(np.max(np.abs(want)), 1e-30)
            rel = float(np.max(err) / scale)
            worst_rel = max(worst_rel, rel)
            nn = (hi - lo) + (0 if partial else num_splits)
            tol_m = kernel_elementwise_bound(kind, wl.cache_dtype, w, C[lo:hi], want, D[h], nn,
                                             partial)
            worst_bound = max(worst_bound, float(np.max(tol_m) / scale))
            assert np.all(err <= tol_m), (b, i, h, lo, hi, float(np.max(err - tol_m)))
            assert rel <= bar, (b, i, h, lo, hi, rel)
            assert abs(lg - lw) <= kernel_lse_bound(kind, D[h], nn), (b, i, h, lg, lw, D[h])
    return worst_rel, worst_bound


@pytest.mark.parametrize("name", NAMES)
def test_decode_on_oracle_state(name):
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=24)
    kind = Q.decode_kernel_kind(Q.dims_for(wl, inp["num_pages"]), wl.num_splits)
    announce(f"decode {name} kind={kind} splits={wl.num_splits}")
    r, ref, ctx = _decode_on_image(wl, inp, wl.num_splits)
    rel, bnd = _compare_decode(wl, r, ref, kind, ctx)
    print(f"  row err {rel:.2e}, elementwise bound up to {bnd:.2e} of the row max", flush=True)


def test_reference_restart_on_rising_logits():
    """The matrix-core kernel fixes each head's exponent reference at the first
    visible tokens of a split and restarts the split when a later logit
    outgrows it by more than its headroom.  Here the stored latents of the
    second half of every sequence are scaled up 80-fold (alpha^k kept), which
    lifts those content logits far past the first tokens' maximum; the result
    must still equal the oracle's softmax over the same stored state."""
    wl = P.small("dsv3", seq_len=256)
    inp = W.make_inputs(wl, seed=31)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    rk = wl.rank
    for b, T in enumerate(inp["seq_lens"]):
        t = np.arange(int(T) // 2, int(T))
        pg, sl = inp["block_table"][b, t // 64], t % 64
        c = O.words_to_f64(img["kv"][pg, sl, :rk], wl.cache_dtype)
        img["kv"][pg, sl, :rk] = O.stored_bits(80.0 * c, wl.cache_dtype)
    ref = _oracle_decode_all(wl, inp, qi, img, 1)
    # precondition: some head's logits rise past the first tile's maximum by
    # more than the kernel's headroom (2^96, i.e. 96 ln 2 in natural units)
    rose = False
    for b, T in enumerate(inp["seq_lens"]):
        t = np.arange(int(T))
        pg, sl = inp["block_table"][b, t // 64], t % 64
        C = O.words_to_f64(img["kv"][pg, sl, :rk], wl.cache_dtype)
        KR = O.words_to_f64(img["kv"][pg, sl, rk:], wl.cache_dtype)
        lg = O.absorbed_logits(wl, O.words_to_f64(qi["q_tilde"][b, 0], wl.cache_dtype),
                               qi["alpha_q"][b, 0].astype(np.float64),
                               O.words_to_f64(qi["qr_hat"][b, 0], wl.cache_dtype), C,
                               img["alpha_k"][pg, sl, :].astype(np.float64), KR, 0)
        rose |= bool(np.any(lg.max(axis=1) - lg[:, :32].max(axis=1) > 96 * np.log(2.0)))
    assert rose
    r = DecodeRunner(wl, inp, num_splits=1)
    kind = Q.decode_kernel_kind(r.dims, 1)
    announce(f"decode restart dsv3 B={wl.batch} T={list(inp['seq_lens'])} kind={kind}")
    assert kind == 1
    r.kv.copy_(upload_words(img["kv"], r.kv))
    r.alpha_k.copy_(torch.from_numpy(img["alpha_k"]).to("cuda"))
    r.q_tilde.copy_(upload_words(qi["q_tilde"], r.q_tilde))
    r.alpha_q.copy_(torch.from_numpy(qi["alpha_q"]).to("cuda"))
    r.q_rope_normed.copy_(upload_words(qi["qr_hat"], r.q_rope_normed))
    r.err_flag.zero_()
    r.decode(0)
    r.combine()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == Q.QKN_FLAG_RESTART
    rel, bnd = _compare_decode(wl, r, ref, 1, _row_context(wl, inp, img, qi))
    print(f"  row err {rel:.2e}, elementwise bound up to {bnd:.2e} of the row max", flush=True)


@pytest.mark.parametrize("name", ["dsv3", "grouped", "mtp"])
def test_decode_generic_kernel(name):
    """The vector-ALU kernel on the bf16 shapes (an independent GPU path)."""
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=25)
    announce(f"decode generic {name}")
    r, ref, ctx = _decode_on_image(wl, inp, 3, flags=Q.QKN_DECODE_FORCE_GENERIC)
    rel, bnd = _compare_decode(wl, r, ref, 0, ctx)
    print(f"  row err {rel:.2e}, elementwise bound up to {bnd:.2e} of the row max", flush=True)


@pytest.mark.parametrize("name", ["tiny", "dsv3", "grouped"])
def test_decode_without_alpha(name):
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=26)
    kind = Q.decode_kernel_kind(Q.dims_for(wl, inp["num_pages"]), 2)
    announce(f"decode no-alpha {name} kind={kind}")
    r, ref, ctx = _decode_on_image(wl, inp, 2, flags=Q.QKN_DECODE_NO_ALPHA)
    rel, bnd = _compare_decode(wl, r, ref, kind, ctx)
    print(f"  row err {rel:.2e}, elementwise bound up to {bnd:.2e} of the row max", flush=True)


# ---------------------------------------------------------------------------
# end to end: float32 inputs through all four calls vs the explicit float64 path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", NAMES)
def test_end_to_end(name):
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=27)
    announce(f"e2e {name} splits={wl.num_splits}")
    r = run_e2e(wl, inp)
    assert int(r.err_flag.item()) == 0
    o_lat = r.o_latent.cpu().numpy()
    lse = r.lse.cpu().numpy()
    tol = TOL_E2E[wl.cache_dtype]
    worst, worst_o = 0.0, 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            e = O.explicit_rows(wl, inp, b, i)
            worst = max(worst, row_err(o_lat[b, i], e["o_lat"]))
            assert np.max(np.abs(lse[b, i] - e["lse"])) < tol
            # the caller's value up-projection of the GPU latent output
            o = O.value_up_projection(wl, o_lat[b, i], inp["w_v"], np.arange(wl.heads))
            worst_o = max(worst_o, row_err(o, e["o"]))
    print(f"  e2e row err {worst:.2e}, o {worst_o:.2e}", flush=True)
    assert worst <= tol and worst_o <= tol


@pytest.mark.parametrize("name,splits,flags", [
    ("tiny", 2, 0), ("dsv3", 3, 0), ("grouped", 5, 0), ("mtp", 4, 0), ("long", 7, 0),
    ("dsv3", 3, Q.QKN_DECODE_NO_ALPHA), ("grouped", 2, Q.QKN_DECODE_FORCE_GENERIC)])
def test_decode_attend_matches_decode_then_combine(name, splits, flags):
    """qkn_mla_decode_attend (partials in a library-sized workspace) leaves the
    same bits as qkn_mla_decode into caller partials followed by
    qkn_mla_combine; a second call on a dirty workspace too."""
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=38)
    announce(f"decode_attend {name} splits={splits} flags={flags}")
    r = DecodeRunner(wl, inp, num_splits=splits)
    r.fill_history()
    r.prepare()
    r.decode(flags)
    r.combine()
    torch.cuda.synchronize()
    o_ref, lse_ref = r.o_latent.clone(), r.lse.clone()
    for _ in range(2):
        r.o_latent.fill_(float("nan"))
        r.lse.fill_(float("nan"))
        r.attend(flags)
        torch.cuda.synchronize()
        assert torch.equal(r.o_latent.view(torch.int32), o_ref.view(torch.int32))
        assert torch.equal(r.lse.view(torch.int32), lse_ref.view(torch.int32))
    assert r.workspace.numel() == Q.decode_workspace_bytes(r.dims, splits)


# ---------------------------------------------------------------------------
# invariants and edge cases
# ---------------------------------------------------------------------------

def test_split_invariance_and_empty_splits():
    wl = P.small("long", seq_len=700)   # 11 pages
    inp = W.make_inputs(wl, seed=28)
    outs = {}
    for splits in (1, 3, 11, 40):       # 40 leaves empty partitions
        announce(f"split invariance P={splits}")
        r = run_e2e(wl, inp, num_splits=splits)
        outs[splits] = (r.o_latent.cpu().numpy(), r.lse.cpu().numpy())
        if splits == 40:
            lp = r.lse_partial.cpu().numpy()
            assert np.all(np.isneginf(lp[..., 11:]))
    # every split count lands within the end-to-end bar of the explicit path,
    # so two of them within twice that of each other
    e = O.explicit_rows(wl, inp, 0, 0)
    for splits in (1, 3, 11, 40):
        assert row_err(outs[splits][0][0, 0], e["o_lat"]) <= TOL_E2E["bf16"]
        assert np.max(np.abs(outs[splits][1][0, 0] - e["lse"])) <= TOL_E2E["bf16"]
    for splits in (3, 11, 40):
        assert row_err(outs[splits][0][0, 0], outs[1][0][0, 0]) <= 2 * TOL_E2E["bf16"]


def test_page_permutation_bitwise():
    wl = P.small("mtp", batch=3)
    inp = W.make_inputs(wl, seed=29)
    inp2 = W.permute_pages(inp, seed=30)
    announce("page permutation")
    a = run_e2e(wl, inp)
    b = run_e2e(wl, inp2)
    assert torch.equal(a.o_latent, b.o_latent) and torch.equal(a.lse, b.lse)


def test_work_dealing_ragged_batch_with_ties():
    """A ragged batch of up to 64 sequences is dealt to the workgroups longest
    sequence first, ties by index.  Every (sequence, split, row block) item
    must be computed exactly once, and its result must not depend on which
    workgroup draws it: 64 sequences of five distinct lengths (many ties, an
    empty split at the shortest) are decoded, then decoded again in reverse
    order, which breaks the ties the other way and hands the items to other
    workgroups.  Put back in order, the partials match bit for bit, and no
    sentinel survives in either run."""
    wl = W.WORKLOADS["mtp"].replace(batch=64, seq_len=200, seq_len_range=None, num_splits=3)
    inp = W.make_inputs(wl, seed=41)
    lens = np.array([4, 64, 65, 130, 200], dtype=np.int32)[np.arange(64) * 7 % 5]
    announce("work dealing: 64 ragged sequences with ties, forward and reversed")
    r = DecodeRunner(wl, inp, num_splits=3)
    r.fill_history()
    r.prepare()
    r.seq_lens.copy_(torch.from_numpy(lens).to("cuda"))

    def run():
        r.o_partial.fill_(float("nan"))
        r.lse_partial.fill_(float("nan"))
        r.err_flag.zero_()
        r.decode()
        torch.cuda.synchronize()
        assert int(r.err_flag.item()) == 0
        o, l = r.o_partial.clone(), r.lse_partial.clone()
        assert not torch.isnan(o).any() and not torch.isnan(l).any()
        return o, l

    a_o, a_l = run()
    perm = torch.arange(63, -1, -1, device="cuda")
    for t in (r.block_table, r.seq_lens, r.q_tilde, r.alpha_q, r.q_rope_normed):
        t.copy_(t[perm].clone())
    b_o, b_l = run()
    assert torch.equal(a_o, b_o[perm]) and torch.equal(a_l, b_l[perm])
    # the shortest sequences leave their later splits empty
    assert torch.all(torch.isneginf(a_l[torch.from_numpy(lens == 4).to("cuda")][..., 1:]))


def test_deterministic():
    wl = P.small("grouped")
    inp = W.make_inputs(wl, seed=31)
    announce("determinism")
    r = run_e2e(wl, inp)
    first = r.o_latent.clone()
    for _ in range(3):
        r.step()
    torch.cuda.synchronize()
    assert torch.equal(first, r.o_latent)


@pytest.mark.parametrize("name", ["dsv3", "mtp"])
def test_rows_sum_to_one(name):
    """Latent dimension 0 set to 1.0 (exact in bf16): o_latent[..., 0] = sum_t p_t = 1."""
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=32)
    inp["c"][:, 0] = 1.0
    announce(f"rows sum to one {name}")
    r = run_e2e(wl, inp)
    o0 = r.o_latent[..., 0].cpu().numpy()
    assert np.max(np.abs(o0 - 1.0)) < 1e-5, np.max(np.abs(o0 - 1.0))


def test_single_token_and_minimal_lengths():
    """T_b = s_q (each query sees a prefix of the new tokens) and T_b = 1."""
    wl = W.WORKLOADS["mtp"].replace(batch=3, seq_len=64, seq_len_range=(4, 6))
    inp = W.make_inputs(wl, seed=33)
    inp["seq_lens"] = inp["seq_lens"].copy()
    announce(f"minimal lengths {list(inp['seq_lens'])}")
    r = run_e2e(wl, inp)
    o_lat = r.o_latent.cpu().numpy()
    for b in range(wl.batch):
        for i in range(wl.s_q):
            e = O.explicit_rows(wl, inp, b, i)
            assert row_err(o_lat[b, i], e["o_lat"]) < TOL_E2E["bf16"]
    wl1 = P.small("dsv3", batch=1, seq_len=1)
    inp1 = W.make_inputs(wl1, seed=34)
    announce("T = 1")
    r1 = run_e2e(wl1, inp1)
    c0 = O.stored_value(inp1["c"][0], "bf16")
    assert np.array_equal(r1.o_latent[0, 0].cpu().numpy(), np.broadcast_to(c0, (wl1.heads, wl1.rank)))


def test_zero_vectors_stay_finite():
    """c_t = 0 gives alpha^k = 1/sqrt(eps) and a zero content logit; q = 0 likewise."""
    wl = P.small("dsv3", batch=1, seq_len=100)
    inp = W.make_inputs(wl, seed=35)
    inp["c"][10:20] = 0.0
    inp["q"][0, 0, :5] = 0.0
    announce("zero vectors")
    r = run_e2e(wl, inp)
    o_lat = r.o_latent.cpu().numpy()
    assert np.all(np.isfinite(o_lat))
    e = O.explicit_rows(wl, inp, 0, 0)
    assert row_err(o_lat[0, 0], e["o_lat"]) < TOL_E2E["bf16"]
    ak = r.alpha_k.cpu().numpy()
    pg = inp["block_table"][0, 0]
    assert np.allclose(ak[pg, 10:20, 0], 1.0 / np.sqrt(np.float32(wl.eps)), rtol=1e-6)


def test_decode_flags_bad_lengths():
    """A sequence length past the block table is clamped and flagged; a page
    entry out of range skips its tokens and is flagged."""
    wl = P.small("dsv3", batch=2, seq_len=128)
    inp = W.make_inputs(wl, seed=36)
    announce("decode bad lengths")
    r = run_e2e(wl, inp)
    r.err_flag.zero_()
    r.seq_lens[1] = 64 * wl.max_pages_per_seq + 5
    r.decode()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == Q.QKN_FLAG_INDEX
    assert np.all(np.isfinite(r.o_partial.float().cpu().numpy()[1][r.lse_partial.cpu().numpy()[1] > -np.inf]))
    r.seq_lens.copy_(torch.from_numpy(inp["seq_lens"]).cuda())
    r.err_flag.zero_()
    r.block_table[0, 1] = inp["num_pages"] + 7
    r.decode()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == Q.QKN_FLAG_INDEX


@pytest.mark.parametrize("flags", [0, Q.QKN_DECODE_FORCE_GENERIC])
def test_half_partials_out_of_range_flagged(flags):
    """Latents beyond the half range make the half partials +-inf and raise
    QKN_FLAG_PARTIAL_RANGE; in-range latents of the same step raise nothing."""
    wl = P.small("dsv3", batch=2, seq_len=128)
    inp = W.make_inputs(wl, seed=37)
    announce(f"half partial range flags={flags}")
    r = run_e2e(wl, inp)
    r.err_flag.zero_()
    r.decode(flags)
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    big = dict(inp)
    big["c"] = inp["c"] * np.float32(1e6)   # |c| far beyond 65504, still a bf16 number
    r2 = run_e2e(wl, big)
    r2.err_flag.zero_()
    r2.decode(flags)
    torch.cuda.synchronize()
    assert int(r2.err_flag.item()) == Q.QKN_FLAG_PARTIAL_RANGE
    assert np.any(np.isinf(r2.o_partial.float().cpu().numpy()))
