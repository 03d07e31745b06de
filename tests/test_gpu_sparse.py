"""GPU parity of the selected-token decode (qkn_mla_decode_sparse) against the
CPU oracle's sparse decode, on the oracle's own stored cache and query images.

Every split partial and the merged row (qkn_mla_combine over the partials) is
held to the same bars as the dense decode: the row-relative 1e-2 of a bf16
cache and, element by element, the bound derived from the kernel's arithmetic
with the oracle's weights over the split's listed tokens (gpu_helpers).  Every
GPU step is announced (case name, seed, shape) before it runs.
"""
import numpy as np
import pytest
import torch

import oracle_pins as P
import qk_normed_mla_amd as Q
import workloads as W
from gpu_helpers import (TOL_E2E, announce, kernel_elementwise_bound, kernel_lse_bound,
                         logit_error_bound, require_gpu, row_err, upload_words)
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _setup(wl, inp):
    """A runner holding the oracle's stored cache and query images."""
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    r = DecodeRunner(wl, inp)
    r.kv.copy_(upload_words(img["kv"], r.kv))
    r.alpha_k.copy_(torch.from_numpy(img["alpha_k"]).to("cuda"))
    r.q_tilde.copy_(upload_words(qi["q_tilde"], r.q_tilde))
    r.alpha_q.copy_(torch.from_numpy(qi["alpha_q"]).to("cuda"))
    r.q_rope_normed.copy_(upload_words(qi["qr_hat"], r.q_rope_normed))
    return r, img, qi


def _run_sparse(wl, r, idx, num_splits, flags=0):
    r.alloc_partials(num_splits)
    r.err_flag.zero_()
    dev_idx = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda")
    Q.qkn_mla_decode_sparse(r.dims, r.q_tilde, r.alpha_q, r.q_rope_normed, r.kv, r.alpha_k,
                            r.block_table, r.seq_lens, dev_idx, num_splits, flags,
                            r.o_partial, r.lse_partial, r.err_flag)
    r.combine()
    torch.cuda.synchronize()


def _listed(wl, inp, img, b, i, entries):
    """Stored latents, RoPE keys and alpha^k of the valid list entries, in order."""
    T = int(inp["seq_lens"][b])
    vis = O.visible_count(T, wl.s_q, i)
    t = np.asarray(entries, dtype=np.int64)
    ok = (t >= 0) & (t < vis)
    t = t[ok]
    page = inp["block_table"][b, t // 64]
    good = (page >= 0) & (page < img["kv"].shape[0])
    page, sl = page[good], t[good] % 64
    C = O.words_to_f64(img["kv"][page, sl, :wl.rank], wl.cache_dtype)
    KR = O.words_to_f64(img["kv"][page, sl, wl.rank:], wl.cache_dtype)
    AK = img["alpha_k"][page, sl, :].astype(np.float64)
    return C, KR, AK


def _compare(wl, inp, img, qi, r, idx, ref, num_splits, use_alpha=True):
    o_part = r.o_partial.float().cpu().numpy()
    lse_part = r.lse_partial.cpu().numpy()
    o_lat = r.o_latent.cpu().numpy()
    lse = r.lse.cpu().numpy()
    K = idx.shape[2]
    bounds = O.sparse_split_bounds(K, num_splits)
    qt = O.words_to_f64(qi["q_tilde"], wl.cache_dtype)
    qr = O.words_to_f64(qi["qr_hat"], wl.cache_dtype)
    hs = np.arange(wl.heads)
    g_of = O.group_of(hs, wl.heads, wl.groups)
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            aq = qi["alpha_q"][b, i].astype(np.float64) if use_alpha else np.ones(wl.heads)
            # (token set, partial index or None for the merged row)
            sets = [(idx[b, i, lo:hi], p) for p, (lo, hi) in enumerate(bounds)]
            sets.append((idx[b, i], None))
            for entries, p in sets:
                C, KR, AK = _listed(wl, inp, img, b, i, entries)
                if not use_alpha:
                    AK = np.ones_like(AK)
                n = C.shape[0]
                for h in range(wl.heads):
                    v = ref[(b, i, h)]
                    want = v["o_lat"] if p is None else v["o_part"][p]
                    want_lse = v["lse"] if p is None else v["lse_part"][p]
                    got = o_lat[b, i, h] if p is None else o_part[b, i, h, p]
                    got_lse = lse[b, i, h] if p is None else lse_part[b, i, h, p]
                    if n == 0:
                        assert np.isneginf(want_lse) and np.isneginf(got_lse), (b, i, h, p)
                        assert not np.any(got), (b, i, h, p)
                        continue
                    g = g_of[h]
                    logits = O.absorbed_logits(wl, qt[b, i, h:h + 1], aq[h:h + 1],
                                               qr[b, i, h:h + 1], C, AK, KR, g)[0]
                    w = np.exp(logits - logits.max())
                    w /= w.sum()
                    D = logit_error_bound(wl.softmax_scale, qt[b, i, h:h + 1], aq[h:h + 1],
                                          qr[b, i, h:h + 1], C, AK[:, g], KR)[0] + 1e-5
                    nn = n if p is not None else n + num_splits
                    tol = kernel_elementwise_bound(1, wl.cache_dtype, w, C, want, D, nn,
                                                   p is not None)
                    err = np.abs(got - want)
                    assert np.all(err <= tol), (b, i, h, p, float(np.max(err - tol)))
                    rel = row_err(got, want)
                    worst = max(worst, rel)
                    assert rel <= TOL_E2E[wl.cache_dtype], (b, i, h, p, rel)
                    assert abs(got_lse - want_lse) <= kernel_lse_bound(1, D, nn), (b, i, h, p)
    return worst


CASES = [
    # (name, workload overrides, list length, list fill, splits)
    ("dsv3", dict(), 96, 0.7, 1),
    ("dsv3", dict(), 96, 0.7, 3),
    ("mtp", dict(), 64, 0.5, 2),                 # s_q = 4: each query token its own list
    ("grouped", dict(), 128, 0.6, 5),            # 4 KV groups; the fifth split is empty
    ("long", dict(seq_len=1000), 700, 0.9, 2),   # 352 entries per split
]


@pytest.mark.parametrize("name,kw,K,fill,splits", CASES)
def test_sparse_decode_matches_oracle(name, kw, K, fill, splits):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=41)
    idx = W.make_selection(wl, inp["seq_lens"], K, seed=42, fill=fill)
    announce(f"sparse {name} {kw} K={K} fill={fill} splits={splits}")
    r, img, qi = _setup(wl, inp)
    _run_sparse(wl, r, idx, splits)
    assert int(r.err_flag.item()) == 0
    ref, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                        inp["seq_lens"], idx, splits)
    assert not err
    worst = _compare(wl, inp, img, qi, r, idx, ref, splits)
    print(f"  worst row error {worst:.2e}", flush=True)


def test_sparse_decode_without_alpha():
    wl = P.small("dsv3")
    inp = W.make_inputs(wl, seed=43)
    idx = W.make_selection(wl, inp["seq_lens"], 64, seed=44, fill=0.8)
    announce("sparse dsv3 without alpha")
    r, img, qi = _setup(wl, inp)
    _run_sparse(wl, r, idx, 2, flags=Q.QKN_DECODE_NO_ALPHA)
    ones = np.ones_like(img["alpha_k"])
    qi1 = dict(qi, alpha_q=np.ones_like(qi["alpha_q"]))
    ref, _ = O.sparse_decode_on_image(wl, qi1, img["kv"], ones, inp["block_table"],
                                      inp["seq_lens"], idx, 2)
    _compare(wl, inp, img, qi, r, idx, ref, 2, use_alpha=False)


def test_sparse_invalid_entries_flagged_and_skipped():
    """Entries past a query's visible end, below -1 or on an out-of-range page
    are reported and contribute nothing; the rest is as without them."""
    wl = P.small("mtp")
    inp = W.make_inputs(wl, seed=45)
    idx = W.make_selection(wl, inp["seq_lens"], 64, seed=46, fill=0.5)
    bad = idx.copy()
    free = np.argwhere(bad[0, 0] == -1)[:3, 0]
    bad[0, 0, free[0]] = int(inp["seq_lens"][0])        # one past the last token
    bad[0, 0, free[1]] = -5
    bad[1, 3, np.argwhere(bad[1, 3] == -1)[0, 0]] = 10 ** 6
    announce("sparse invalid entries")
    r, img, qi = _setup(wl, inp)
    _run_sparse(wl, r, bad, 2)
    assert int(r.err_flag.item()) & Q.QKN_FLAG_INDEX
    ref, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                        inp["seq_lens"], bad, 2)
    assert err
    _compare(wl, inp, img, qi, r, idx, ref, 2)


def test_sparse_empty_lists_and_all_visible():
    """A list of -1 only (and a list of length 0) gives the empty sum (o = 0,
    lse = -inf); listing every visible token in order matches the dense decode
    of the same state to the kernel bars."""
    wl = P.small("dsv3")
    inp = W.make_inputs(wl, seed=47)
    announce("sparse empty lists")
    r, img, qi = _setup(wl, inp)
    for K in (40, 0):
        idx = np.full((wl.batch, wl.s_q, K), -1, dtype=np.int32)
        _run_sparse(wl, r, idx, 2)
        assert int(r.err_flag.item()) == 0
        assert torch.all(torch.isneginf(r.lse)) and not torch.any(r.o_latent)
    K = int(np.max(inp["seq_lens"])) + 7
    idx = W.make_selection(wl, inp["seq_lens"], K, seed=48, fill=1.0, shuffle=False)
    announce("sparse listing every visible token")
    _run_sparse(wl, r, idx, 3)
    ref, _ = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                      inp["seq_lens"], idx, 3)
    _compare(wl, inp, img, qi, r, idx, ref, 3)
    dense = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                              inp["seq_lens"], 2)
    got = r.o_latent.cpu().numpy()
    for (b, i, h), v in dense.items():
        assert row_err(got[b, i, h], v["o_lat"]) <= TOL_E2E["bf16"]


def test_sparse_full_list_length():
    """2048-entry lists over a 4096-token context with shuffled pages, in the
    launch shape the benchmark uses (512 entries per split)."""
    wl = W.WORKLOADS["sparse"].replace(batch=3, seq_len=4096)
    inp = W.make_inputs(wl, seed=49)
    idx = W.make_selection(wl, inp["seq_lens"], W.SPARSE_LIST_LEN, seed=50)
    announce(f"sparse full list B={wl.batch} T=4096 K={W.SPARSE_LIST_LEN} splits=4")
    r, img, qi = _setup(wl, inp)
    _run_sparse(wl, r, idx, 4)
    assert int(r.err_flag.item()) == 0
    ref, _ = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                      inp["seq_lens"], idx, 4)
    _compare(wl, inp, img, qi, r, idx, ref, 4)


def test_sparse_rejections():
    wl = P.small("dsv3")
    inp = W.make_inputs(wl, seed=51)
    r = DecodeRunner(wl, inp)
    r.alloc_partials(1)
    idx = torch.full((wl.batch, 1, 4096), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(Q.QknError):   # 4096 entries in one split: over the per-split limit
        Q.qkn_mla_decode_sparse(r.dims, r.q_tilde, r.alpha_q, r.q_rope_normed, r.kv, r.alpha_k,
                                r.block_table, r.seq_lens, idx, 1, 0, r.o_partial, r.lse_partial)
