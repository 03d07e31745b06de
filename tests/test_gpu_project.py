"""GPU parity of qkn_mla_combine_project: the split-KV merge followed by the
value up-projection o = o^lat W^V_g.

* o_latent and lse are the bits qkn_mla_combine writes, in every form (fused,
  two-pass, automatic).
* o against the oracle's value up-projection of the kernel's own o_latent, per
  element, within the error bound of the arithmetic:
    - matrix cores: both operands split into bf16 hi + lo words; each product
      is within 3 * 2^-16 of exact and the float32 sum of the 3 r products
      adds gamma_{3r}: |do_j| <= (3 * 2^-16 + gamma_{3r}) sum_m |L_m W_mj|.
    - vector ALUs (float32, r terms): |do_j| <= gamma_r sum_m |L_m W_mj|.
* Every form gives the same o bits on a second run (fixed summation order).
* End to end (absorb, append, decode, combine_project) against the explicit
  path of the oracle (materialised keys and values).
"""
import numpy as np
import pytest
import torch

import oracle_pins as P
import qk_normed_mla_amd as Q
import workloads as W
from gpu_helpers import TOL_E2E, announce, gamma_k, require_gpu, row_err, upload_words
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner

pytestmark = pytest.mark.gpu
NAMES = ["tiny", "dsv3", "grouped", "long", "mtp"]
FORMS = {"auto": 0, "fused": Q.QKN_PROJECT_FUSED, "two_pass": Q.QKN_PROJECT_TWO_PASS}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def matrix_core_applies(wl) -> bool:
    """The shapes the matrix-core projection takes (the rest is float32 vector code)."""
    return (wl.rank % 128 == 0 and wl.rank <= 512 and wl.head_dim in (32, 64, 128, 256)
            and wl.rank % min(256, 16384 // wl.head_dim) == 0
            and (wl.heads // wl.groups) % 32 == 0)


def project_bound(wl, o_lat, w_v):
    """Per-element bound on |o_gpu - o_exact| for the kernel's own o_lat rows."""
    L = np.abs(np.asarray(o_lat, dtype=np.float64)).reshape(-1, wl.heads, wl.rank)
    g = O.group_of(np.arange(wl.heads), wl.heads, wl.groups)
    Wabs = np.abs(np.asarray(w_v, dtype=np.float64))
    mag = np.stack([L[:, h] @ Wabs[g[h]] for h in range(wl.heads)], axis=1)
    coef = 3 * 2.0 ** -16 + gamma_k(3 * wl.rank) if matrix_core_applies(wl) else gamma_k(wl.rank)
    return coef * mag + 1e-30


def reference_o(wl, o_lat, w_v):
    L = np.asarray(o_lat, dtype=np.float64).reshape(-1, wl.heads, wl.rank)
    return np.stack([O.value_up_projection(wl, L[n], w_v, np.arange(wl.heads))
                     for n in range(L.shape[0])])


def _runner_on_image(wl, inp):
    """Decode on the oracle's stored state (cache and query side uploaded)."""
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    r = DecodeRunner(wl, inp, num_splits=wl.num_splits)
    r.kv.copy_(upload_words(img["kv"], r.kv))
    r.alpha_k.copy_(torch.from_numpy(img["alpha_k"]).to("cuda"))
    r.q_tilde.copy_(upload_words(qi["q_tilde"], r.q_tilde))
    r.alpha_q.copy_(torch.from_numpy(qi["alpha_q"]).to("cuda"))
    r.q_rope_normed.copy_(upload_words(qi["qr_hat"], r.q_rope_normed))
    r.decode()
    return r


def _check_forms(wl, inp):
    r = _runner_on_image(wl, inp)
    r.combine()
    torch.cuda.synchronize()
    lat_ref = r.o_latent.clone()
    lse_ref = r.lse.clone()
    w_v = inp["w_v"]
    for form, flags in FORMS.items():
        r.o_latent.fill_(float("nan"))
        r.lse.fill_(float("nan"))
        r.o.fill_(float("nan"))
        r.combine_project(flags)
        torch.cuda.synchronize()
        assert torch.equal(r.o_latent.view(torch.int32), lat_ref.view(torch.int32)), form
        assert torch.equal(r.lse.view(torch.int32), lse_ref.view(torch.int32)), form
        o = r.o.cpu().numpy().reshape(-1, wl.heads, wl.head_dim)
        assert np.all(np.isfinite(o)), form
        o_lat = r.o_latent.cpu().numpy()
        err = np.abs(o - reference_o(wl, o_lat, w_v))
        bound = project_bound(wl, o_lat, w_v)
        worst = float(np.max(err / bound))
        print(f"  {form}: max err / bound {worst:.3f}", flush=True)
        assert worst <= 1.0, form
        first = r.o.clone()
        r.o.fill_(float("nan"))
        r.combine_project(flags)
        torch.cuda.synchronize()
        assert torch.equal(r.o.view(torch.int32), first.view(torch.int32)), form


@pytest.mark.parametrize("name", NAMES)
def test_combine_project_forms(name):
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=31)
    announce(f"combine_project {name} splits={wl.num_splits} "
             f"matrix_core={matrix_core_applies(wl)}")
    _check_forms(wl, inp)


@pytest.mark.parametrize("name,kw", [
    ("dsv3", dict(batch=1, seq_len=64, num_splits=16)),    # splits past the last page: empty
    ("dsv3", dict(batch=3, seq_len=130, num_splits=1)),    # one split
    ("grouped", dict(batch=1, seq_len=100, num_splits=20)),  # more splits than the fused form takes
    ("dsv3", dict(batch=1, seq_len=100, head_dim=64)),     # d_v = 64: 4 reduction slices
    ("dsv3", dict(batch=1, seq_len=100, head_dim=96)),     # d_v = 96: vector path
    ("dsv3", dict(batch=2, seq_len=100, num_splits=3)),    # 128-row fused tiles, 3 splits
    ("dsv3", dict(batch=1, seq_len=64, num_splits=4)),     # 128-row fused tiles, empty splits
    ("mtp", dict(batch=2, seq_len=90, rank=256, num_splits=2)),  # 128-row fused tiles, r = 256
])
def test_combine_project_shapes(name, kw):
    wl = P.small(name, **kw)
    inp = W.make_inputs(wl, seed=32)
    announce(f"combine_project {name} {kw} matrix_core={matrix_core_applies(wl)}")
    _check_forms(wl, inp)


@pytest.mark.parametrize("name", NAMES)
def test_combine_project_end_to_end(name):
    wl = P.small(name)
    inp = W.make_inputs(wl, seed=33)
    announce(f"combine_project e2e {name}")
    r = DecodeRunner(wl, inp, num_splits=wl.num_splits)
    r.fill_history()
    r.prepare()
    r.decode()
    r.combine_project()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    o = r.o.cpu().numpy()
    tol = TOL_E2E[wl.cache_dtype]
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            e = O.explicit_rows(wl, inp, b, i)
            worst = max(worst, row_err(o[b, i], e["o"]))
    print(f"  e2e o row err {worst:.2e}", flush=True)
    assert worst <= tol
