"""qkn_mla_decode_attend_noalloc (partials in the library's static device
scratch) against qkn_mla_decode_attend (partials in a caller workspace): the
same bits, on two calls in a row, the second with a smaller input, so that
the second call runs over what the first left in the scratch."""
import numpy as np
import pytest
import torch

import oracle_pins as P
import qk_normed_mla_amd as Q
import workloads as W
from gpu_helpers import TOL_E2E, announce, require_gpu, row_err
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(r, flags=0):
    """(o_latent, lse) of the workspace call and of the allocation-free call."""
    r.attend(flags)
    torch.cuda.synchronize()
    ref = (r.o_latent.clone(), r.lse.clone())
    r.o_latent.fill_(float("nan"))
    r.lse.fill_(float("nan"))
    Q.qkn_mla_decode_attend_noalloc(r.dims, r.q_tilde, r.alpha_q, r.q_rope_normed, r.kv,
                                    r.alpha_k, r.block_table, r.seq_lens, r.num_splits, flags,
                                    r.o_latent, r.lse, r.err_flag)
    torch.cuda.synchronize()
    return ref, (r.o_latent.clone(), r.lse.clone())


@pytest.mark.parametrize("first,second", [
    # (workload, size overrides, splits): the second call is smaller
    (("mtp", dict(batch=6, seq_len=400, seq_len_range=(100, 400)), 5),
     ("mtp", dict(batch=2, seq_len=120, seq_len_range=(20, 120)), 2)),
    (("grouped", dict(batch=3, seq_len=700), 9), ("dsv3", dict(batch=1, seq_len=90), 3)),
    (("tiny", dict(), 4), ("tiny", dict(seq_len=40), 1)),
])
def test_noalloc_matches_workspace_call(first, second):
    for name, kw, splits in (first, second):
        wl = P.small(name, **kw)
        inp = W.make_inputs(wl, seed=40)
        announce(f"decode_attend_noalloc {name} B={wl.batch} T={list(inp['seq_lens'])[:4]} "
                 f"splits={splits}")
        r = DecodeRunner(wl, inp, num_splits=splits)
        assert Q.decode_workspace_bytes(r.dims, splits) <= Q.NOALLOC_SCRATCH_BYTES
        r.fill_history()
        r.prepare()
        r.err_flag.zero_()
        (o_ref, lse_ref), (o, lse) = _both(r)
        assert int(r.err_flag.item()) == 0
        assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
        # and the result itself holds the end-to-end bar against the explicit path
        o_np, lse_np = o.cpu().numpy(), lse.cpu().numpy()
        tol = TOL_E2E[wl.cache_dtype]
        for b in range(wl.batch):
            for i in range(wl.s_q):
                e = O.explicit_rows(wl, inp, b, i)
                assert row_err(o_np[b, i], e["o_lat"]) <= tol
                assert np.max(np.abs(lse_np[b, i] - e["lse"])) <= tol
        del r
        torch.cuda.empty_cache()


def test_noalloc_rejects_beyond_scratch_on_the_device():
    """A request past the scratch size is refused with QKN_ERR_SCRATCH and
    leaves the outputs untouched."""
    wl = W.WORKLOADS["dsv3"].replace(batch=32, seq_len=128)
    inp = W.make_inputs(wl, seed=41)
    r = DecodeRunner(wl, inp, num_splits=16)
    assert Q.decode_workspace_bytes(r.dims, 16) > Q.NOALLOC_SCRATCH_BYTES
    r.o_latent.fill_(7.0)
    with pytest.raises(Q.QknError) as ei:
        Q.qkn_mla_decode_attend_noalloc(r.dims, r.q_tilde, r.alpha_q, r.q_rope_normed, r.kv,
                                        r.alpha_k, r.block_table, r.seq_lens, 16, 0,
                                        r.o_latent, r.lse, r.err_flag)
    assert ei.value.status == Q.QKN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(r.o_latent == 7.0))
