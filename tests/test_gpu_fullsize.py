"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (its default split count), on sampled outputs.

The whole step runs on the GPU (query absorption, append of the new tokens,
split-KV decode, combine) over the full synthetic cache; the oracle then
computes a sample of the output rows one by one from the float32 inputs by the
explicit path (materialised keys, post-projection RMSNorm), including the
value up-projection of qkn_mla_combine_project.  The sample covers
the first, middle and last sequence, the first and last query token, and heads
at both edges of every 32-head wave and every KV group.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import TOL_E2E, announce, require_gpu, row_err
from oracle import qkn_oracle as O
from qk_normed_mla_amd.runner import DecodeRunner
import bench  # the benchmark's split rule

pytestmark = pytest.mark.gpu
FULL = ["dsv3", "grouped", "long", "mtp"]
EDGE_HEADS = [0, 31, 32, 63, 64, 95, 96, 127]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)
    splits = bench.default_splits(wl, inp["seq_lens"])
    wl = wl.replace(num_splits=splits)
    announce(f"full-size {name} B={wl.batch} s_q={wl.s_q} H={wl.heads} G={wl.groups} "
             f"T~{int(np.mean(inp['seq_lens']))} splits={splits} seed=0")
    r = DecodeRunner(wl, inp, num_splits=splits)
    r.fill_history()
    r.step()
    torch.cuda.synchronize()
    assert int(r.err_flag.item()) == 0
    o_lat = r.o_latent.cpu().numpy()
    lse = r.lse.cpu().numpy()
    # the same merge with the value up-projection (fused or two-pass by size)
    r.combine_project()
    torch.cuda.synchronize()
    assert np.array_equal(r.o_latent.cpu().numpy().view(np.int32), o_lat.view(np.int32))
    o = r.o.cpu().numpy()
    del r
    torch.cuda.empty_cache()

    tol = TOL_E2E[wl.cache_dtype]
    heads = np.array([h for h in EDGE_HEADS if h < wl.heads])
    worst, worst_lse, worst_o, n = 0.0, 0.0, 0.0, 0
    for b in sorted({0, wl.batch // 2, wl.batch - 1}):
        for i in sorted({0, wl.s_q - 1}):
            e = O.explicit_rows(wl, inp, b, i, heads=heads)
            for k, h in enumerate(heads):
                worst = max(worst, row_err(o_lat[b, i, h], e["o_lat"][k]))
                worst_lse = max(worst_lse, abs(float(lse[b, i, h]) - float(e["lse"][k])))
                worst_o = max(worst_o, row_err(o[b, i, h], e["o"][k]))
                n += 1
    print(f"  {n} rows: latent row err {worst:.2e}, lse err {worst_lse:.2e}, "
          f"o row err {worst_o:.2e}", flush=True)
    assert worst <= tol
    assert worst_o <= tol
    assert worst_lse <= tol
