"""The read-only HBM stream (qkn_mla_stream_read) reads every word once: the
XOR it leaves in the sink equals the XOR of all 32-bit words of the buffer,
for sizes below one wave of loads, with a ragged last round, and over many
rounds of the grid."""
import ctypes

import numpy as np
import pytest
import torch

import qk_normed_mla_amd as Q
from gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 1000, 64 << 20])
def test_stream_read_xor(nbytes):
    require_gpu()
    announce(f"stream read {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((1,), 0x1234567, dtype=torch.int32, device="cuda")
    st = Q.library().qkn_mla_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                         ctypes.c_void_p(sink.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(words)) ^ 0x1234567
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == want
