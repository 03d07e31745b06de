"""Host-side checks of libqknmla.so that need no GPU.

The library must load, export every entry point include/qkn_mla.h declares,
and reject bad arguments on the host -- before any HIP call -- with the
documented status codes.  No call here can reach a kernel launch: every one
fails validation first (fake pointers are only ever paired with a failing check).
"""
import ctypes
import os
import re

import pytest

import qk_normed_mla_amd as Q

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "qkn_mla.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QKN_API\s+[\w\s\*]+?\b(qkn_\w+)\s*\(", text)))


def good_dims(**kw):
    base = dict(batch=2, s_q=1, heads=128, groups=1, rank=512, head_dim=128, rope_dim=64,
                max_pages_per_seq=4, num_pages=8, eps=1e-6, softmax_scale=192 ** -0.5,
                rope_theta=10000.0, cache_dtype="bf16")
    base.update(kw)
    return Q.make_dims(**base)


def test_library_exports_header_symbols():
    lib = Q.library()
    syms = declared_symbols()
    assert len(syms) == 21, syms
    assert set(syms) == set(Q.EXPORTED_SYMBOLS)
    for s in syms:
        assert hasattr(lib, s), f"{s} not exported"


def test_only_the_c_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {Q.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(Q.EXPORTED_SYMBOLS), exported ^ set(Q.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    lib = Q.library()
    assert lib.qkn_mla_abi_version() == Q.ABI_VERSION == 9
    for st in (0, -1, -2, -3, -4, -5):
        assert len(Q.status_string(st)) >= 2
    assert Q.status_string(123) == "unknown status"


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, -1), ("s_q", 0, -1), ("heads", 0, -1), ("groups", 3, -1),
    ("rank", 4, -1), ("rank", 100, -2), ("rank", 2048, -2), ("head_dim", 6, -2),
    ("rope_dim", 12, -2), ("rope_dim", -8, -1), ("max_pages_per_seq", 0, -1),
    ("num_pages", 0, -1), ("eps", -1.0, -1), ("eps", float("nan"), -1),
    ("softmax_scale", 0.0, -1), ("rope_theta", -1.0, -1), ("cache_dtype", 7, -1),
    ("page_size", 32, -2),
])
def test_dims_validation(field, value, status):
    d = good_dims()
    setattr(d, field, value)
    assert Q.library().qkn_mla_check_dims(ctypes.byref(d)) == status


def test_good_dims_and_kernel_kind():
    lib = Q.library()
    d = good_dims()
    assert lib.qkn_mla_check_dims(ctypes.byref(d)) == 0
    assert Q.decode_kernel_kind(d, 8, 0) in (0, 1)
    assert Q.decode_kernel_kind(d, 8, Q.QKN_DECODE_FORCE_GENERIC) == 0
    assert Q.decode_kernel_kind(good_dims(cache_dtype="f32", heads=8, rank=64, head_dim=32,
                                          rope_dim=16), 1, 0) == 0
    assert Q.decode_kernel_kind(d, 0, 0) == -1
    assert Q.decode_kernel_kind(d, 5000, 0) == -1


def _call_decode(d, ptr, num_splits=1, flags=0):
    P = ctypes.c_void_p
    return Q.library().qkn_mla_decode(ctypes.byref(d), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr),
                                      P(ptr), P(ptr), num_splits, flags, P(ptr), P(ptr), None,
                                      None)


def test_null_pointers_rejected_before_launch():
    lib = Q.library()
    d = good_dims()
    P = ctypes.c_void_p
    assert _call_decode(d, None) == -1
    assert lib.qkn_mla_combine(ctypes.byref(d), 2, None, None, None, None, None) == -1
    assert lib.qkn_mla_append(ctypes.byref(d), 4, None, None, None, None, None, None, None,
                              None, None, None, None) == -1
    assert lib.qkn_mla_absorb_query(ctypes.byref(d), *([None] * 11)) == -1
    # n_tokens == 0 is a no-op that needs no pointers; negative is an error
    assert lib.qkn_mla_append(ctypes.byref(d), 0, *([None] * 11)) == 0
    assert lib.qkn_mla_append(ctypes.byref(d), -1, *([None] * 11)) == -1
    # a null dims pointer
    assert lib.qkn_mla_check_dims(None) == -1
    del P


def test_misaligned_pointers_rejected_before_launch():
    d = good_dims()
    assert _call_decode(d, 0x1008) == -3
    assert Q.library().qkn_mla_combine(ctypes.byref(d), 2, *([ctypes.c_void_p(0x1004)] * 4),
                                       None) == -3


def test_bad_flags_and_splits_rejected():
    d = good_dims()
    assert _call_decode(d, 0x1000, num_splits=0) == -1
    assert _call_decode(d, 0x1000, flags=8) == -1
    bad = good_dims(heads=0)
    assert _call_decode(bad, 0x1000) == -1


def test_binding_refuses_host_tensors():
    import torch
    d = good_dims(batch=1, heads=8, rank=64, head_dim=32, rope_dim=16, num_pages=1,
                  max_pages_per_seq=1, cache_dtype="f32")
    with pytest.raises(ValueError):
        Q.qkn_mla_combine(d, 1, torch.zeros(8 * 64), torch.zeros(8), torch.zeros(8 * 64),
                          torch.zeros(8))


def test_combine_project_rejects_bad_arguments():
    """Host-side checks of qkn_mla_combine_project run before anything touches
    a device: bad flags, split counts and missing or misaligned pointers."""
    lib = Q.library()
    d = good_dims()
    ok = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below is rejected first
    bad = ctypes.c_void_p((1 << 20) + 4)

    def call(num_splits=8, flags=0, w_v=ok, o=ok, o_lat=ok):
        return lib.qkn_mla_combine_project(ctypes.byref(d), num_splits, ok, ok, w_v, o_lat, ok, o,
                                           ctypes.c_uint32(flags), None)
    assert call(flags=4) == -1
    assert call(num_splits=0) == -1
    assert call(num_splits=5000) == -1
    assert call(w_v=None) == -1
    assert call(o=None) == -1
    assert call(o_lat=None) == -1
    assert call(o=bad) == -3
    d.groups = 3
    assert call() == -1


def test_partial_dtype_query():
    """The partial dtype comes from the library: half for a bf16 cache, float32
    for a float32 cache, an error status for invalid dims."""
    import torch
    lib = Q.library()
    assert lib.qkn_mla_partial_dtype(ctypes.byref(good_dims())) == Q.QKN_F16
    assert lib.qkn_mla_partial_dtype(ctypes.byref(good_dims(cache_dtype="f32"))) == Q.QKN_F32
    assert lib.qkn_mla_partial_dtype(ctypes.byref(good_dims(heads=0))) == -1
    assert lib.qkn_mla_partial_dtype(None) == -1
    assert Q.partial_torch_dtype(good_dims()) == torch.float16
    assert Q.partial_torch_dtype(good_dims(cache_dtype="f32")) == torch.float32


@pytest.mark.parametrize("kw,splits", [
    (dict(), 8), (dict(cache_dtype="f32"), 3), (dict(batch=64, s_q=4), 4),
    (dict(batch=1, heads=8, rank=64, head_dim=32, rope_dim=16), 1), (dict(batch=3), 37),
])
def test_workspace_bytes(kw, splits):
    """Both partial arrays fit, each starting on a 256-byte boundary: o_partial
    [rows, P, r] in the partial dtype, then lse_partial [rows, P] float32."""
    d = good_dims(**kw)
    n = Q.decode_workspace_bytes(d, splits)
    rows = d.batch * d.s_q * d.heads * splits
    elem = 2 if d.cache_dtype == Q.QKN_BF16 else 4
    o_bytes = -(-rows * d.rank * elem // 256) * 256
    lse_bytes = -(-rows * 4 // 256) * 256
    assert n == o_bytes + lse_bytes
    assert n % 256 == 0


def test_workspace_bytes_invalid():
    lib = Q.library()
    assert lib.qkn_mla_decode_workspace_bytes(ctypes.byref(good_dims()), 0) == 0
    assert lib.qkn_mla_decode_workspace_bytes(ctypes.byref(good_dims()), 5000) == 0
    assert lib.qkn_mla_decode_workspace_bytes(ctypes.byref(good_dims(groups=3)), 4) == 0
    assert lib.qkn_mla_decode_workspace_bytes(None, 4) == 0


def test_decode_attend_rejects_bad_workspace():
    """A missing, misaligned or short workspace is refused before any launch."""
    lib = Q.library()
    d = good_dims()
    P = ctypes.c_void_p
    ok = P(1 << 20)  # never dereferenced: every call below is rejected first
    need = Q.decode_workspace_bytes(d, 8)

    def call(ws=ok, nbytes=need, splits=8, flags=0, o_lat=ok, q=ok):
        return lib.qkn_mla_decode_attend(ctypes.byref(d), q, ok, ok, ok, ok, ok, ok, splits,
                                         ctypes.c_uint32(flags), ws, ctypes.c_size_t(nbytes),
                                         o_lat, ok, None, None)
    assert call(ws=None) == -1
    assert call(nbytes=need - 1) == -1
    assert call(nbytes=0) == -1
    assert call(ws=P((1 << 20) + 128)) == -3   # 16-byte but not 256-byte aligned
    assert call(o_lat=None) == -1
    assert call(q=None) == -1
    assert call(q=P((1 << 20) + 8)) == -3
    assert call(splits=0) == -1
    assert call(flags=16) == -1


def test_noalloc_rejects_requests_beyond_its_scratch():
    """The allocation-free variant refuses, before any launch, a request whose
    partials would not fit its static scratch, and bad arguments as the
    workspace variant does."""
    lib = Q.library()
    P = ctypes.c_void_p
    ok = P(1 << 20)  # never dereferenced: every call below is rejected first

    def call(d, splits, o_lat=ok, q=ok):
        return lib.qkn_mla_decode_attend_noalloc(ctypes.byref(d), q, ok, ok, ok, ok, ok, ok, splits,
                                                 ctypes.c_uint32(0), o_lat, ok, None, None)
    big = good_dims(batch=64, s_q=4)             # 32768 rows: 4 splits need 128 MiB of partials
    assert Q.decode_workspace_bytes(big, 4) > Q.NOALLOC_SCRATCH_BYTES
    assert call(big, 4) == Q.QKN_ERR_SCRATCH
    d = good_dims(batch=32)                      # 4096 rows: 16 splits need 64 MiB + the lse
    assert Q.decode_workspace_bytes(d, 16) > Q.NOALLOC_SCRATCH_BYTES
    assert Q.decode_workspace_bytes(d, 15) <= Q.NOALLOC_SCRATCH_BYTES
    assert call(d, 16) == Q.QKN_ERR_SCRATCH
    assert call(d, 8, o_lat=None) == -1
    assert call(d, 8, q=None) == -1
    assert call(d, 8, o_lat=P((1 << 20) + 4)) == -3
    assert call(good_dims(groups=3), 8) == -1
    assert "static scratch" in Q.status_string(Q.QKN_ERR_SCRATCH)


def _call_sparse(d, ptr, idx_ptr, K, num_splits=1, flags=0):
    P = ctypes.c_void_p
    return Q.library().qkn_mla_decode_sparse(ctypes.byref(d), P(ptr), P(ptr), P(ptr), P(ptr),
                                             P(ptr), P(ptr), P(ptr), idx_ptr, K, num_splits,
                                             flags, P(ptr), P(ptr), None, None)


def test_sparse_decode_rejections():
    """The selected-token decode checks its arguments before any launch: the
    dense decode's checks, the list pointer and length, and the dims it takes
    (heads a multiple of 128, a cache under 4 GiB, at most 2048 entries per
    split, no forced vector-ALU kernel)."""
    P = ctypes.c_void_p
    d = good_dims()
    assert _call_sparse(d, 0x1000, None, 16) == -1                   # no list, entries > 0
    assert _call_sparse(d, 0x1000, P(0x1000), -1) == -1              # negative length
    assert _call_sparse(d, 0x1000, P(0x1004), 16) == -3              # misaligned list
    assert _call_sparse(d, 0x1008, P(0x1000), 16) == -3              # misaligned operands
    assert _call_sparse(d, 0x1000, P(0x1000), 16, num_splits=0) == -1
    assert _call_sparse(d, 0x1000, P(0x1000), 4096, num_splits=1) == -2   # 4096 entries in a split
    assert _call_sparse(d, 0x1000, P(0x1000), 16, flags=Q.QKN_DECODE_FORCE_GENERIC) == -2
    assert _call_sparse(good_dims(heads=64), 0x1000, P(0x1000), 16) == -2  # two tokens per workgroup
    assert _call_sparse(good_dims(cache_dtype="f32"), 0x1000, P(0x1000), 16) == -2
    big = good_dims(num_pages=60000)                                 # 4.4 GB of cache rows
    assert _call_sparse(big, 0x1000, P(0x1000), 16) == -2


def test_prefill_rejections():
    """The prefill calls check their arguments before any launch: the dims they
    take (bf16 cache, r = 512, d = 128, d_R = 64, a multiple of 32 heads per
    group), null pointers and misalignment."""
    lib = Q.library()
    P = ctypes.c_void_p
    a = [P(0x1000)] * 11
    d = good_dims(s_q=64)
    for bad in (good_dims(cache_dtype="f32"), good_dims(head_dim=64), good_dims(heads=48, groups=1)):
        assert lib.qkn_mla_prefill_query(ctypes.byref(bad), *a[:7], None) == -2
        assert lib.qkn_mla_prefill_expand(ctypes.byref(bad), *a[:9], None, None) == -2
        assert lib.qkn_mla_prefill_attend(ctypes.byref(bad), *a[:9], None, None) == -2
    assert lib.qkn_mla_prefill_query(ctypes.byref(d), None, *a[:6], None) == -1
    assert lib.qkn_mla_prefill_expand(ctypes.byref(d), *a[:8], None, None, None) == -1
    assert lib.qkn_mla_prefill_attend(ctypes.byref(d), *a[:8], None, None, None) == -1
    assert lib.qkn_mla_prefill_query(ctypes.byref(d), P(0x1004), *a[:6], None) == -3
    assert lib.qkn_mla_prefill_expand(ctypes.byref(d), P(0x1008), *a[:8], None, None) == -3
    assert lib.qkn_mla_prefill_attend(ctypes.byref(d), *a[:8], P(0x1004), None, None) == -3


def test_gqa_rejections():
    """The GQA-path calls check their arguments before any launch: the dims
    they take (bf16 latent dtype, d = 128, d_R = 64, r a multiple of 16, a
    multiple of 32 heads per group), null pointers, misalignment, split counts
    and the workspace of a split attention."""
    lib = Q.library()
    P = ctypes.c_void_p
    a = [P(0x1000)] * 12
    d = good_dims(s_q=4)
    for bad in (good_dims(cache_dtype="f32"), good_dims(head_dim=64), good_dims(heads=48, groups=1),
                good_dims(rank=72)):
        assert lib.qkn_mla_gqa_append(ctypes.byref(bad), 4, *a[:10], None, None) == -2
        assert lib.qkn_mla_gqa_attend(ctypes.byref(bad), *a[:5], 1, None, 0, *a[:2], None,
                                      None) == -2
    assert lib.qkn_mla_gqa_append(ctypes.byref(d), 0, *[None] * 10, None, None) == 0  # nothing to do
    assert lib.qkn_mla_gqa_append(ctypes.byref(d), -1, *a[:10], None, None) == -1
    assert lib.qkn_mla_gqa_append(ctypes.byref(d), 4, *a[:9], None, None, None) == -1
    assert lib.qkn_mla_gqa_append(ctypes.byref(d), 4, P(0x1008), *a[:9], None, None) == -3
    ws = lib.qkn_mla_gqa_workspace_bytes(ctypes.byref(d), 3)
    rows = d.batch * d.s_q * d.heads * 3
    assert ws >= rows * d.head_dim * 2 + rows * 4 and ws % 256 == 0
    assert lib.qkn_mla_gqa_workspace_bytes(ctypes.byref(d), 0) == 0
    attend = lambda P_, w, nb, q=P(0x1000): lib.qkn_mla_gqa_attend(  # noqa: E731
        ctypes.byref(d), q, *a[:4], P_, w, nb, *a[:2], None, None)
    assert attend(0, None, 0) == -1
    assert attend(3, None, 0) == -1                          # no workspace
    assert attend(3, P(0x1000), ws - 1) == -1                # too small
    assert attend(3, P(0x1010), ws) == -3                    # not 256-byte aligned
    assert attend(1, None, 0, q=None) == -1
    assert attend(1, None, 0, q=P(0x1004)) == -3


def test_stream_read_rejections():
    lib = Q.library()
    P = ctypes.c_void_p
    assert lib.qkn_mla_stream_read(None, 64, P(0x1000), None) == -1        # no source
    assert lib.qkn_mla_stream_read(P(0x1000), 64, None, None) == -1        # no sink
    assert lib.qkn_mla_stream_read(P(0x1000), 0, P(0x1000), None) == -1    # nothing to read
    assert lib.qkn_mla_stream_read(P(0x1000), 40, P(0x1000), None) == -1   # not whole 16-byte words
    assert lib.qkn_mla_stream_read(P(0x1008), 64, P(0x1000), None) == -3   # misaligned source
    assert lib.qkn_mla_stream_read(P(0x1000), 64, P(0x1002), None) == -3   # misaligned sink
