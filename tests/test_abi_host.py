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
    assert len(syms) == 9, syms
    assert set(syms) == set(Q.EXPORTED_SYMBOLS)
    for s in syms:
        assert hasattr(lib, s), f"{s} not exported"


def test_only_the_c_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {Q.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(Q.EXPORTED_SYMBOLS), exported ^ set(Q.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    lib = Q.library()
    assert lib.qkn_mla_abi_version() == Q.ABI_VERSION == 3
    for st in (0, -1, -2, -3, -4):
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
