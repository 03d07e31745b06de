"""Python binding of libqknmla.so (QK-Normed MLA absorbed-latent decode on MI355X).

Argument marshalling only: every step of the decode runs in the HIP kernels of
the shared library.  Tensors supply device pointers; the current torch stream
supplies the HIP stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

The functions carry the names of the C entry points (include/qkn_mla.h):

    qkn_mla_absorb_query, qkn_mla_append, qkn_mla_decode, qkn_mla_combine,
    qkn_mla_decode_attend, qkn_mla_combine_project

and check on the host that every tensor is a contiguous device tensor of the
dtype and element count the kernels and their grids assume before launching.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqknmla.so")

ABI_VERSION = 9
QKN_OK = 0
QKN_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 64 << 20
QKN_F32 = 0
QKN_BF16 = 1
QKN_F16 = 2
QKN_DECODE_NO_ALPHA = 1
QKN_DECODE_FORCE_GENERIC = 2
QKN_FLAG_INDEX = 1
QKN_FLAG_PARTIAL_RANGE = 2
QKN_FLAG_RESTART = 4
QKN_PROJECT_FUSED = 1
QKN_PROJECT_TWO_PASS = 2
PAGE_SIZE = 64

_c_int32 = ctypes.c_int32
_c_float = ctypes.c_float


class Dims(ctypes.Structure):
    """qkn_mla_dims."""
    _fields_ = [
        ("batch", _c_int32), ("s_q", _c_int32), ("heads", _c_int32), ("groups", _c_int32),
        ("rank", _c_int32), ("head_dim", _c_int32), ("rope_dim", _c_int32),
        ("page_size", _c_int32), ("max_pages_per_seq", _c_int32), ("num_pages", _c_int32),
        ("eps", _c_float), ("softmax_scale", _c_float), ("rope_theta", _c_float),
        ("cache_dtype", _c_int32),
    ]

    def __repr__(self):
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class QknError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


_lib = None


def library() -> ctypes.CDLL:
    """Load libqknmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m qk_normed_mla_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(Dims)
        lib.qkn_mla_abi_version.restype = ctypes.c_int
        lib.qkn_mla_abi_version.argtypes = []
        lib.qkn_status_string.restype = ctypes.c_char_p
        lib.qkn_status_string.argtypes = [ctypes.c_int]
        lib.qkn_mla_check_dims.restype = ctypes.c_int
        lib.qkn_mla_check_dims.argtypes = [D]
        lib.qkn_mla_partial_dtype.restype = ctypes.c_int
        lib.qkn_mla_partial_dtype.argtypes = [D]
        lib.qkn_mla_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.qkn_mla_decode_workspace_bytes.argtypes = [D, _c_int32]
        lib.qkn_mla_decode_kernel_kind.restype = ctypes.c_int
        lib.qkn_mla_decode_kernel_kind.argtypes = [D, _c_int32, ctypes.c_uint32]
        lib.qkn_mla_absorb_query.restype = ctypes.c_int
        lib.qkn_mla_absorb_query.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
        lib.qkn_mla_append.restype = ctypes.c_int
        lib.qkn_mla_append.argtypes = [D, _c_int32, P, P, P, P, P, P, P, P, P, P, P]
        lib.qkn_mla_decode.restype = ctypes.c_int
        lib.qkn_mla_decode.argtypes = [D, P, P, P, P, P, P, P, _c_int32, ctypes.c_uint32,
                                       P, P, P, P]
        lib.qkn_mla_prefill_query.restype = ctypes.c_int
        lib.qkn_mla_prefill_query.argtypes = [D, P, P, P, P, P, P, P, P]
        lib.qkn_mla_prefill_expand.restype = ctypes.c_int
        lib.qkn_mla_prefill_expand.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
        lib.qkn_mla_prefill_attend.restype = ctypes.c_int
        lib.qkn_mla_prefill_attend.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
        lib.qkn_mla_decode_sparse.restype = ctypes.c_int
        lib.qkn_mla_decode_sparse.argtypes = [D, P, P, P, P, P, P, P, P, _c_int32, _c_int32,
                                              ctypes.c_uint32, P, P, P, P]
        lib.qkn_mla_decode_attend.restype = ctypes.c_int
        lib.qkn_mla_decode_attend.argtypes = [D, P, P, P, P, P, P, P, _c_int32, ctypes.c_uint32,
                                              P, ctypes.c_size_t, P, P, P, P]
        lib.qkn_mla_decode_attend_noalloc.restype = ctypes.c_int
        lib.qkn_mla_decode_attend_noalloc.argtypes = [D, P, P, P, P, P, P, P, _c_int32,
                                                      ctypes.c_uint32, P, P, P, P]
        lib.qkn_mla_combine.restype = ctypes.c_int
        lib.qkn_mla_combine.argtypes = [D, _c_int32, P, P, P, P, P]
        lib.qkn_mla_combine_project.restype = ctypes.c_int
        lib.qkn_mla_combine_project.argtypes = [D, _c_int32, P, P, P, P, P, P, ctypes.c_uint32, P]
        lib.qkn_mla_gqa_append.restype = ctypes.c_int
        lib.qkn_mla_gqa_append.argtypes = [D, _c_int32, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.qkn_mla_gqa_workspace_bytes.restype = ctypes.c_size_t
        lib.qkn_mla_gqa_workspace_bytes.argtypes = [D, _c_int32]
        lib.qkn_mla_gqa_attend.restype = ctypes.c_int
        lib.qkn_mla_gqa_attend.argtypes = [D, P, P, P, P, P, _c_int32, P, ctypes.c_size_t, P, P, P,
                                           P]
        lib.qkn_mla_stream_read.restype = ctypes.c_int
        lib.qkn_mla_stream_read.argtypes = [P, ctypes.c_uint64, P, P]
        if lib.qkn_mla_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.qkn_mla_abi_version()}, "
                               f"this binding needs {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


EXPORTED_SYMBOLS = (
    "qkn_mla_abi_version", "qkn_status_string", "qkn_mla_check_dims",
    "qkn_mla_partial_dtype", "qkn_mla_decode_workspace_bytes",
    "qkn_mla_decode_kernel_kind", "qkn_mla_absorb_query", "qkn_mla_append",
    "qkn_mla_decode", "qkn_mla_decode_sparse", "qkn_mla_decode_attend",
    "qkn_mla_decode_attend_noalloc",
    "qkn_mla_combine", "qkn_mla_combine_project",
    "qkn_mla_prefill_query", "qkn_mla_prefill_expand", "qkn_mla_prefill_attend",
    "qkn_mla_gqa_append", "qkn_mla_gqa_workspace_bytes", "qkn_mla_gqa_attend",
    "qkn_mla_stream_read",
)


def status_string(status: int) -> str:
    return library().qkn_status_string(int(status)).decode()


def make_dims(*, batch, s_q, heads, groups, rank, head_dim, rope_dim, max_pages_per_seq,
              num_pages, eps, softmax_scale, rope_theta, cache_dtype) -> Dims:
    dt = {"f32": QKN_F32, "bf16": QKN_BF16}.get(cache_dtype, cache_dtype)
    return Dims(batch, s_q, heads, groups, rank, head_dim, rope_dim, PAGE_SIZE,
                max_pages_per_seq, num_pages, eps, softmax_scale, rope_theta, dt)


def dims_for(wl, num_pages: int) -> Dims:
    """Dims of a workloads.Workload with a pool of ``num_pages`` pages."""
    return make_dims(batch=wl.batch, s_q=wl.s_q, heads=wl.heads, groups=wl.groups,
                     rank=wl.rank, head_dim=wl.head_dim, rope_dim=wl.rope_dim,
                     max_pages_per_seq=wl.max_pages_per_seq, num_pages=num_pages, eps=wl.eps,
                     softmax_scale=wl.softmax_scale, rope_theta=wl.rope_theta,
                     cache_dtype=wl.cache_dtype)


def cache_torch_dtype(dims: Dims) -> torch.dtype:
    return torch.bfloat16 if dims.cache_dtype == QKN_BF16 else torch.float32


_TORCH_OF = {QKN_F32: torch.float32, QKN_BF16: torch.bfloat16, QKN_F16: torch.float16}


def partial_torch_dtype(dims: Dims) -> torch.dtype:
    """Element type of the split-KV partials, as the library reports it."""
    code = library().qkn_mla_partial_dtype(ctypes.byref(dims))
    if code < 0:
        raise QknError("qkn_mla_partial_dtype", code)
    return _TORCH_OF[code]


def decode_workspace_bytes(dims: Dims, num_splits: int) -> int:
    """Device bytes qkn_mla_decode_attend needs for ``num_splits`` partitions."""
    n = int(library().qkn_mla_decode_workspace_bytes(ctypes.byref(dims), int(num_splits)))
    if n == 0:
        raise QknError("qkn_mla_decode_workspace_bytes", -1)
    return n


def alloc_decode_workspace(dims: Dims, num_splits: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of the size qkn_mla_decode_workspace_bytes states
    (torch's allocator returns 256-byte aligned blocks)."""
    ws = torch.empty(decode_workspace_bytes(dims, num_splits), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace not 256-byte aligned")
    return ws


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype, numel: int, allow_none=False):
    if t is None:
        if allow_none or numel == 0:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()} {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _check(fn: str, status: int):
    if status != QKN_OK:
        raise QknError(fn, status)


def decode_kernel_kind(dims: Dims, num_splits: int, flags: int = 0) -> int:
    return library().qkn_mla_decode_kernel_kind(ctypes.byref(dims), int(num_splits), int(flags))


def qkn_mla_absorb_query(dims: Dims, q, q_rope, q_pos, w_k, gamma_q, gamma_k, gamma_qr,
                         q_tilde, alpha_q, q_rope_normed, stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    st = library().qkn_mla_absorb_query(
        ctypes.byref(d),
        _ptr(q, "q", f32, rows * d.head_dim),
        _ptr(q_rope, "q_rope", f32, rows * d.rope_dim),
        _ptr(q_pos, "q_pos", i32, d.batch * d.s_q),
        _ptr(w_k, "w_k", f32, d.groups * d.rank * d.head_dim),
        _ptr(gamma_q, "gamma_q", f32, d.head_dim),
        _ptr(gamma_k, "gamma_k", f32, d.groups * d.head_dim),
        _ptr(gamma_qr, "gamma_qr", f32, d.rope_dim),
        _ptr(q_tilde, "q_tilde", ct, rows * d.rank),
        _ptr(alpha_q, "alpha_q", f32, rows),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_absorb_query", st)


def qkn_mla_append(dims: Dims, c_new, k_rope_new, seq_idx, pos, block_table, w_k, gamma_kr,
                   kv_cache, alpha_k_cache, err_flag=None, stream=None):
    d = dims
    n = int(seq_idx.numel()) if seq_idx is not None else 0
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    st = library().qkn_mla_append(
        ctypes.byref(d), n,
        _ptr(c_new, "c_new", f32, n * d.rank),
        _ptr(k_rope_new, "k_rope_new", f32, n * d.rope_dim),
        _ptr(seq_idx, "seq_idx", i32, n),
        _ptr(pos, "pos", i32, n),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(w_k, "w_k", f32, d.groups * d.rank * d.head_dim),
        _ptr(gamma_kr, "gamma_kr", f32, d.rope_dim),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(alpha_k_cache, "alpha_k_cache", f32, d.num_pages * PAGE_SIZE * d.groups),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_append", st)


def qkn_mla_decode(dims: Dims, q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache,
                   block_table, seq_lens, num_splits: int, flags: int, o_partial, lse_partial,
                   err_flag=None, stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    P = int(num_splits)
    st = library().qkn_mla_decode(
        ctypes.byref(d),
        _ptr(q_tilde, "q_tilde", ct, rows * d.rank),
        _ptr(alpha_q, "alpha_q", f32, rows),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(alpha_k_cache, "alpha_k_cache", f32, d.num_pages * PAGE_SIZE * d.groups),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", i32, d.batch),
        P, int(flags),
        _ptr(o_partial, "o_partial", partial_torch_dtype(d), rows * P * d.rank),
        _ptr(lse_partial, "lse_partial", f32, rows * P),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_decode", st)


def qkn_mla_prefill_query(dims: Dims, q, q_rope, q_pos, gamma_q, gamma_qr, q_hat, q_rope_normed,
                          stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    st = library().qkn_mla_prefill_query(
        ctypes.byref(d),
        _ptr(q, "q", f32, rows * d.head_dim),
        _ptr(q_rope, "q_rope", f32, rows * d.rope_dim),
        _ptr(q_pos, "q_pos", i32, d.batch * d.s_q),
        _ptr(gamma_q, "gamma_q", f32, d.head_dim),
        _ptr(gamma_qr, "gamma_qr", f32, d.rope_dim),
        _ptr(q_hat, "q_hat", torch.float16, rows * d.head_dim),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_prefill_query", st)


def qkn_mla_prefill_expand(dims: Dims, kv_cache, alpha_k_cache, block_table, seq_lens, w_k, w_v,
                           gamma_k, k_hat, v, err_flag=None, stream=None):
    d = dims
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    n_kv = d.batch * d.max_pages_per_seq * PAGE_SIZE * d.groups * d.head_dim
    st = library().qkn_mla_prefill_expand(
        ctypes.byref(d),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(alpha_k_cache, "alpha_k_cache", f32, d.num_pages * PAGE_SIZE * d.groups),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", i32, d.batch),
        _ptr(w_k, "w_k", f32, d.groups * d.rank * d.head_dim),
        _ptr(w_v, "w_v", f32, d.groups * d.rank * d.head_dim),
        _ptr(gamma_k, "gamma_k", f32, d.groups * d.head_dim),
        _ptr(k_hat, "k_hat", torch.float16, n_kv),
        _ptr(v, "v", torch.float16, n_kv),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_prefill_expand", st)


def qkn_mla_prefill_attend(dims: Dims, q_hat, q_rope_normed, k_hat, v, kv_cache, block_table,
                           seq_lens, o, lse, err_flag=None, stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    n_kv = d.batch * d.max_pages_per_seq * PAGE_SIZE * d.groups * d.head_dim
    st = library().qkn_mla_prefill_attend(
        ctypes.byref(d),
        _ptr(q_hat, "q_hat", torch.float16, rows * d.head_dim),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        _ptr(k_hat, "k_hat", torch.float16, n_kv),
        _ptr(v, "v", torch.float16, n_kv),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", i32, d.batch),
        _ptr(o, "o", f32, rows * d.head_dim),
        _ptr(lse, "lse", f32, rows),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_prefill_attend", st)


def qkn_mla_decode_sparse(dims: Dims, q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache,
                          block_table, seq_lens, indices, num_splits: int, flags: int, o_partial,
                          lse_partial, err_flag=None, stream=None):
    """Selected-token decode: ``indices`` [B, s_q, K] int32 (logical positions,
    -1 unused) on the device; partials as for :func:`qkn_mla_decode`."""
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    P = int(num_splits)
    K = int(indices.shape[-1]) if indices is not None else 0
    st = library().qkn_mla_decode_sparse(
        ctypes.byref(d),
        _ptr(q_tilde, "q_tilde", ct, rows * d.rank),
        _ptr(alpha_q, "alpha_q", f32, rows),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(alpha_k_cache, "alpha_k_cache", f32, d.num_pages * PAGE_SIZE * d.groups),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", i32, d.batch),
        _ptr(indices, "indices", i32, d.batch * d.s_q * K, allow_none=K == 0),
        K, P, int(flags),
        _ptr(o_partial, "o_partial", partial_torch_dtype(d), rows * P * d.rank),
        _ptr(lse_partial, "lse_partial", f32, rows * P),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_decode_sparse", st)


def qkn_mla_decode_attend(dims: Dims, q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache,
                          block_table, seq_lens, num_splits: int, flags: int, workspace,
                          o_latent, lse, err_flag=None, stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    need = decode_workspace_bytes(d, num_splits)
    if workspace is None or workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 device tensor of at least {need} bytes")
    st = library().qkn_mla_decode_attend(
        ctypes.byref(d),
        _ptr(q_tilde, "q_tilde", ct, rows * d.rank),
        _ptr(alpha_q, "alpha_q", f32, rows),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(alpha_k_cache, "alpha_k_cache", f32, d.num_pages * PAGE_SIZE * d.groups),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", i32, d.batch),
        int(num_splits), int(flags),
        _ptr(workspace, "workspace", torch.uint8, workspace.numel()),
        ctypes.c_size_t(workspace.numel()),
        _ptr(o_latent, "o_latent", f32, rows * d.rank),
        _ptr(lse, "lse", f32, rows),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_decode_attend", st)


def qkn_mla_decode_attend_noalloc(dims: Dims, q_tilde, alpha_q, q_rope_normed, kv_cache,
                                  alpha_k_cache, block_table, seq_lens, num_splits: int,
                                  flags: int, o_latent, lse, err_flag=None, stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    ct = cache_torch_dtype(d)
    f32, i32 = torch.float32, torch.int32
    st = library().qkn_mla_decode_attend_noalloc(
        ctypes.byref(d),
        _ptr(q_tilde, "q_tilde", ct, rows * d.rank),
        _ptr(alpha_q, "alpha_q", f32, rows),
        _ptr(q_rope_normed, "q_rope_normed", ct, rows * d.rope_dim),
        _ptr(kv_cache, "kv_cache", ct, d.num_pages * PAGE_SIZE * (d.rank + d.rope_dim)),
        _ptr(alpha_k_cache, "alpha_k_cache", f32, d.num_pages * PAGE_SIZE * d.groups),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", i32, d.batch),
        int(num_splits), int(flags),
        _ptr(o_latent, "o_latent", f32, rows * d.rank),
        _ptr(lse, "lse", f32, rows),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_decode_attend_noalloc", st)


def qkn_mla_combine(dims: Dims, num_splits: int, o_partial, lse_partial, o_latent, lse,
                    stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    f32 = torch.float32
    P = int(num_splits)
    st = library().qkn_mla_combine(
        ctypes.byref(d), P,
        _ptr(o_partial, "o_partial", partial_torch_dtype(d), rows * P * d.rank),
        _ptr(lse_partial, "lse_partial", f32, rows * P),
        _ptr(o_latent, "o_latent", f32, rows * d.rank),
        _ptr(lse, "lse", f32, rows),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_combine", st)


def qkn_mla_combine_project(dims: Dims, num_splits: int, o_partial, lse_partial, w_v, o_latent,
                            lse, o, flags: int = 0, stream=None):
    d = dims
    rows = d.batch * d.s_q * d.heads
    f32 = torch.float32
    P = int(num_splits)
    st = library().qkn_mla_combine_project(
        ctypes.byref(d), P,
        _ptr(o_partial, "o_partial", partial_torch_dtype(d), rows * P * d.rank),
        _ptr(lse_partial, "lse_partial", f32, rows * P),
        _ptr(w_v, "w_v", f32, d.groups * d.rank * d.head_dim),
        _ptr(o_latent, "o_latent", f32, rows * d.rank),
        _ptr(lse, "lse", f32, rows),
        _ptr(o, "o", f32, rows * d.head_dim),
        ctypes.c_uint32(int(flags)), ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_combine_project", st)


# -- the GQA path ----------------------------------------------------------------

def gqa_row_words(dims: Dims) -> int:
    """16-bit words per token of the GQA cache: every group's key and value
    (half) and the shared RoPE key (bf16)."""
    return 2 * dims.groups * dims.head_dim + dims.rope_dim


def gqa_workspace_bytes(dims: Dims, num_splits: int) -> int:
    n = int(library().qkn_mla_gqa_workspace_bytes(ctypes.byref(dims), int(num_splits)))
    if n == 0:
        raise QknError("qkn_mla_gqa_workspace_bytes", -1)
    return n


def qkn_mla_gqa_append(dims: Dims, c_new, k_rope_new, seq_idx, pos, block_table, w_k, w_v,
                       gamma_k, gamma_kr, kvg_cache, err_flag=None, stream=None):
    """``kvg_cache``: int16 words [num_pages, 64, gqa_row_words(dims)]."""
    d = dims
    n = int(seq_idx.numel()) if seq_idx is not None else 0
    f32, i32 = torch.float32, torch.int32
    st = library().qkn_mla_gqa_append(
        ctypes.byref(d), n,
        _ptr(c_new, "c_new", f32, n * d.rank),
        _ptr(k_rope_new, "k_rope_new", f32, n * d.rope_dim),
        _ptr(seq_idx, "seq_idx", i32, n),
        _ptr(pos, "pos", i32, n),
        _ptr(block_table, "block_table", i32, d.batch * d.max_pages_per_seq),
        _ptr(w_k, "w_k", f32, d.groups * d.rank * d.head_dim),
        _ptr(w_v, "w_v", f32, d.groups * d.rank * d.head_dim),
        _ptr(gamma_k, "gamma_k", f32, d.groups * d.head_dim),
        _ptr(gamma_kr, "gamma_kr", f32, d.rope_dim),
        _ptr(kvg_cache, "kvg_cache", torch.int16, d.num_pages * PAGE_SIZE * gqa_row_words(d)),
        _ptr(err_flag, "err_flag", i32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_gqa_append", st)


def qkn_mla_gqa_attend(dims: Dims, q_hat, q_rope_normed, kvg_cache, block_table, seq_lens,
                       num_splits: int, workspace, o, lse, err_flag=None, stream=None):
    """``workspace``: a uint8 device buffer of gqa_workspace_bytes(dims,
    num_splits) bytes, or None when num_splits == 1."""
    d = dims
    rows = d.batch * d.s_q * d.heads
    ws_bytes = 0 if workspace is None else int(workspace.numel())
    st = library().qkn_mla_gqa_attend(
        ctypes.byref(d),
        _ptr(q_hat, "q_hat", torch.float16, rows * d.head_dim),
        _ptr(q_rope_normed, "q_rope_normed", cache_torch_dtype(d), rows * d.rope_dim),
        _ptr(kvg_cache, "kvg_cache", torch.int16, d.num_pages * PAGE_SIZE * gqa_row_words(d)),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_pages_per_seq),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        int(num_splits),
        _ptr(workspace, "workspace", torch.uint8, ws_bytes, allow_none=True),
        ws_bytes,
        _ptr(o, "o", torch.float32, rows * d.head_dim),
        _ptr(lse, "lse", torch.float32, rows),
        _ptr(err_flag, "err_flag", torch.int32, 1, allow_none=True),
        ctypes.c_void_p(_stream_ptr(stream)))
    _check("qkn_mla_gqa_attend", st)
