"""Shared pieces of the GPU parity tests (inputs, uploads, comparisons)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import qk_normed_mla_amd as Q
from qk_normed_mla_amd.runner import DecodeRunner

# Tolerances.  Floating point: row-normwise max relative error
# max |gpu - ref| / max |ref| over each latent row (b, i, h), and absolute error
# on lse.  Float32 cache: 1e-4; bf16 cache with float32 accumulation: 1e-2
# end to end (from the float32 inputs against the float64 explicit path).
#
# The decode kernel alone, run on the oracle's own stored state:
#  * vector-ALU kernel (float32 throughout): 1e-5 row-relative.
#  * matrix-core kernel: each probability enters the P.C product rounded to
#    bf16, p~_t = p_t (1 + e_t) with |e_t| <= 2^-9, and the row is normalised by
#    the sum of the same rounded values, so o = sum_t w_t c_t stays a convex
#    combination whose weights moved by w_t (e_t - e_mean) / (1 + e_mean), i.e.
#    by at most ~2^-8 relative.  Hence |delta o_m| <= 2^-8 sum_t w_t |c_tm - o_m|
#    <= 2^-8 * 2 max_t |c_tm| = 2^-7 max_t |c_tm|.  The split-KV combine keeps
#    one rounding per token, so the bound holds for the merged result too.  It
#    is absolute, per row, in units of the largest latent entry the row can
#    see (KERNEL_P_ROUND), plus 1e-5 relative for float32 accumulation.  lse
#    moves by <= ln(1 + 2^-9) from the rounding of the weights, plus the float32
#    error of the logits themselves: a K = 576 dot accumulated in float32 is off
#    by ~576 * 2^-24 * sum |q~_m c_m| (~1e-3 for the unnormalised logits of the
#    alpha-free test), times the softmax scale; 2e-4 covers it.
#    The logits themselves carry the float32 error of a K-term dot product,
#    |dS_t| <= gamma_K * sum_m |q~_m c_tm| (standard bound, gamma_K = K u / (1 - K u),
#    u = 2^-24), computed per row by logit_error_bound(); it adds to the lse bound
#    and, through the weights (|dw/w| <= 2 max_t |dl_t|), to the latent bound.
#  * the split partials are stored as half for a bf16 cache: each is a convex
#    combination of the latent rows its split sees, so storing it moves it by
#    at most 2^-11 of its largest entry, <= 2^-11 max_t |c_tm| (KERNEL_PART_ROUND,
#    absolute, in the same units as KERNEL_P_ROUND); the combine's weights sum
#    to 1, so the merged row moves by no more.  A float32 cache keeps float32
#    partials (0).
TOL_E2E = {"f32": 1e-4, "bf16": 1e-2}
KERNEL_PART_ROUND = {"f32": 0.0, "bf16": 2.0 ** -11}
TOL_KERNEL_GENERIC = 1e-5
KERNEL_P_ROUND = 2.0 ** -7
KERNEL_LSE = float(np.log1p(2.0 ** -9))


def gamma_k(k: int) -> float:
    u = 2.0 ** -24
    return k * u / (1.0 - k * u)


def logit_error_bound(scale, q_tilde, alpha_q, qr_hat, C, alpha_k, KR):
    """Per-head bound (natural-log logit units) on the float32 error of
    l_t = scale * (a_q a_k,t (q~ . c_t) + q^R . k^R_t) over the tokens C, KR."""
    content = np.abs(q_tilde) @ np.abs(C).T * np.abs(alpha_q)[:, None] * np.abs(alpha_k)[None, :]
    rope = np.abs(qr_hat) @ np.abs(KR).T
    K = C.shape[1] + KR.shape[1]
    return scale * gamma_k(K) * np.max(content + rope, axis=1) * 1.01 + 1e-6


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    Q.library()  # raises when the HIP library is missing


def row_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))


def ulp_distance_bf16(a_words, b_words):
    """Distance in representable bf16 steps between two arrays of words."""
    def ordered(w):
        w = np.asarray(w, dtype=np.uint16).astype(np.int32)
        return np.where(w & 0x8000, -(w & 0x7FFF), w)
    return np.abs(ordered(a_words) - ordered(b_words))


def upload_words(words, like: torch.Tensor) -> torch.Tensor:
    """Host storage words -> a device tensor of ``like``'s dtype and shape."""
    if like.dtype == torch.bfloat16:
        t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).to(like.device)
        return t.view(torch.bfloat16).reshape(like.shape)
    return torch.from_numpy(np.ascontiguousarray(words, dtype=np.float32)).to(like.device).reshape(like.shape)


def run_e2e(wl, inp, num_splits=None, flags=0, kv_fill_word=None):
    r = DecodeRunner(wl, inp, num_splits=num_splits, kv_fill_word=kv_fill_word)
    r.fill_history()
    r.step(flags)
    torch.cuda.synchronize()
    return r
