"""Shared pieces of the GPU parity tests (inputs, uploads, comparisons)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import qk_normed_mla_amd as Q
from qk_normed_mla_amd.runner import DecodeRunner

# Tolerances.  Floating point: row-normwise max relative error
# max |gpu - ref| / max |ref| over each latent row (b, i, h), and absolute error
# on lse.  Float32 cache: 1e-4; bf16 cache with float32 accumulation: 1e-2.
# Every floating-point comparison is held to these, end to end (float32 inputs
# against the float64 explicit path) and for the decode kernel alone (on the
# oracle's own stored state) alike.
#
# The decode kernel alone is also held element by element to a bound derived
# from its arithmetic, with the oracle's float64 weights w_t of the same tokens
# (one split for a partial, every visible token for the merged row) and the
# exact result o:
#  * the matrix-core kernel feeds each probability into the P.C product rounded
#    to bf16, p~_t = p_t (1 + e_t), |e_t| <= u = 2^-8, and normalises by the sum
#    of the same rounded values; its logits carry the float32 error of a
#    K-term dot product, |dl_t| <= D (logit_error_bound(), natural-log units,
#    plus the exponent's own rounding).  The weights it uses are
#    w~_t = w_t f_t / sum_s w_s f_s with f_t = (1 + e_t) e^{dl_t}, so
#    |w~_t / w_t - 1| <= R - 1, R = (1 + u) / (1 - u) * e^{2 D}.  Since both
#    weight sets sum to 1,
#        o~_m - o_m = sum_t (w~_t - w_t)(c_tm - o_m),
#        |o~_m - o_m| <= (R - 1) * S_m,   S_m = sum_t w_t |c_tm - o_m|.
#  * the sums run in float32 over n tokens: gamma_n (A_m + |o_m|), with
#    A_m = sum_t w_t |c_tm| (the P.C sum and its normaliser).
#  * for a bf16 cache the split partials are stored as IEEE half (relative
#    step 2^-11): 2^-11 |o_p,m| for a partial; the combine's weights sum to 1,
#    so the merged row moves by at most 2^-11 A_m.
#  * lse: ln R from the weights plus D from the logits, plus float32 rounding.
# The vector-ALU kernel keeps probabilities and partials (for a float32 cache)
# in float32: the same form with u = 2^-24.
TOL_E2E = {"f32": 1e-4, "bf16": 1e-2}
U_PROB = {1: 2.0 ** -8, 0: 2.0 ** -24, 2: 2.0 ** -11}  # probability rounding: bf16, float32, half
U_PART = {"f32": 0.0, "bf16": 2.0 ** -11}   # storage of the split partials
# a float32 cache keeps float32 partials: the vector-ALU kernel's row-relative bar
TOL_KERNEL_GENERIC = 1e-5
KERNEL_PART_ROUND = U_PART


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
    """Distance in representable steps between two arrays of 16-bit
    sign-magnitude words (bf16, or IEEE half: the same ordering holds)."""
    def ordered(w):
        w = np.asarray(w, dtype=np.uint16).astype(np.int32)
        return np.where(w & 0x8000, -(w & 0x7FFF), w)
    return np.abs(ordered(a_words) - ordered(b_words))


def upload_words(words, like: torch.Tensor) -> torch.Tensor:
    """Host storage words -> a device tensor of ``like``'s dtype and shape."""
    if like.dtype in (torch.bfloat16, torch.float16):
        t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).to(like.device)
        return t.view(like.dtype).reshape(like.shape)
    return torch.from_numpy(np.ascontiguousarray(words, dtype=np.float32)).to(like.device).reshape(like.shape)


def run_e2e(wl, inp, num_splits=None, flags=0, kv_fill_word=None):
    r = DecodeRunner(wl, inp, num_splits=num_splits, kv_fill_word=kv_fill_word)
    r.fill_history()
    r.step(flags)
    torch.cuda.synchronize()
    return r


def weighted_moments(C, w, o):
    """S_m = sum_t w_t |c_tm - o_m| and A_m = sum_t w_t |c_tm| for weights w [n]
    over latent rows C [n, r] with the exact result o [r]."""
    return w @ np.abs(C - o[None, :]), w @ np.abs(C)


def kernel_elementwise_bound(kind, cache_dtype, w, C, o, D, n, partial):
    """Per-element bound on |o~_m - o_m| for one row (see the derivation at the
    top of this module).  ``partial``: the row is a stored split partial (its
    own half step) rather than the merged row."""
    u = U_PROB[kind]
    R = (1.0 + u) / (1.0 - u) * np.exp(2.0 * D)
    S, A = weighted_moments(C, w, o)
    g = gamma_k(n + 1)
    half = U_PART[cache_dtype]
    store = half * (np.abs(o) if partial else A)
    return (R - 1.0) * S * 1.001 + g * (A + np.abs(o)) + store + 1e-7 * np.max(np.abs(o))


def kernel_lse_bound(kind, D, n):
    u = U_PROB[kind]
    return float(np.log((1.0 + u) / (1.0 - u))) + D + 2.0 * gamma_k(n + 1) + 2e-6
