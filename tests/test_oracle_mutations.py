"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Each case monkeypatches one oracle function with a wrong variant (a dropped
term, a wrong sign or index, a misplaced epsilon, a transposed operand ...) and
runs the pins that should notice; the test passes only if at least one of them
fails.  The mistakes are planted in the oracle, on the CPU, never in GPU code.
"""
import numpy as np
import pytest

import oracle_pins as P
from oracle import qkn_oracle as O

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _absorb_without_gamma_k(wl, q, q_rope, w_k, gamma_q, gamma_k, gamma_qr, q_pos):
    return _orig["absorb_query"](wl, q, q_rope, w_k, gamma_q, np.ones_like(gamma_k), gamma_qr, q_pos)


def _absorb_shifted_position(wl, q, q_rope, w_k, gamma_q, gamma_k, gamma_qr, q_pos):
    return _orig["absorb_query"](wl, q, q_rope, w_k, gamma_q, gamma_k, gamma_qr, np.asarray(q_pos) + 1)


def _absorb_transposed_w(wl, q, q_rope, w_k, gamma_q, gamma_k, gamma_qr, q_pos):
    # uses W^K_g of the wrong group order (groups reversed) -- a wrong index
    return _orig["absorb_query"](wl, q, q_rope, np.asarray(w_k)[::-1], gamma_q, gamma_k[::-1],
                                 gamma_qr, q_pos)


def _inv_rms_eps_outside(z, eps):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (np.sqrt(np.mean(z * z, axis=-1)) + eps)


def _inv_rms_sum_not_mean(z, eps):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / np.sqrt(np.sum(z * z, axis=-1) + eps)


def _rope_sign_error(x, pos, theta):
    y = _orig["rope"](x, pos, theta)
    x = np.asarray(x, dtype=np.float64)
    if theta == 0.0 or x.shape[-1] == 0:
        return y
    half = x.shape[-1] // 2
    # second half rotated the other way
    y2 = _orig["rope"](x, -np.asarray(pos), theta)
    return np.concatenate([y[..., :half], y2[..., half:]], axis=-1)


def _bf16_truncate(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _visible_off_by_one(T, s_q, i):
    return int(T) - s_q + i


def _split_len_unpaged(T, num_splits, page=64):
    return -(-int(T) // int(num_splits))


def _combine_unnormalised(o_part, lse_part):
    lse_part = np.asarray(lse_part, dtype=np.float64)
    M = np.max(lse_part, axis=-1, keepdims=True)
    w = np.exp(lse_part - M)
    lse = (M + np.log(np.sum(w, axis=-1, keepdims=True)))[..., 0]
    return np.sum(w[..., None] * np.asarray(o_part), axis=-2), lse


def _logits_without_alpha_k(wl, q_tilde, alpha_q, qr_hat, C, alpha_k, kr_hat, g):
    return _orig["absorbed_logits"](wl, q_tilde, alpha_q, qr_hat, C, np.ones_like(alpha_k), kr_hat, g)


def _logits_rope_sign(wl, q_tilde, alpha_q, qr_hat, C, alpha_k, kr_hat, g):
    return _orig["absorbed_logits"](wl, q_tilde, alpha_q, -np.asarray(qr_hat), C, alpha_k, kr_hat, g)


def _cache_image_wrong_slot(wl, inp, seq_ids, positions, rows, kv_init, ak_init):
    img = _orig["cache_image"](wl, inp, seq_ids, positions, rows, kv_init, ak_init)
    # slot t % 64 stored at (t + 32) % 64: the two halves of every page swapped
    kv = np.concatenate([img["kv"][:, 32:], img["kv"][:, :32]], axis=1)
    return {"kv": kv, "alpha_k": img["alpha_k"]}


def _explicit_unnormalised_key(wl, inp, b, i, heads=None):
    saved = O.rmsnorm

    def no_key_norm(z, gamma, eps):
        z = np.asarray(z, dtype=np.float64)
        if z.ndim == 2 and z.shape[-1] == wl.head_dim and z.shape[0] != wl.heads:
            return z * np.asarray(gamma, dtype=np.float64)
        return saved(z, gamma, eps)

    O.rmsnorm = no_key_norm
    try:
        return _orig["explicit_rows"](wl, inp, b, i, heads)
    finally:
        O.rmsnorm = saved


MUTATIONS = {
    "absorb drops gamma_k": ("absorb_query", _absorb_without_gamma_k,
                             [lambda: P.check_explicit_equals_absorbed("grouped")]),
    "absorb query position off by one": ("absorb_query", _absorb_shifted_position,
                                         [lambda: P.check_explicit_equals_absorbed("dsv3")]),
    "absorb uses another group's W^K": ("absorb_query", _absorb_transposed_w,
                                        [lambda: P.check_explicit_equals_absorbed("grouped")]),
    "eps outside the square root": ("inv_rms", _inv_rms_eps_outside,
                                    [P.check_rmsnorm_against_torch]),
    "sum instead of mean in RMS": ("inv_rms", _inv_rms_sum_not_mean,
                                   [P.check_rmsnorm_against_torch]),
    "RoPE half rotated backwards": ("rope", _rope_sign_error, [P.check_rope_properties]),
    "bf16 truncation instead of RNE": ("f32_to_bf16_bits", _bf16_truncate,
                                       [P.check_bf16_against_torch]),
    "causal window off by one": ("visible_count", _visible_off_by_one,
                                 [P.check_single_token, P.check_textbook_reduction]),
    "split length not whole pages": ("split_len", _split_len_unpaged, [P.check_split_bounds]),
    "combine weights not normalised": ("combine", _combine_unnormalised,
                                       [P.check_combine_closed_form, P.check_split_invariance]),
    "alpha^k dropped from the logits": ("absorbed_logits", _logits_without_alpha_k,
                                        [lambda: P.check_explicit_equals_absorbed("dsv3")]),
    "RoPE dot with the wrong sign": ("absorbed_logits", _logits_rope_sign,
                                     [lambda: P.check_explicit_equals_absorbed("dsv3")]),
    "cache slot index wrong": ("cache_image", _cache_image_wrong_slot,
                               [P.check_cache_image_layout]),
    "explicit path skips the key norm": ("explicit_rows", _explicit_unnormalised_key,
                                         [P.check_textbook_reduction,
                                          lambda: P.check_explicit_equals_absorbed("dsv3")]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    fn_name, bad, checks = MUTATIONS[name]
    monkeypatch.setattr(O, fn_name, bad)
    caught = []
    for chk in checks:
        try:
            chk()
        except Exception as e:  # noqa: BLE001 -- any failure means the pin noticed
            caught.append(type(e).__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"
