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


def _rope_wrong_ladder(x, pos, theta):
    # frequencies theta^(-j/d_R) instead of theta^(-2j/d_R): the first pair is
    # still right, every other pair turns too fast
    x = np.asarray(x, dtype=np.float64)
    if theta == 0.0 or x.shape[-1] == 0:
        return x.copy()
    dR = x.shape[-1]
    half = dR // 2
    inv_freq = float(theta) ** (-np.arange(half, dtype=np.float64) / dR)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * np.cos(ang) - x2 * np.sin(ang),
                           x2 * np.cos(ang) + x1 * np.sin(ang)], axis=-1)


def _value_projection_group0(wl, o_lat, w_v, heads):
    # every head takes group 0's W^V
    return np.stack([np.asarray(o_lat[k], dtype=np.float64) @ np.asarray(w_v[0], dtype=np.float64)
                     for k in range(len(heads))])


def _value_projection_wrong_group_map(wl, o_lat, w_v, heads):
    # heads dealt to groups round-robin (h mod G) instead of in blocks
    return np.stack([np.asarray(o_lat[k], dtype=np.float64)
                     @ np.asarray(w_v[int(h) % wl.groups], dtype=np.float64)
                     for k, h in enumerate(heads)])


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


def _sparse_padding_as_token0(wl, q_img, kv, alpha_k, block_table, seq_lens, indices,
                              num_splits, rows=None):
    # the -1 marker read as position 0 instead of an unused entry
    idx = np.where(np.asarray(indices) == -1, 0, indices)
    return _orig["sparse_decode_on_image"](wl, q_img, kv, alpha_k, block_table, seq_lens, idx,
                                           num_splits, rows)


def _sparse_positions_off_by_one(wl, q_img, kv, alpha_k, block_table, seq_lens, indices,
                                 num_splits, rows=None):
    idx = np.asarray(indices).copy()
    idx[idx >= 0] += 1
    return _orig["sparse_decode_on_image"](wl, q_img, kv, alpha_k, block_table, seq_lens, idx,
                                           num_splits, rows)


def _sparse_bounds_unstaged(K, num_splits, stage=32):
    return _orig["sparse_split_bounds"](K, num_splits, 1)


def _expand_values_with_w_k(wl, kv, alpha_k, block_table, seq_lens, w_k, w_v, gamma_k, max_T):
    return _orig["expand_image"](wl, kv, alpha_k, block_table, seq_lens, w_k, w_k, gamma_k, max_T)


def _expand_without_gamma_k(wl, kv, alpha_k, block_table, seq_lens, w_k, w_v, gamma_k, max_T):
    return _orig["expand_image"](wl, kv, alpha_k, block_table, seq_lens, w_k, w_v,
                                 np.ones_like(gamma_k), max_T)


def _prefill_window_one_longer(wl, q_img, e_img, kv, block_table, seq_lens, rows=None):
    # every query sees one token past its causal end
    return _orig["prefill_on_images"](wl, q_img, e_img, kv, block_table,
                                      np.asarray(seq_lens) + 1, rows)


def _gqa_values_with_w_k(wl, inp, seq_ids, positions, rows, kvg_init):
    return _orig["gqa_cache_image"](wl, dict(inp, w_v=inp["w_k"]), seq_ids, positions, rows, kvg_init)


def _gqa_keys_not_normed(wl, inp, seq_ids, positions, rows, kvg_init):
    # the key stored as gamma_k * (c W^K_g), the RMS division forgotten
    out = _orig["gqa_cache_image"](wl, inp, seq_ids, positions, rows, kvg_init)
    d, P = wl.head_dim, wl.page_size
    c = O.stored_value(np.asarray(inp["c"][rows], dtype=np.float64), wl.cache_dtype).astype(np.float64)
    page = inp["block_table"][np.asarray(seq_ids), np.asarray(positions) // P]
    slot = np.asarray(positions) % P
    for g in range(wl.groups):
        k = (c @ np.asarray(inp["w_k"][g], dtype=np.float64)) * np.asarray(inp["gamma_k"][g])
        out["kvg"][page, slot, 2 * d * g:2 * d * g + d] = O.stored_bits(k, O.prefill_dtype(wl))
    return out


def _gqa_rope_key_of_next_slot(wl, inp, seq_ids, positions, rows, kvg_init):
    out = _orig["gqa_cache_image"](wl, inp, seq_ids, positions, rows, kvg_init)
    off = 2 * wl.groups * wl.head_dim
    out["kvg"][:, :, off:] = np.roll(out["kvg"][:, :, off:], 1, axis=1)
    return out


def _gqa_decode_groups_swapped(wl, q_img, kvg, block_table, seq_lens, num_splits, rows=None):
    # heads of group 0 read group 1's keys and values and the reverse
    d = wl.head_dim
    kvg = np.array(kvg, copy=True)
    if wl.groups > 1:
        g0 = kvg[:, :, 0:2 * d].copy()
        kvg[:, :, 0:2 * d] = kvg[:, :, 2 * d:4 * d]
        kvg[:, :, 2 * d:4 * d] = g0
    return _orig["gqa_decode_on_image"](wl, q_img, kvg, block_table, seq_lens, num_splits, rows)


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
    "RoPE frequency ladder theta^(-j/d_R)": ("rope", _rope_wrong_ladder,
                                             [P.check_rope_frequency_ladder]),
    "value projection uses group 0's W^V": ("value_up_projection", _value_projection_group0,
                                            [lambda: P.check_value_up_projection("grouped")]),
    "value projection maps heads to groups round-robin": (
        "value_up_projection", _value_projection_wrong_group_map,
        [lambda: P.check_value_up_projection("grouped")]),
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
    "sparse -1 marker read as position 0": ("sparse_decode_on_image", _sparse_padding_as_token0,
                                            [P.check_sparse_subset_against_explicit,
                                             P.check_sparse_invalid_entries]),
    "sparse positions off by one": ("sparse_decode_on_image", _sparse_positions_off_by_one,
                                    [P.check_sparse_subset_against_explicit]),
    "sparse splits not whole stages": ("sparse_split_bounds", _sparse_bounds_unstaged,
                                       [P.check_sparse_split_bounds]),
    "prefill values projected with W^K": ("expand_image", _expand_values_with_w_k,
                                          [P.check_prefill_matches_explicit_f32]),
    "prefill keys without gamma_k": ("expand_image", _expand_without_gamma_k,
                                     [P.check_expanded_keys_unit_rms,
                                      P.check_prefill_matches_explicit_f32]),
    "prefill causal window one token long": ("prefill_on_images", _prefill_window_one_longer,
                                             [P.check_prefill_matches_explicit_f32]),
    "GQA values projected with W^K": ("gqa_cache_image", _gqa_values_with_w_k,
                                      [P.check_gqa_image_against_torch,
                                       P.check_gqa_matches_explicit_f32]),
    "GQA keys stored without the norm": ("gqa_cache_image", _gqa_keys_not_normed,
                                         [P.check_gqa_image_against_torch,
                                          P.check_gqa_matches_explicit_f32]),
    "GQA RoPE key of the neighbouring slot": ("gqa_cache_image", _gqa_rope_key_of_next_slot,
                                              [P.check_gqa_image_against_torch,
                                               P.check_gqa_matches_explicit_f32]),
    "GQA decode swaps two groups": ("gqa_decode_on_image", _gqa_decode_groups_swapped,
                                    [P.check_gqa_matches_explicit_f32,
                                     P.check_gqa_equals_absorbed_f32]),
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
