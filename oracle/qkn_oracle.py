"""CPU oracle for QK-Normed MLA absorbed-latent decode -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The HIP library never calls it, links it or reads anything
it writes; the two share no code.  Everything here is plain NumPy in float64,
written for a reader to check against the pages by eye, not for speed.

Sources (page title, then the section the step comes from):

* [QKN] "QK-Normed MLA: QK normalization without full key caching" -- the
  gist.science technical summary (sections "Planteamiento del Problema",
  "Metodologia" with its RMSNorm decomposition and its decode-logit equation,
  "Contribuciones Clave") and the arXiv abstract 2606.16310v1 on fugumt.com.
* [GQLA] "GQLA: Atencion Latente de Consulta por Grupos ..." -- gist.science
  technical summary, section 2 "Arquitectura", MQA-absorbed path (latent cache
  plus one shared RoPE key; up-projections indexed by KV group).

Notation: r latent rank, d content head dim, d_R RoPE dim, H query heads, G KV
groups, g(h) = h // (H/G), T sequence length counting the s_q new tokens,
query i sits at position T - s_q + i and sees the tokens t <= T - s_q + i.

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository):

* RMS(z) = sqrt(mean(z^2) + eps): eps inside the root, on the mean.
* one norm per head over d for q, one per (token, group) over d for k;
  gamma_q [d] shared by heads, gamma_k [G, d] per group.
* content and RoPE parts are normalised separately ([QKN] Metodologia item 4);
  the RoPE part is normalised first, then rotated (NeoX halves, theta = 10000).
  rope_theta == 0 disables the rotation.
* one RoPE key per token shared by every head and group ([GQLA] section 2).
* the value head dim equals d; values are not normalised.
* under a bf16 cache, alpha^k is taken from the stored (rounded) latent.
* storage rounding: the value is first rounded to float32 (the precision the
  HIP path computes in), then to bfloat16 with round-to-nearest-even.

Parity status: every function below is pinned by a test under tests/ that does
not re-derive it (identities, closed forms, library routines, invariants).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# storage rounding (an encoding, not part of the method)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    bfloat16 keeps the top 16 bits of the float32 pattern; the dropped half is
    rounded: add 0x7FFF plus the lowest kept bit, then truncate.  NaN stays NaN
    (quiet bit set)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    bits = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(x)
    if np.any(nan):
        bits[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return bits.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_value(x64, dtype: str) -> np.ndarray:
    """The value a device computing in float32 leaves in storage of ``dtype``."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32))
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float32)   # IEEE half, nearest-even
    raise ValueError(dtype)


def stored_bits(x64, dtype: str) -> np.ndarray:
    """Raw storage words: uint16 patterns for bf16 and f16 (IEEE half, nearest
    even), float32 for f32."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(x32)


# ----------------------------------------------------------------------------
# RMSNorm, decomposed as in [QKN] Metodologia: RMSNorm(z) = z * gamma / S(z)
# ----------------------------------------------------------------------------

def rms(z, eps: float) -> np.ndarray:
    """The dynamic scalar S(z) of the decomposition, one per vector (last axis)."""
    z = np.asarray(z, dtype=np.float64)
    return np.sqrt(np.mean(z * z, axis=-1) + eps)


def inv_rms(z, eps: float) -> np.ndarray:
    """alpha = 1 / S(z): the inverse-RMS scalar kept per token and group."""
    return 1.0 / rms(z, eps)


def rmsnorm(z, gamma, eps: float) -> np.ndarray:
    """RMSNorm(z) = z * gamma / S(z)."""
    z = np.asarray(z, dtype=np.float64)
    if z.shape[-1] == 0:
        return z.copy()
    return z * np.asarray(gamma, dtype=np.float64) * inv_rms(z, eps)[..., None]


# ----------------------------------------------------------------------------
# rotary position embedding of the RoPE block (a reading: NeoX halves)
# ----------------------------------------------------------------------------

def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate pairs (j, j + d_R/2) of ``x`` by angle pos * theta^(-2j/d_R)."""
    x = np.asarray(x, dtype=np.float64)
    if theta == 0.0 or x.shape[-1] == 0:
        return x.copy()
    dR = x.shape[-1]
    half = dR // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / dR)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# ----------------------------------------------------------------------------
# helpers on the workload layout
# ----------------------------------------------------------------------------

def group_of(h, heads: int, groups: int):
    return np.asarray(h) // (heads // groups)


def query_position(T: int, s_q: int, i: int) -> int:
    return int(T) - s_q + i


def visible_count(T: int, s_q: int, i: int) -> int:
    """Query i sees tokens 0 .. T - s_q + i (causal among the new tokens)."""
    return int(T) - s_q + i + 1


def _seq(inp, b):
    o = inp["tok_offsets"]
    return (np.asarray(inp["c"][o[b]:o[b + 1]], dtype=np.float64),
            np.asarray(inp["k_rope"][o[b]:o[b + 1]], dtype=np.float64))


def _softmax_stats(logits):
    """Row-wise max, sum of exp, probabilities and log-sum-exp (natural log)."""
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


# ----------------------------------------------------------------------------
# explicit path: materialise k = c W^K_g, then post-projection QK RMSNorm
# ([QKN] Planteamiento del Problema; this defines the result)
# ----------------------------------------------------------------------------

def explicit_rows(wl, inp, b: int, i: int, heads=None) -> dict:
    """Attention of query token i of sequence b for ``heads`` (default: all).

    Returns o [h, d] (values c W^V_g), o_lat [h, r] (sum_t p_t c_t), lse [h],
    p [h, n_visible]."""
    H, G = wl.heads, wl.groups
    heads = np.arange(H) if heads is None else np.asarray(heads)
    T = int(inp["seq_lens"][b])
    C, KR = _seq(inp, b)
    n_vis = visible_count(T, wl.s_q, i)
    C, KR = C[:n_vis], KR[:n_vis]
    q = np.asarray(inp["q"][b, i], dtype=np.float64)
    qr = np.asarray(inp["q_rope"][b, i], dtype=np.float64)
    q_hat = rmsnorm(q, inp["gamma_q"], wl.eps)                                   # [H, d]
    qr_hat = rope(rmsnorm(qr, inp["gamma_qr"], wl.eps),
                  query_position(T, wl.s_q, i), wl.rope_theta)                 # [H, d_R]
    kr_hat = rope(rmsnorm(KR, inp["gamma_kr"], wl.eps),
                  np.arange(n_vis), wl.rope_theta)                             # [t, d_R]
    out_o = np.zeros((len(heads), wl.head_dim))
    out_lat = np.zeros((len(heads), wl.rank))
    out_lse = np.zeros((len(heads),))
    out_p = np.zeros((len(heads), n_vis))
    g_of = group_of(heads, H, G)
    for g in range(G):
        sel = np.nonzero(g_of == g)[0]
        if len(sel) == 0:
            continue
        Wk = np.asarray(inp["w_k"][g], dtype=np.float64)                      # [r, d]
        Wv = np.asarray(inp["w_v"][g], dtype=np.float64)
        K = C @ Wk                                                            # k_{t,g}
        V = C @ Wv                                                            # v_{t,g}
        K_hat = rmsnorm(K, inp["gamma_k"][g], wl.eps)
        hs = heads[sel]
        logits = wl.softmax_scale * (q_hat[hs] @ K_hat.T + qr_hat[hs] @ kr_hat.T)
        p, lse = _softmax_stats(logits)
        out_o[sel] = p @ V
        out_lat[sel] = p @ C
        out_lse[sel] = lse
        out_p[sel] = p
    return {"o": out_o, "o_lat": out_lat, "lse": out_lse, "p": out_p}


# ----------------------------------------------------------------------------
# absorbed path ([QKN] Metodologia items 1-3 and the decode-logit equation)
# ----------------------------------------------------------------------------

def absorb_query(wl, q, q_rope, w_k, gamma_q, gamma_k, gamma_qr, q_pos) -> dict:
    """Step 1 of the method: fold gamma_q and gamma_k into the query and absorb
    W^K_g, giving q~ = (gamma_q * gamma_k,g * q) W^K_g^T in latent space;
    alpha^q = 1/RMS(q) per head; the RoPE query is RMS-normed on its own and
    rotated.  ``q`` [..., H, d], ``q_rope`` [..., H, d_R], ``q_pos`` [...]."""
    q = np.asarray(q, dtype=np.float64)
    H, G = wl.heads, wl.groups
    g_of = group_of(np.arange(H), H, G)
    q_tilde = np.zeros(q.shape[:-1] + (wl.rank,))
    for g in range(G):
        hs = np.nonzero(g_of == g)[0]
        folded = q[..., hs, :] * np.asarray(gamma_q, dtype=np.float64) \
            * np.asarray(gamma_k[g], dtype=np.float64)                           # [..., h, d]
        q_tilde[..., hs, :] = folded @ np.asarray(w_k[g], dtype=np.float64).T     # [..., h, r]
    alpha_q = inv_rms(q, wl.eps)
    qr_hat = rope(rmsnorm(q_rope, gamma_qr, wl.eps),
                  np.asarray(q_pos)[..., None], wl.rope_theta)
    return {"q_tilde": q_tilde, "alpha_q": alpha_q, "qr_hat": qr_hat}


def key_side(wl, C, KR, w_k, gamma_kr, positions) -> dict:
    """Step 2 and the RoPE block of step 4: alpha^k_{t,g} = 1/RMS(c_t W^K_g) for
    every group (the projected key is formed only to take its RMS), and the
    separately RMS-normed, rotated RoPE key of every token."""
    C = np.asarray(C, dtype=np.float64)
    G = wl.groups
    alpha_k = np.stack([inv_rms(C @ np.asarray(w_k[g], dtype=np.float64), wl.eps)
                        for g in range(G)], axis=-1)                             # [t, G]
    kr_hat = rope(rmsnorm(KR, gamma_kr, wl.eps), np.asarray(positions), wl.rope_theta)
    return {"alpha_k": alpha_k, "kr_hat": kr_hat}


def absorbed_logits(wl, q_tilde, alpha_q, qr_hat, C, alpha_k, kr_hat, g) -> np.ndarray:
    """The decode-logit equation with the RoPE dot added and the softmax scale
    applied: l_t = scale * ((q~ . c_t) * alpha^q * alpha^k_{t,g} + q^R . k^R_t).
    alpha^q varies along rows, alpha^k along columns (row-column scaling).
    ``alpha_k`` is [t, G]; ``g`` selects the group of these rows."""
    content = np.asarray(q_tilde) @ np.asarray(C).T                            # [h, t]
    content = content * np.asarray(alpha_q)[:, None] * np.asarray(alpha_k)[None, :, g]
    return wl.softmax_scale * (content + np.asarray(qr_hat) @ np.asarray(kr_hat).T)


def absorbed_rows(wl, inp, b: int, i: int, heads=None) -> dict:
    """Same outputs as :func:`explicit_rows`, through the absorbed formulation:
    the cache holds c_t, alpha^k and the normed RoPE key; o = (sum_t p_t c_t) W^V_g."""
    H, G = wl.heads, wl.groups
    heads = np.arange(H) if heads is None else np.asarray(heads)
    T = int(inp["seq_lens"][b])
    C, KR = _seq(inp, b)
    n_vis = visible_count(T, wl.s_q, i)
    C, KR = C[:n_vis], KR[:n_vis]
    qs = absorb_query(wl, inp["q"][b, i], inp["q_rope"][b, i], inp["w_k"], inp["gamma_q"],
                      inp["gamma_k"], inp["gamma_qr"], query_position(T, wl.s_q, i))
    ks = key_side(wl, C, KR, inp["w_k"], inp["gamma_kr"], np.arange(n_vis))
    out_o = np.zeros((len(heads), wl.head_dim))
    out_lat = np.zeros((len(heads), wl.rank))
    out_lse = np.zeros((len(heads),))
    g_of = group_of(heads, H, G)
    for g in range(G):
        sel = np.nonzero(g_of == g)[0]
        if len(sel) == 0:
            continue
        hs = heads[sel]
        logits = absorbed_logits(wl, qs["q_tilde"][hs], qs["alpha_q"][hs], qs["qr_hat"][hs],
                                 C, ks["alpha_k"], ks["kr_hat"], g)
        p, lse = _softmax_stats(logits)
        o_lat = p @ C
        out_lat[sel] = o_lat
        out_o[sel] = value_up_projection(wl, o_lat, inp["w_v"], hs)
        out_lse[sel] = lse
    return {"o": out_o, "o_lat": out_lat, "lse": out_lse}


# ----------------------------------------------------------------------------
# what the four library calls leave in memory (storage images)
# ----------------------------------------------------------------------------

def split_len(T: int, num_splits: int, page: int = 64) -> int:
    """Tokens per split-KV partition: ceil(T / P) rounded up to whole pages."""
    per = -(-int(T) // int(num_splits))
    return page * (-(-per // page))


def split_bounds(T: int, num_splits: int, page: int = 64):
    L = split_len(T, num_splits, page)
    return [(min(p * L, T), min((p + 1) * L, T)) for p in range(num_splits)]


def cache_image(wl, inp, seq_ids, positions, rows, kv_init, ak_init) -> dict:
    """Cache after appending the tokens ``rows`` of ``inp['c']``/``inp['k_rope']``
    belonging to sequences ``seq_ids`` at ``positions``.

    Slot of (b, t): page block_table[b][t // page], row t % page.  Each slot row
    holds [stored c_t (r) | stored normed RoPE key (d_R)]; the side cache holds
    alpha^k_{t,g} in float32 computed from the stored latent.  Slots not
    appended keep ``kv_init`` / ``ak_init``.  Returns raw storage words
    (``kv`` uint16 for bf16, float32 for f32) and ``alpha_k`` float32."""
    dt = wl.cache_dtype
    r, P = wl.rank, wl.page_size
    kv = np.array(kv_init, copy=True)
    ak = np.array(ak_init, copy=True)
    bt = inp["block_table"]
    c_rows = np.asarray(inp["c"][rows], dtype=np.float64)
    kr_rows = np.asarray(inp["k_rope"][rows], dtype=np.float64)
    c_store = stored_value(c_rows, dt).astype(np.float64)
    ks = key_side(wl, c_store, kr_rows, inp["w_k"], inp["gamma_kr"], positions)
    page = bt[np.asarray(seq_ids), np.asarray(positions) // P]
    slot = np.asarray(positions) % P
    kv[page, slot, :r] = stored_bits(c_rows, dt)
    kv[page, slot, r:] = stored_bits(ks["kr_hat"], dt)
    ak[page, slot, :] = ks["alpha_k"].astype(np.float32)
    return {"kv": kv, "alpha_k": ak}


def query_image(wl, inp) -> dict:
    """Outputs of query absorption for every (b, i, h), as stored: q~ and the
    normed RoPE query in the cache dtype, alpha^q in float32."""
    B, sq = wl.batch, wl.s_q
    pos = np.asarray(inp["seq_lens"], dtype=np.int64)[:, None] - sq + np.arange(sq)[None, :]
    qs = absorb_query(wl, inp["q"], inp["q_rope"], inp["w_k"], inp["gamma_q"],
                      inp["gamma_k"], inp["gamma_qr"], pos)
    return {"q_tilde": stored_bits(qs["q_tilde"], wl.cache_dtype),
            "alpha_q": qs["alpha_q"].astype(np.float32),
            "qr_hat": stored_bits(qs["qr_hat"], wl.cache_dtype)}


def words_to_f64(words, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(words).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(words, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(words, dtype=np.float64)


def decode_on_image(wl, q_img, kv, alpha_k, block_table, seq_lens, num_splits,
                    rows=None, use_alpha: bool = True) -> dict:
    """Split-KV decode over the stored state (the oracle of the decode call).

    For each query row (b, i, h) and split p, over the visible tokens of the
    split's range: l_t = scale * ((q~ . c_t) alpha^q alpha^k_{t,g} + q^R . k^R_t),
    o_p = sum_t softmax(l)_t c_t, lse_p = ln sum_t e^{l_t}; an empty split gives
    lse_p = -inf and o_p = 0.  ``rows`` optionally restricts to a list of
    (b, i, h).  ``use_alpha=False`` drops both inverse-RMS factors (plain
    absorbed MLA).  Returns partials and the combined result."""
    dt = wl.cache_dtype
    r, P, H, G, sq = wl.rank, wl.page_size, wl.heads, wl.groups, wl.s_q
    B = len(seq_lens)
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(sq) for h in range(H)]
    by_bi = {}
    for (b, i, h) in rows:
        by_bi.setdefault((b, i), []).append(h)
    qt = words_to_f64(q_img["q_tilde"], dt)
    qr = words_to_f64(q_img["qr_hat"], dt)
    aq = np.asarray(q_img["alpha_q"], dtype=np.float64)
    res = {}
    for (b, i), hs in by_bi.items():
        hs = np.asarray(hs)
        T = int(seq_lens[b])
        t = np.arange(T)
        page = block_table[b, t // P]
        slot = t % P
        C = words_to_f64(kv[page, slot, :r], dt)
        KR = words_to_f64(kv[page, slot, r:], dt)
        AK = np.asarray(alpha_k[page, slot, :], dtype=np.float64)               # [T, G]
        if not use_alpha:
            AK = np.ones_like(AK)
        n_vis = visible_count(T, sq, i)
        g_of = group_of(hs, H, G)
        o_part = np.zeros((len(hs), num_splits, r))
        lse_part = np.full((len(hs), num_splits), NEG_INF)
        for g in range(G):
            sel = np.nonzero(g_of == g)[0]
            if len(sel) == 0:
                continue
            a_q = aq[b, i, hs[sel]] if use_alpha else np.ones(len(sel))
            logits = absorbed_logits(wl, qt[b, i, hs[sel]], a_q, qr[b, i, hs[sel]],
                                     C, AK, KR, g)
            for p, (lo, hi) in enumerate(split_bounds(T, num_splits, P)):
                hi = min(hi, n_vis)
                if hi <= lo:
                    continue
                pr, lse = _softmax_stats(logits[:, lo:hi])
                o_part[sel, p] = pr @ C[lo:hi]
                lse_part[sel, p] = lse
        o_lat, lse = combine(o_part, lse_part)
        for k, h in enumerate(hs):
            res[(b, i, int(h))] = {"o_part": o_part[k], "lse_part": lse_part[k],
                                   "o_lat": o_lat[k], "lse": lse[k]}
    return res


def sparse_split_bounds(K: int, num_splits: int, stage: int = 32):
    """List entries per split of a sparse decode: ceil(K / P) rounded up to whole
    32-entry stages, as contiguous runs [lo, hi) of the K-entry list."""
    per = -(-int(K) // int(num_splits))
    L = stage * (-(-per // stage))
    return [(min(p * L, K), min((p + 1) * L, K)) for p in range(num_splits)]


def sparse_decode_on_image(wl, q_img, kv, alpha_k, block_table, seq_lens, indices,
                           num_splits, rows=None):
    """Selected-token decode over the stored state ([GQLA] section 2, "GQLA
    Disperso": fine-grained sparse attention kept on the MQA-absorbed path).

    Query token (b, i) attends only to the cache tokens listed in
    indices[b, i, :] (logical positions, shared by every head and group; -1
    marks an unused entry).  The logits are those of :func:`decode_on_image`
    for the listed tokens; the softmax runs over the listed tokens only, taken
    as listed (a position listed twice counts twice).  An entry that is not -1
    and falls outside the visible tokens 0 .. T - s_q + i, or whose page entry
    is out of range, is ignored and reported.  Split p covers the list entries
    sparse_split_bounds(K, P)[p]; a split with no valid entry gives lse_p =
    -inf and o_p = 0.  Returns (results per (b, i, h) as in decode_on_image,
    whether any entry was reported)."""
    dt = wl.cache_dtype
    r, P, H, G, sq = wl.rank, wl.page_size, wl.heads, wl.groups, wl.s_q
    indices = np.asarray(indices)
    B, _, K = indices.shape
    num_pages = kv.shape[0]
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(sq) for h in range(H)]
    by_bi = {}
    for (b, i, h) in rows:
        by_bi.setdefault((b, i), []).append(h)
    qt = words_to_f64(q_img["q_tilde"], dt)
    qr = words_to_f64(q_img["qr_hat"], dt)
    aq = np.asarray(q_img["alpha_q"], dtype=np.float64)
    err = False
    res = {}
    for (b, i), hs in by_bi.items():
        hs = np.asarray(hs)
        T = int(seq_lens[b])
        n_vis = visible_count(T, sq, i)
        g_of = group_of(hs, H, G)
        o_part = np.zeros((len(hs), num_splits, r))
        lse_part = np.full((len(hs), num_splits), NEG_INF)
        for p, (lo, hi) in enumerate(sparse_split_bounds(K, num_splits)):
            t = indices[b, i, lo:hi].astype(np.int64)
            used = t != -1
            vis = used & (t >= 0) & (t < n_vis)
            page = np.full(t.shape, -1, dtype=np.int64)
            page[vis] = block_table[b, t[vis] // P]
            ok = vis & (page >= 0) & (page < num_pages)
            err = err or bool(np.any(used & ~ok))
            if not np.any(ok):
                continue
            pg, sl = page[ok], t[ok] % P
            C = words_to_f64(kv[pg, sl, :r], dt)
            KR = words_to_f64(kv[pg, sl, r:], dt)
            AK = np.asarray(alpha_k[pg, sl, :], dtype=np.float64)
            for g in range(G):
                sel = np.nonzero(g_of == g)[0]
                if len(sel) == 0:
                    continue
                logits = absorbed_logits(wl, qt[b, i, hs[sel]], aq[b, i, hs[sel]],
                                         qr[b, i, hs[sel]], C, AK, KR, g)
                pr, lse = _softmax_stats(logits)
                o_part[sel, p] = pr @ C
                lse_part[sel, p] = lse
        o_lat, lse = combine(o_part, lse_part)
        for k, h in enumerate(hs):
            res[(b, i, int(h))] = {"o_part": o_part[k], "lse_part": lse_part[k],
                                   "o_lat": o_lat[k], "lse": lse[k]}
    return res, err


# ----------------------------------------------------------------------------
# chunked prefill on the explicit path ([QKN] Planteamiento del Problema: keys
# k = c W^K_g are materialised and RMS-normed after the projection; Metodologia
# item 4: the RoPE block is normed on its own).  A chunk of s_q new query
# tokens per sequence attends causally to the whole cache, the chunk included.
# ----------------------------------------------------------------------------

def prefill_dtype(wl) -> str:
    """Storage of the prefill's materialised q^, k^ and v: IEEE half with a bf16
    cache (the norm bounds |q^_j| by sqrt(d) |gamma_q,j| and |k^_j| likewise,
    and half keeps 3 more bits than bf16), float32 with a float32 cache."""
    return "f16" if wl.cache_dtype == "bf16" else "f32"


def prefill_query_image(wl, inp) -> dict:
    """The explicit path's query side as stored: q^ = gamma_q * q / RMS(q) per
    head (in :func:`prefill_dtype`), and the normed, rotated RoPE query in the
    cache dtype (as in :func:`query_image`)."""
    B, sq = wl.batch, wl.s_q
    pos = np.asarray(inp["seq_lens"], dtype=np.int64)[:, None] - sq + np.arange(sq)[None, :]
    q_hat = rmsnorm(inp["q"], inp["gamma_q"], wl.eps)
    qr_hat = rope(rmsnorm(inp["q_rope"], inp["gamma_qr"], wl.eps), pos[..., None], wl.rope_theta)
    return {"q_hat": stored_bits(q_hat, prefill_dtype(wl)),
            "qr_hat": stored_bits(qr_hat, wl.cache_dtype)}


def expand_image(wl, kv, alpha_k, block_table, seq_lens, w_k, w_v, gamma_k, max_T) -> dict:
    """Keys and values of the explicit path materialised from the stored cache.
    For token t < T_b of sequence b and group g, with c_t the stored latent:
    k^_{t,g} = gamma_k,g * (c_t W^K_g) * alpha^k_{t,g} (the stored inverse RMS of
    that same projection, so k^ = RMSNorm(c_t W^K_g)) and v_{t,g} = c_t W^V_g.
    Returns the exact float64 values and their storage words (in
    :func:`prefill_dtype`), [B, max_T, G, d]; rows t >= T_b are zero."""
    dt = wl.cache_dtype
    B, G, d, r, P = len(seq_lens), wl.groups, wl.head_dim, wl.rank, wl.page_size
    k_hat = np.zeros((B, max_T, G, d))
    v = np.zeros((B, max_T, G, d))
    for b in range(B):
        T = int(seq_lens[b])
        t = np.arange(T)
        page, sl = block_table[b, t // P], t % P
        C = words_to_f64(kv[page, sl, :r], dt)
        AK = np.asarray(alpha_k[page, sl, :], dtype=np.float64)
        for g in range(G):
            K = C @ np.asarray(w_k[g], dtype=np.float64)
            k_hat[b, :T, g] = K * np.asarray(gamma_k[g], dtype=np.float64)[None, :] * AK[:, g:g + 1]
            v[b, :T, g] = C @ np.asarray(w_v[g], dtype=np.float64)
    pd = prefill_dtype(wl)
    return {"k_hat": k_hat, "v": v, "k_hat_words": stored_bits(k_hat, pd),
            "v_words": stored_bits(v, pd)}


def prefill_on_images(wl, q_img, e_img, kv, block_table, seq_lens, rows=None) -> dict:
    """Attention of the explicit path over stored images: query token i of
    sequence b, head h (group g), over the keys t <= T_b - s_q + i:
    l_t = scale * (q^ . k^_{t,g} + q^R . k^R_t), p = softmax(l),
    o = sum_t p_t v_{t,g}, lse = ln sum_t e^{l_t}.  The inputs are the stored
    words of q^, q^R (query image), k^, v (expanded image) and k^R (cache).
    ``rows`` optionally restricts to a list of (b, i, h).  Returns
    {(b, i, h): {"o": [d], "lse": float}}."""
    dt = wl.cache_dtype
    r, P, H, G, sq = wl.rank, wl.page_size, wl.heads, wl.groups, wl.s_q
    B = len(seq_lens)
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(sq) for h in range(H)]
    by_bi = {}
    for (b, i, h) in rows:
        by_bi.setdefault((b, i), []).append(h)
    pd = prefill_dtype(wl)
    qh = words_to_f64(q_img["q_hat"], pd)
    qr = words_to_f64(q_img["qr_hat"], dt)
    kh = words_to_f64(e_img["k_hat_words"], pd)
    vv = words_to_f64(e_img["v_words"], pd)
    res = {}
    for (b, i), hs in by_bi.items():
        hs = np.asarray(hs)
        T = int(seq_lens[b])
        n = visible_count(T, sq, i)
        t = np.arange(n)
        KR = words_to_f64(kv[block_table[b, t // P], t % P, r:], dt)
        for h in hs:
            g = int(group_of(h, H, G))
            logits = wl.softmax_scale * (kh[b, :n, g] @ qh[b, i, h] + KR @ qr[b, i, h])
            pr, lse = _softmax_stats(logits[None, :])
            res[(b, i, int(h))] = {"o": (pr @ vv[b, :n, g])[0], "lse": float(lse[0])}
    return res


def gqa_row_len(wl) -> int:
    """Words per token of the GQA-path cache: every group's key and value (d
    each) and the one shared RoPE key (d_R)."""
    return 2 * wl.groups * wl.head_dim + wl.rope_dim


def gqa_cache_image(wl, inp, seq_ids, positions, rows, kvg_init) -> dict:
    """Cache of the GQA path ([GQLA] section 2: the latent expanded into g groups
    of keys and values, stored per group, plus the shared RoPE key) under
    QK-norm ([QKN] Planteamiento: the key is normed after its up-projection, so
    the stored key is the normed one).  For each appended token, with c_t its
    latent as the latent cache stores it (the reading alpha^k takes, so that
    both paths are functions of one stored latent):
      k^_{t,g} = gamma_k,g * k / RMS(k),  k = c_t W^K_g;   v_{t,g} = c_t W^V_g;
    the RoPE key as :func:`cache_image` stores it.  Row of slot
    (page, t % page): group g's key at [2dg, 2dg + d), its value at
    [2dg + d, 2d(g + 1)), in :func:`prefill_dtype`; the RoPE key at
    [2dG, 2dG + d_R) in the cache dtype.  Slots not appended keep ``kvg_init``.
    Returns {"kvg": words, "k_hat": [n, G, d], "v": [n, G, d]} (the exact
    values of the appended rows, float64)."""
    dt, pd = wl.cache_dtype, prefill_dtype(wl)
    G, d, P = wl.groups, wl.head_dim, wl.page_size
    kvg = np.array(kvg_init, copy=True)
    bt = inp["block_table"]
    c_store = stored_value(np.asarray(inp["c"][rows], dtype=np.float64), dt).astype(np.float64)
    kr_rows = np.asarray(inp["k_rope"][rows], dtype=np.float64)
    kr_hat = rope(rmsnorm(kr_rows, inp["gamma_kr"], wl.eps), np.asarray(positions), wl.rope_theta)
    page = bt[np.asarray(seq_ids), np.asarray(positions) // P]
    slot = np.asarray(positions) % P
    k_hat = np.zeros((len(c_store), G, d))
    v = np.zeros((len(c_store), G, d))
    for g in range(G):
        k_hat[:, g] = rmsnorm(c_store @ np.asarray(inp["w_k"][g], dtype=np.float64),
                              inp["gamma_k"][g], wl.eps)
        v[:, g] = c_store @ np.asarray(inp["w_v"][g], dtype=np.float64)
        kvg[page, slot, 2 * d * g:2 * d * g + d] = stored_bits(k_hat[:, g], pd)
        kvg[page, slot, 2 * d * g + d:2 * d * (g + 1)] = stored_bits(v[:, g], pd)
    kvg[page, slot, 2 * d * G:] = stored_bits(kr_hat, dt)
    return {"kvg": kvg, "k_hat": k_hat, "v": v}


def gqa_empty_image(wl, num_pages: int, fill_word=None) -> np.ndarray:
    """Initial (never written) GQA-path cache words, the sentinel of tests."""
    shape = (num_pages, wl.page_size, gqa_row_len(wl))
    if wl.cache_dtype == "bf16":
        return np.full(shape, 0x7E01 if fill_word is None else fill_word, dtype=np.uint16)
    return np.full(shape, np.nan if fill_word is None else fill_word, dtype=np.float32)


def gqa_full_image(wl, inp, kvg_init=None) -> dict:
    """GQA-path cache after appending every token of every sequence."""
    if kvg_init is None:
        kvg_init = gqa_empty_image(wl, inp["num_pages"])
    seq = np.repeat(np.arange(len(inp["seq_lens"]), dtype=np.int64), inp["seq_lens"])
    pos = np.concatenate([np.arange(int(T)) for T in inp["seq_lens"]])
    return gqa_cache_image(wl, inp, seq, pos, np.arange(len(seq)), kvg_init)


def gqa_decode_on_image(wl, q_img, kvg, block_table, seq_lens, num_splits, rows=None) -> dict:
    """Split-KV decode of the GQA path over its stored cache: standard grouped
    attention with no latent expansion per step ([GQLA] section 2).  For query
    row (b, i, h) of group g and split p (the decode's whole-page split rule),
    over the visible tokens of the split:
      l_t = scale * (q^ . k^_{t,g} + q^R . k^R_t),
      o_p = sum_t softmax(l)_t v_{t,g},  lse_p = ln sum_t e^{l_t};
    an empty split gives lse_p = -inf, o_p = 0.  q^, q^R are the stored words of
    :func:`prefill_query_image`.  Returns partials and the combined result per
    (b, i, h)."""
    dt, pd = wl.cache_dtype, prefill_dtype(wl)
    P, H, G, sq, d = wl.page_size, wl.heads, wl.groups, wl.s_q, wl.head_dim
    B = len(seq_lens)
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(sq) for h in range(H)]
    by_bi = {}
    for (b, i, h) in rows:
        by_bi.setdefault((b, i), []).append(h)
    qh = words_to_f64(q_img["q_hat"], pd)
    qr = words_to_f64(q_img["qr_hat"], dt)
    res = {}
    for (b, i), hs in by_bi.items():
        T = int(seq_lens[b])
        t = np.arange(T)
        page, slot = block_table[b, t // P], t % P
        KR = words_to_f64(kvg[page, slot, 2 * d * G:], dt)
        n_vis = visible_count(T, sq, i)
        for h in hs:
            g = int(group_of(h, H, G))
            K = words_to_f64(kvg[page, slot, 2 * d * g:2 * d * g + d], pd)
            V = words_to_f64(kvg[page, slot, 2 * d * g + d:2 * d * (g + 1)], pd)
            logits = wl.softmax_scale * (K @ qh[b, i, h] + KR @ qr[b, i, h])
            o_part = np.zeros((num_splits, d))
            lse_part = np.full(num_splits, NEG_INF)
            for p, (lo, hi) in enumerate(split_bounds(T, num_splits, P)):
                hi = min(hi, n_vis)
                if hi <= lo:
                    continue
                pr, lse = _softmax_stats(logits[None, lo:hi])
                o_part[p] = (pr @ V[lo:hi])[0]
                lse_part[p] = lse[0]
            o, lse = combine(o_part, lse_part)
            res[(b, i, int(h))] = {"o_part": o_part, "lse_part": lse_part, "o": o, "lse": float(lse)}
    return res


def combine(o_part, lse_part):
    """Merge split partials ([..., P, r], [..., P]) by log-sum-exp weights:
    M = max_p lse_p, lse = M + ln sum_p e^{lse_p - M}, o = sum_p e^{lse_p - lse} o_p.
    Empty splits (lse_p = -inf) get weight 0; when every split is empty (a
    sparse decode whose list holds no valid entry) the result is the empty
    sum: o = 0, lse = -inf."""
    lse_part = np.asarray(lse_part, dtype=np.float64)
    o_part = np.asarray(o_part, dtype=np.float64)
    M = np.max(lse_part, axis=-1, keepdims=True)
    empty = np.isneginf(M)
    M = np.where(empty, 0.0, M)
    w = np.exp(lse_part - M)
    s = np.sum(w, axis=-1, keepdims=True)
    s1 = np.where(empty, 1.0, s)
    lse = np.where(empty, NEG_INF, M + np.log(s1))[..., 0]
    o = np.sum((w / s1)[..., None] * o_part, axis=-2)
    return o, lse


def value_up_projection(wl, o_lat, w_v, heads) -> np.ndarray:
    """o = o^lat W^V_g for each head (the value side of the absorbed path)."""
    g_of = group_of(np.asarray(heads), wl.heads, wl.groups)
    return np.stack([np.asarray(o_lat[k], dtype=np.float64) @ np.asarray(w_v[g], dtype=np.float64)
                     for k, g in enumerate(g_of)])


def empty_images(wl, num_pages: int, kv_fill_word=None, ak_fill=np.nan) -> tuple:
    """Initial (never written) cache words, used as the sentinel in tests."""
    shape = (num_pages, wl.page_size, wl.rank + wl.rope_dim)
    if wl.cache_dtype == "bf16":
        kv = np.full(shape, 0x7FC1 if kv_fill_word is None else kv_fill_word, dtype=np.uint16)
    else:
        kv = np.full(shape, np.nan if kv_fill_word is None else kv_fill_word, dtype=np.float32)
    ak = np.full((num_pages, wl.page_size, wl.groups), ak_fill, dtype=np.float32)
    return kv, ak


def full_cache_image(wl, inp, kv_init=None, ak_init=None) -> dict:
    """Cache image after appending every token of every sequence."""
    if kv_init is None:
        kv_init, ak_init = empty_images(wl, inp["num_pages"])
    seq = np.repeat(np.arange(len(inp["seq_lens"]), dtype=np.int64), inp["seq_lens"])
    pos = np.concatenate([np.arange(int(T)) for T in inp["seq_lens"]])
    rows = np.arange(len(seq))
    return cache_image(wl, inp, seq, pos, rows, kv_init, ak_init)
