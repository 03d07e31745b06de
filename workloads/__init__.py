"""Seeded synthetic workloads for QK-Normed MLA absorbed-latent decode.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no normalisation, no projection, no softmax, no rounding to
a storage dtype).  Both the CPU oracle (tests) and the HIP path (tests, bench)
take their inputs from here, so the two sides see identical bytes.

Shapes and distributions follow the five decode workloads this project is
measured on:

* ``tiny``     B=1, s_q=1, 8 heads, 1 KV group, r=64, d=32, d_R=16, T=256, fp32 cache
* ``dsv3``     B=32, s_q=1, 128 heads, 1 group, r=512, d=128, d_R=64, T=4096, bf16 cache
* ``grouped``  B=8, s_q=1, 128 heads, 4 groups (32 heads each), r=512, d=128, d_R=64, T=32768
* ``long``     B=1, s_q=1, 128 heads, 1 group, r=512, T=262144, split-KV, log-normal sigma 1.0
* ``mtp``      B=64, s_q=4 causal, 128 heads, 1 group, r=512, T_b ~ U{1024..16384},
               64-token pages in a shuffled block table

Latents are ``c_t = s_t * N(0, I)`` with a per-token log-normal scale
``s_t = exp(sigma * N(0, 1))``; ``W^K, W^V ~ N(0, 1/r)``; every norm weight is
``1 + 0.1 * N(0, 1)``; queries and raw RoPE keys are ``N(0, 1)``.  The content
head dim of the last four workloads is taken as 128 (DeepSeek-V3 shaped), so the
softmax scale is ``1/sqrt(128 + 64)``; the tiny one uses ``1/sqrt(32 + 16)``.

Draw order (numpy ``default_rng(seed)``, PCG64): W^K, W^V, gamma_q, gamma_k,
gamma_qR, gamma_kR, sequence lengths, then per sequence (s_t, c, k^R), then q,
q^R, then the page permutation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAGE_SIZE = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    s_q: int
    heads: int
    groups: int
    rank: int          # latent rank r
    head_dim: int      # content head dim d (value head dim is the same)
    rope_dim: int      # d_R
    seq_len: int       # fixed T_b (used when seq_len_range is None)
    cache_dtype: str   # "f32" or "bf16"
    latent_log_sigma: float
    num_splits: int
    seq_len_range: Optional[tuple] = None   # inclusive (lo, hi) for ragged batches
    shuffled_pages: bool = False
    eps: float = 1e-6
    rope_theta: float = 10000.0
    page_size: int = PAGE_SIZE

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim + self.rope_dim)

    @property
    def max_seq_len(self) -> int:
        return self.seq_len if self.seq_len_range is None else self.seq_len_range[1]

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.max_seq_len // self.page_size)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", batch=1, s_q=1, heads=8, groups=1, rank=64, head_dim=32,
                     rope_dim=16, seq_len=256, cache_dtype="f32", latent_log_sigma=0.5,
                     num_splits=1),
    "dsv3": Workload("dsv3", batch=32, s_q=1, heads=128, groups=1, rank=512, head_dim=128,
                     rope_dim=64, seq_len=4096, cache_dtype="bf16", latent_log_sigma=0.5,
                     num_splits=8),
    "grouped": Workload("grouped", batch=8, s_q=1, heads=128, groups=4, rank=512,
                        head_dim=128, rope_dim=64, seq_len=32768, cache_dtype="bf16",
                        latent_log_sigma=0.5, num_splits=32),
    "long": Workload("long", batch=1, s_q=1, heads=128, groups=1, rank=512, head_dim=128,
                     rope_dim=64, seq_len=262144, cache_dtype="bf16", latent_log_sigma=1.0,
                     num_splits=256),
    "mtp": Workload("mtp", batch=64, s_q=4, heads=128, groups=1, rank=512, head_dim=128,
                    rope_dim=64, seq_len=16384, seq_len_range=(1024, 16384),
                    cache_dtype="bf16", latent_log_sigma=0.5, num_splits=4,
                    shuffled_pages=True),
    # selected-token decode: 2048 listed tokens per query out of 16384
    "sparse": Workload("sparse", batch=32, s_q=1, heads=128, groups=1, rank=512, head_dim=128,
                       rope_dim=64, seq_len=16384, cache_dtype="bf16", latent_log_sigma=0.5,
                       num_splits=2, shuffled_pages=True),
    # chunked prefill on the explicit path: a 512-token chunk per sequence
    "prefill": Workload("prefill", batch=2, s_q=512, heads=128, groups=1, rank=512, head_dim=128,
                        rope_dim=64, seq_len=8192, cache_dtype="bf16", latent_log_sigma=0.5,
                        num_splits=1),
}

# entries per query list of the selected-token workload
SPARSE_LIST_LEN = 2048

# Order in which the workloads are listed by the project (index 0 is the tiny
# correctness case).
WORKLOAD_ORDER = ["tiny", "dsv3", "grouped", "long", "mtp"]


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _norm_weight(rng, shape):
    return (np.float32(1.0) + np.float32(0.1) * rng.standard_normal(shape, dtype=np.float32))


def make_inputs(wl: Workload, seed: int = 0, *, extra_pages: int = 0) -> dict:
    """Draw every input of one decode step of ``wl``.

    Returns a dict of numpy arrays (all float32 / int32):

    ``w_k, w_v`` [G, r, d]; ``gamma_q`` [d]; ``gamma_k`` [G, d]; ``gamma_qr``,
    ``gamma_kr`` [d_R]; ``seq_lens`` [B] (T_b, counting the s_q new tokens);
    ``c`` [N, r] and ``k_rope`` [N, d_R] for all N = sum(T_b) tokens, sequence
    after sequence, token position ascending; ``tok_offsets`` [B+1];
    ``q`` [B, s_q, H, d]; ``q_rope`` [B, s_q, H, d_R]; ``block_table``
    [B, max_pages_per_seq] (unused entries are -1); ``num_pages``.
    """
    rng = np.random.default_rng(seed)
    G, r, d, dR, H = wl.groups, wl.rank, wl.head_dim, wl.rope_dim, wl.heads
    B, sq = wl.batch, wl.s_q
    out = {}
    out["w_k"] = _normal(rng, (G, r, d), 1.0 / math.sqrt(r))
    out["w_v"] = _normal(rng, (G, r, d), 1.0 / math.sqrt(r))
    out["gamma_q"] = _norm_weight(rng, (d,))
    out["gamma_k"] = _norm_weight(rng, (G, d))
    out["gamma_qr"] = _norm_weight(rng, (dR,))
    out["gamma_kr"] = _norm_weight(rng, (dR,))
    if wl.seq_len_range is None:
        seq_lens = np.full((B,), wl.seq_len, dtype=np.int32)
    else:
        lo, hi = wl.seq_len_range
        seq_lens = rng.integers(lo, hi + 1, size=(B,), dtype=np.int64).astype(np.int32)
    if np.any(seq_lens < sq):
        raise ValueError("every sequence must hold at least the s_q new tokens")
    out["seq_lens"] = seq_lens
    n_tok = int(seq_lens.sum())
    offs = np.zeros((B + 1,), dtype=np.int64)
    offs[1:] = np.cumsum(seq_lens)
    out["tok_offsets"] = offs
    c = np.empty((n_tok, r), dtype=np.float32)
    kr = np.empty((n_tok, dR), dtype=np.float32)
    for b in range(B):
        T = int(seq_lens[b])
        s = np.exp(np.float32(wl.latent_log_sigma) * rng.standard_normal((T,), dtype=np.float32))
        blk = rng.standard_normal((T, r), dtype=np.float32)
        blk *= s[:, None]
        c[offs[b]:offs[b + 1]] = blk
        kr[offs[b]:offs[b + 1]] = rng.standard_normal((T, dR), dtype=np.float32)
    out["c"] = c
    out["k_rope"] = kr
    out["q"] = _normal(rng, (B, sq, H, d))
    out["q_rope"] = _normal(rng, (B, sq, H, dR))
    P = wl.page_size
    pages_per_seq = (seq_lens.astype(np.int64) + P - 1) // P
    num_pages = int(pages_per_seq.sum()) + extra_pages
    order = np.arange(num_pages, dtype=np.int64)
    if wl.shuffled_pages:
        order = rng.permutation(num_pages)
    bt = np.full((B, wl.max_pages_per_seq), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        for j in range(int(pages_per_seq[b])):
            bt[b, j] = order[k]
            k += 1
    out["block_table"] = bt
    out["num_pages"] = num_pages
    return out


def make_selection(wl: Workload, seq_lens, list_len: int, seed: int, fill: float = 1.0,
                   shuffle: bool = True) -> np.ndarray:
    """Token lists for a selected-token decode: int32 [B, s_q, list_len].  For
    query token i of sequence b, min(visible, round(fill * list_len)) distinct
    positions drawn uniformly from its visible tokens 0 .. T_b - s_q + i, in
    random entries of the list (shuffle) or in order at its start; every
    other entry is -1."""
    rng = np.random.default_rng(seed)
    B, sq = len(seq_lens), wl.s_q
    out = np.full((B, sq, list_len), -1, dtype=np.int32)
    for b in range(B):
        for i in range(sq):
            vis = int(seq_lens[b]) - sq + i + 1
            m = min(vis, int(round(fill * list_len)))
            pos = np.sort(rng.choice(vis, size=m, replace=False)).astype(np.int32)
            if shuffle:
                slots = np.sort(rng.choice(list_len, size=m, replace=False))
                out[b, i, slots] = rng.permutation(pos)
            else:
                out[b, i, :m] = pos
    return out


def permute_pages(inputs: dict, seed: int) -> dict:
    """Same logical cache, different physical page placement (fresh permutation)."""
    rng = np.random.default_rng(seed)
    bt = inputs["block_table"]
    perm = rng.permutation(inputs["num_pages"]).astype(np.int32)
    new = dict(inputs)
    nbt = bt.copy()
    mask = bt >= 0
    nbt[mask] = perm[bt[mask]]
    new["block_table"] = nbt
    return new


def new_token_index(inputs: dict, s_q: int):
    """Flat indices, sequence ids and positions of the s_q newest tokens of every
    sequence (the tokens one decode step appends)."""
    seq_lens = inputs["seq_lens"]
    offs = inputs["tok_offsets"]
    idx, seq, pos = [], [], []
    for b, T in enumerate(seq_lens):
        for i in range(s_q):
            t = int(T) - s_q + i
            idx.append(int(offs[b]) + t)
            seq.append(b)
            pos.append(t)
    return (np.asarray(idx, dtype=np.int64), np.asarray(seq, dtype=np.int32),
            np.asarray(pos, dtype=np.int32))


def all_token_index(inputs: dict):
    """Sequence ids and positions of every token (a full cache fill)."""
    seq_lens = inputs["seq_lens"]
    seq = np.repeat(np.arange(len(seq_lens), dtype=np.int32), seq_lens)
    pos = np.concatenate([np.arange(int(T), dtype=np.int32) for T in seq_lens])
    return seq, pos


def flops_and_bytes(wl: Workload, seq_lens, cache_elem_bytes: int = 2):
    """Algorithmic work of one decode (+combine) over the cache.

    Bytes: every visible token's latent and RoPE key once, plus its G fp32
    inverse-RMS scalars.  FLOPs: per token and query row, the content dot
    (2r), the RoPE dot (2 d_R) and the value accumulation (2r).
    """
    T = np.asarray(seq_lens, dtype=np.int64)
    per_tok_bytes = cache_elem_bytes * (wl.rank + wl.rope_dim) + 4 * wl.groups
    nbytes = int(T.sum()) * per_tok_bytes
    # query i of a sequence of length T sees T - s_q + i + 1 tokens
    visible = int(T.sum()) * wl.s_q - len(T) * (wl.s_q * (wl.s_q - 1) // 2)
    flops = visible * wl.heads * (4 * wl.rank + 2 * wl.rope_dim)
    return flops, nbytes
