"""Device buffers and call sequence of one QK-Normed MLA decode step.

``DecodeRunner`` uploads a workload's inputs (as drawn by ``workloads``), owns
the paged cache, the alpha^k side cache, the query-side outputs and the split
partials, and issues the four library calls of a step in order:

    absorb_query -> append (the s_q new tokens) -> decode -> combine

torch is used for allocation and copies only; all arithmetic is in the HIP
kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import (QKN_BF16, PAGE_SIZE, Dims, alloc_decode_workspace, cache_torch_dtype, dims_for,
               partial_torch_dtype, qkn_mla_absorb_query, qkn_mla_append, qkn_mla_combine,
               qkn_mla_combine_project, qkn_mla_decode, qkn_mla_decode_attend,
               gqa_row_words, gqa_workspace_bytes, qkn_mla_gqa_append, qkn_mla_gqa_attend,
               qkn_mla_prefill_attend, qkn_mla_prefill_expand, qkn_mla_prefill_query)


def _dev(x, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class DecodeRunner:
    def __init__(self, wl, inputs: dict, device="cuda", num_splits: Optional[int] = None,
                 kv_fill_word: Optional[int] = None, alpha_fill: float = float("nan"),
                 upload_all_tokens: bool = True):
        self.wl = wl
        self.inp = inputs
        self.device = torch.device(device)
        self.num_pages = int(inputs["num_pages"])
        self.dims: Dims = dims_for(wl, self.num_pages)
        self.num_splits = int(num_splits if num_splits is not None else wl.num_splits)
        d, dev = self.dims, self.device
        self.cache_dtype = cache_torch_dtype(d)
        B, sq, H = wl.batch, wl.s_q, wl.heads
        f32 = torch.float32
        self.w_k = _dev(inputs["w_k"], dev)
        self.w_v = _dev(inputs["w_v"], dev)
        self.gamma_q = _dev(inputs["gamma_q"], dev)
        self.gamma_k = _dev(inputs["gamma_k"], dev)
        self.gamma_qr = _dev(inputs["gamma_qr"], dev)
        self.gamma_kr = _dev(inputs["gamma_kr"], dev)
        self.block_table = _dev(inputs["block_table"], dev)
        self.seq_lens = _dev(inputs["seq_lens"], dev)
        self.q = _dev(inputs["q"], dev)
        self.q_rope = _dev(inputs["q_rope"], dev)
        seq = np.asarray(inputs["seq_lens"], dtype=np.int64)
        self.q_pos = _dev((seq[:, None] - sq + np.arange(sq)[None, :]).astype(np.int32), dev)
        # tokens: every token (for the cache fill) and the s_q new ones of each sequence
        offs = np.asarray(inputs["tok_offsets"])
        all_seq = np.repeat(np.arange(B, dtype=np.int32), seq)
        all_pos = np.concatenate([np.arange(int(T), dtype=np.int32) for T in seq])
        is_new = np.zeros(len(all_seq), dtype=bool)
        for b in range(B):
            is_new[offs[b + 1] - sq: offs[b + 1]] = True
        self._old_rows = np.nonzero(~is_new)[0]
        self._new_rows = np.nonzero(is_new)[0]
        self.new_seq = _dev(all_seq[self._new_rows], dev)
        self.new_pos = _dev(all_pos[self._new_rows], dev)
        self.c_new = _dev(inputs["c"][self._new_rows], dev)
        self.kr_new = _dev(inputs["k_rope"][self._new_rows], dev)
        self._all_seq, self._all_pos = all_seq, all_pos
        # cache
        row = wl.rank + wl.rope_dim
        self.kv = torch.empty((self.num_pages, PAGE_SIZE, row), dtype=self.cache_dtype, device=dev)
        if kv_fill_word is not None:
            if d.cache_dtype == QKN_BF16:
                self.kv.view(torch.int16).fill_(np.int16(np.uint16(kv_fill_word).view(np.int16)))
            else:
                self.kv.fill_(float(kv_fill_word))
        else:
            self.kv.zero_()
        self.alpha_k = torch.full((self.num_pages, PAGE_SIZE, wl.groups), alpha_fill, dtype=f32,
                                  device=dev)
        # query side and outputs
        self.q_tilde = torch.empty((B, sq, H, wl.rank), dtype=self.cache_dtype, device=dev)
        self.alpha_q = torch.empty((B, sq, H), dtype=f32, device=dev)
        self.q_rope_normed = torch.empty((B, sq, H, wl.rope_dim), dtype=self.cache_dtype,
                                         device=dev)
        self.alloc_partials(self.num_splits)
        self.o_latent = torch.empty((B, sq, H, wl.rank), dtype=f32, device=dev)
        self.lse = torch.empty((B, sq, H), dtype=f32, device=dev)
        self.o = torch.empty((B, sq, H, wl.head_dim), dtype=f32, device=dev)
        self.err_flag = torch.zeros((1,), dtype=torch.int32, device=dev)

    def alloc_partials(self, num_splits: int):
        wl = self.wl
        self.num_splits = int(num_splits)
        shape = (wl.batch, wl.s_q, wl.heads, self.num_splits)
        self.o_partial = torch.empty(shape + (wl.rank,), dtype=partial_torch_dtype(self.dims),
                                     device=self.device)
        self.lse_partial = torch.empty(shape, dtype=torch.float32, device=self.device)

    # -- the four calls ------------------------------------------------------
    def absorb(self, stream=None):
        qkn_mla_absorb_query(self.dims, self.q, self.q_rope, self.q_pos, self.w_k, self.gamma_q,
                             self.gamma_k, self.gamma_qr, self.q_tilde, self.alpha_q,
                             self.q_rope_normed, stream)

    def append_rows(self, rows, chunk: int = 1 << 18, stream=None):
        """Append the tokens ``rows`` (indices into the workload's token list)."""
        rows = np.asarray(rows)
        for s in range(0, len(rows), chunk):
            r = rows[s:s + chunk]
            seq = _dev(self._all_seq[r], self.device)
            pos = _dev(self._all_pos[r], self.device)
            c = _dev(self.inp["c"][r], self.device)
            kr = _dev(self.inp["k_rope"][r], self.device)
            qkn_mla_append(self.dims, c, kr, seq, pos, self.block_table, self.w_k, self.gamma_kr,
                           self.kv, self.alpha_k, self.err_flag, stream)

    def history_inputs(self, limit: int = 1 << 18):
        """Device copies of the first ``limit`` history tokens' append inputs
        (latent, RoPE key, sequence, position)."""
        r = np.asarray(self._old_rows)[:limit]
        return (_dev(self.inp["c"][r], self.device), _dev(self.inp["k_rope"][r], self.device),
                _dev(self._all_seq[r], self.device), _dev(self._all_pos[r], self.device))

    def append_tokens(self, c, kr, seq, pos, stream=None):
        qkn_mla_append(self.dims, c, kr, seq, pos, self.block_table, self.w_k, self.gamma_kr,
                       self.kv, self.alpha_k, self.err_flag, stream)

    def fill_history(self, stream=None):
        """Append every token except the s_q newest of each sequence."""
        if len(self._old_rows):
            self.append_rows(self._old_rows, stream=stream)

    def append_new(self, stream=None):
        qkn_mla_append(self.dims, self.c_new, self.kr_new, self.new_seq, self.new_pos,
                       self.block_table, self.w_k, self.gamma_kr, self.kv, self.alpha_k,
                       self.err_flag, stream)

    def decode(self, flags: int = 0, stream=None, kv=None, alpha_k=None):
        qkn_mla_decode(self.dims, self.q_tilde, self.alpha_q, self.q_rope_normed,
                       self.kv if kv is None else kv,
                       self.alpha_k if alpha_k is None else alpha_k, self.block_table,
                       self.seq_lens, self.num_splits, flags, self.o_partial, self.lse_partial,
                       self.err_flag, stream)

    def attend(self, flags: int = 0, stream=None, kv=None, alpha_k=None):
        """Decode and combine in one library call, the partials in a workspace
        sized by the library (allocated on first use)."""
        if getattr(self, "_ws_splits", None) != self.num_splits:
            self.workspace = alloc_decode_workspace(self.dims, self.num_splits, self.device)
            self._ws_splits = self.num_splits
        qkn_mla_decode_attend(self.dims, self.q_tilde, self.alpha_q, self.q_rope_normed,
                              self.kv if kv is None else kv,
                              self.alpha_k if alpha_k is None else alpha_k, self.block_table,
                              self.seq_lens, self.num_splits, flags, self.workspace,
                              self.o_latent, self.lse, self.err_flag, stream)

    def combine(self, stream=None):
        qkn_mla_combine(self.dims, self.num_splits, self.o_partial, self.lse_partial,
                        self.o_latent, self.lse, stream)

    def combine_project(self, flags: int = 0, stream=None):
        """The combine and the value up-projection into self.o."""
        qkn_mla_combine_project(self.dims, self.num_splits, self.o_partial, self.lse_partial,
                                self.w_v, self.o_latent, self.lse, self.o, flags, stream)

    def prepare(self):
        """The query side and the append of the new tokens."""
        self.absorb()
        self.append_new()

    def step(self, flags: int = 0):
        """One decode step on the current stream."""
        self.prepare()
        self.decode(flags)
        self.combine()

    # -- chunked prefill on the explicit path (s_q = the chunk length) ----------
    def alloc_prefill(self):
        """Buffers of the prefill calls: q^ (half), the materialised keys and
        values [B, max_T, G, d] (half) and the output o, lse."""
        wl, dev = self.wl, self.device
        B, sq, H = wl.batch, wl.s_q, wl.heads
        max_T = self.dims.max_pages_per_seq * PAGE_SIZE
        self.q_hat = torch.empty((B, sq, H, wl.head_dim), dtype=torch.float16, device=dev)
        self.k_hat = torch.empty((B, max_T, wl.groups, wl.head_dim), dtype=torch.float16,
                                 device=dev)
        self.v_exp = torch.empty_like(self.k_hat)
        self.o_prefill = torch.empty((B, sq, H, wl.head_dim), dtype=torch.float32, device=dev)
        self.lse_prefill = torch.empty((B, sq, H), dtype=torch.float32, device=dev)

    def prefill_query(self, stream=None):
        qkn_mla_prefill_query(self.dims, self.q, self.q_rope, self.q_pos, self.gamma_q,
                              self.gamma_qr, self.q_hat, self.q_rope_normed, stream)

    def prefill_expand(self, stream=None):
        qkn_mla_prefill_expand(self.dims, self.kv, self.alpha_k, self.block_table, self.seq_lens,
                               self.w_k, self.w_v, self.gamma_k, self.k_hat, self.v_exp,
                               self.err_flag, stream)

    def prefill_attend(self, stream=None):
        qkn_mla_prefill_attend(self.dims, self.q_hat, self.q_rope_normed, self.k_hat, self.v_exp,
                               self.kv, self.block_table, self.seq_lens, self.o_prefill,
                               self.lse_prefill, self.err_flag, stream)

    # -- the GQA path: cache of per-group normed keys and values ------------------
    def alloc_gqa(self, num_splits: int = 1, fill_word: int = 0x7E01):
        """The GQA cache (int16 words [num_pages, 64, 2 G d + d_R], every word
        ``fill_word`` until written), the half query, the output and, for
        several splits, the workspace."""
        wl, dev = self.wl, self.device
        B, sq, H = wl.batch, wl.s_q, wl.heads
        w = np.uint16(fill_word).view(np.int16)
        self.kvg = torch.full((self.num_pages, PAGE_SIZE, gqa_row_words(self.dims)), int(w),
                              dtype=torch.int16, device=dev)
        if not hasattr(self, "q_hat"):
            self.q_hat = torch.empty((B, sq, H, wl.head_dim), dtype=torch.float16, device=dev)
        self.o_gqa = torch.empty((B, sq, H, wl.head_dim), dtype=torch.float32, device=dev)
        self.lse_gqa = torch.empty((B, sq, H), dtype=torch.float32, device=dev)
        self.set_gqa_splits(num_splits)

    def set_gqa_splits(self, num_splits: int):
        self.gqa_splits = int(num_splits)
        self.gqa_ws = None
        if self.gqa_splits > 1:
            self.gqa_ws = torch.empty(gqa_workspace_bytes(self.dims, self.gqa_splits),
                                      dtype=torch.uint8, device=self.device)

    def gqa_append_tokens(self, c, kr, seq, pos, stream=None):
        qkn_mla_gqa_append(self.dims, c, kr, seq, pos, self.block_table, self.w_k, self.w_v,
                           self.gamma_k, self.gamma_kr, self.kvg, self.err_flag, stream)

    def gqa_fill_history(self, chunk: int = 1 << 18, stream=None):
        """GQA-append every token except the s_q newest of each sequence."""
        rows = np.asarray(self._old_rows)
        for s in range(0, len(rows), chunk):
            r = rows[s:s + chunk]
            self.gqa_append_tokens(_dev(self.inp["c"][r], self.device),
                                   _dev(self.inp["k_rope"][r], self.device),
                                   _dev(self._all_seq[r], self.device),
                                   _dev(self._all_pos[r], self.device), stream)

    def gqa_append_new(self, stream=None):
        self.gqa_append_tokens(self.c_new, self.kr_new, self.new_seq, self.new_pos, stream)

    def gqa_attend(self, stream=None, kvg=None):
        qkn_mla_gqa_attend(self.dims, self.q_hat, self.q_rope_normed,
                           self.kvg if kvg is None else kvg, self.block_table, self.seq_lens,
                           self.gqa_splits, self.gqa_ws, self.o_gqa, self.lse_gqa, self.err_flag,
                           stream)

    def gqa_step(self, stream=None, kvg=None):
        """One decode step of the GQA path: the query side, the append of the
        new tokens, the attention (on ``kvg``, default the runner's cache)."""
        kvg = self.kvg if kvg is None else kvg
        self.prefill_query(stream)
        qkn_mla_gqa_append(self.dims, self.c_new, self.kr_new, self.new_seq, self.new_pos,
                           self.block_table, self.w_k, self.w_v, self.gamma_k, self.gamma_kr, kvg,
                           self.err_flag, stream)
        self.gqa_attend(stream, kvg)

    # -- host copies -------------------------------------------------------------
    def kv_words(self) -> np.ndarray:
        """Cache as raw storage words (uint16 for bf16, float32 for f32)."""
        if self.dims.cache_dtype == QKN_BF16:
            return self.kv.view(torch.int16).cpu().numpy().view(np.uint16)
        return self.kv.cpu().numpy()

    def words(self, t: torch.Tensor) -> np.ndarray:
        if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
