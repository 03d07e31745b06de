/*
 * qkn_mla.h -- C ABI of the QK-Normed MLA absorbed-latent decode library
 * (libqknmla.so, HIP kernels for gfx950 / MI355X).
 *
 * The method: "QK-Normed MLA: QK normalization without full key caching"
 * (arXiv 2606.16310; gist.science technical summary, section "Metodologia",
 * and the arXiv abstract).  Post-projection QK RMSNorm is kept compatible with
 * the latent decode path of multi-head latent attention by splitting
 * RMSNorm(z) = z * gamma / S(z) into a static weight gamma, folded into the
 * query, and a dynamic scalar 1/S(z), kept as one float per token and KV group.
 * The decode cache holds only the latent c_t, a separately RMS-normed RoPE key
 * and those scalars; full keys are never stored.
 *
 * Notation (also the names of the qkn_mla_dims fields):
 *   B batch, s_q query tokens per step, H query heads, G KV groups (H % G == 0,
 *   head h belongs to group g(h) = h / (H/G)), r latent rank, d content head
 *   dim, d_R RoPE dim, T_b length of sequence b counting its s_q new tokens.
 *   Query token i of sequence b sits at position T_b - s_q + i and attends to
 *   the tokens t <= T_b - s_q + i.
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer; `dims` is a host pointer.
 *     Arrays are dense, row-major, innermost dimension last, with the shapes
 *     given per call.  Float arrays marked (cache dtype) hold float32 when
 *     dims->cache_dtype == QKN_F32 and bfloat16 when it is QKN_BF16.
 *   - The caller owns and allocates every buffer, including the split-KV
 *     partials.  The library allocates no device memory and keeps no state
 *     between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream) and never synchronise the host.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns a negative qkn_status and launches nothing.  No C++
 *     exception crosses this interface.  QKN_ERR_HIP reports a failed launch.
 *   - Pointers must be 16-byte aligned.
 */
#ifndef QKN_MLA_H
#define QKN_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define QKN_API __attribute__((visibility("default")))
#else
#define QKN_API
#endif

#define QKN_MLA_ABI_VERSION 9
#define QKN_MLA_PAGE_SIZE 64

typedef enum {
  QKN_OK = 0,
  QKN_ERR_INVALID_ARG = -1, /* null pointer, non-positive or inconsistent size */
  QKN_ERR_UNSUPPORTED = -2, /* a size the kernels do not handle (see checks)  */
  QKN_ERR_ALIGNMENT = -3,   /* a pointer not 16-byte aligned                  */
  QKN_ERR_HIP = -4,         /* the HIP runtime reported an error on launch    */
  QKN_ERR_SCRATCH = -5      /* the request needs more than the static scratch
                               of qkn_mla_decode_attend_noalloc holds          */
} qkn_status;

typedef enum { QKN_F32 = 0, QKN_BF16 = 1, QKN_F16 = 2 } qkn_dtype;

/* Bits that qkn_mla_append and qkn_mla_decode OR into *err_flag. */
#define QKN_FLAG_INDEX 1         /* an index, position, length or page entry out of range */
#define QKN_FLAG_PARTIAL_RANGE 2 /* a half-precision split partial beyond +-65504 */
#define QKN_FLAG_RESTART 4       /* informational, not an error: a split of the
                                    matrix-core decode took its exact restart (a
                                    logit outgrew the split's exponent reference
                                    by more than 2^96); the result is unaffected */

/* Flags of qkn_mla_decode. */
#define QKN_DECODE_NO_ALPHA 1u      /* drop both inverse-RMS factors: plain absorbed
                                       MLA, kept only to measure the cost of QK-norm */
#define QKN_DECODE_FORCE_GENERIC 2u /* run the generic (vector-ALU) kernel even when
                                       the matrix-core kernel applies */

typedef struct {
  int32_t batch;             /* B  >= 1 */
  int32_t s_q;               /* query tokens per sequence and step, >= 1 */
  int32_t heads;             /* H  >= 1 */
  int32_t groups;            /* G  >= 1, H % G == 0 */
  int32_t rank;              /* r  latent rank, multiple of 8 */
  int32_t head_dim;          /* d  content head dim, multiple of 4 */
  int32_t rope_dim;          /* d_R, even, multiple of 8 (may be 0) */
  int32_t page_size;         /* must be QKN_MLA_PAGE_SIZE */
  int32_t max_pages_per_seq; /* columns of the block table */
  int32_t num_pages;         /* pages in the cache pool */
  float eps;                 /* RMSNorm epsilon, inside the root: 1/sqrt(mean(z^2)+eps) */
  float softmax_scale;       /* applied to the full logit (content + RoPE) */
  float rope_theta;          /* RoPE base; 0 disables the rotation */
  int32_t cache_dtype;       /* qkn_dtype of the cache and of q~ / normed RoPE query */
} qkn_mla_dims;

/*
 * Element type of the split-KV partials o_partial of qkn_mla_decode and
 * qkn_mla_combine ("partial dtype"), as qkn_mla_partial_dtype() returns it:
 * today IEEE binary16 (QKN_F16) when the cache is bfloat16 and float32 when it
 * is float32.  A partial is a convex combination of cached latent rows, so
 * half keeps it to within 2^-11 of its own magnitude, eight times finer than
 * the bfloat16 rounding of the latents it is made of, and halves the bytes
 * the split-KV path writes and reads back.  Callers that do not need the
 * partials themselves use qkn_mla_decode_attend with a workspace sized by
 * qkn_mla_decode_workspace_bytes and need not know this type at all.
 */

/* QKN_MLA_ABI_VERSION of the loaded library. */
QKN_API int qkn_mla_abi_version(void);

/* Partial dtype (QKN_F16 or QKN_F32) for these dims, or a negative qkn_status
 * when the dims are invalid. */
QKN_API int qkn_mla_partial_dtype(const qkn_mla_dims* dims);

/*
 * Bytes of device workspace qkn_mla_decode_attend needs for `num_splits`
 * split-KV partitions: the partials o_partial [B, s_q, H, num_splits, r]
 * (partial dtype) and lse_partial [B, s_q, H, num_splits] float32, each
 * starting on a 256-byte boundary.  Returns 0 when the dims or num_splits are
 * invalid (every valid request needs more than 0 bytes).
 *   Source: the split-KV partitions whose partial results the log-sum-exp
 *   combine merges (the long-context decode of the QK-Normed MLA summary,
 *   "Resultados", reaching 256k tokens).
 */
QKN_API size_t qkn_mla_decode_workspace_bytes(const qkn_mla_dims* dims, int32_t num_splits);

/* Static text for a qkn_status value. */
QKN_API const char* qkn_status_string(int status);

/* Validates `dims` alone (the checks every call repeats). */
QKN_API int qkn_mla_check_dims(const qkn_mla_dims* dims);

/* Which decode kernel qkn_mla_decode would launch for these sizes and flags:
 * 1 = matrix-core (MFMA) kernel, 0 = generic kernel, < 0 = a qkn_status error.
 * The matrix-core kernel takes a bfloat16 cache with r = 512, d_R = 64, at most
 * 8 KV groups and a multiple of 32 heads per group; every other valid size
 * runs on the generic kernel. */
QKN_API int qkn_mla_decode_kernel_kind(const qkn_mla_dims* dims, int32_t num_splits, uint32_t flags);

/*
 * qkn_mla_absorb_query -- query side of one decode step.
 *   Source: QK-Normed MLA summary, "Metodologia" item 1 (the static key weight
 *   gamma_k, together with gamma_q, is pre-multiplied into the query and
 *   absorbed into the query-side projection) and the decode-logit equation
 *   (alpha^q per query row); item 4 (the RoPE block is normalised on its own
 *   and stays a materialised vector).
 *
 *   For every (b, i, h), with g = g(h):
 *     q_tilde[b,i,h,:]  = (gamma_q * gamma_k[g] * q[b,i,h,:]) . W^K_g^T   (length r)
 *     alpha_q[b,i,h]    = 1 / sqrt(mean(q[b,i,h,:]^2) + eps)
 *     q_rope_normed[b,i,h,:] = RoPE(gamma_qr * q_rope[b,i,h,:] / RMS, q_pos[b,i])
 *   RoPE rotates the pairs (j, j + d_R/2) by q_pos * theta^(-2j/d_R).
 *
 *   q       [B, s_q, H, d]   float32      q_rope [B, s_q, H, d_R] float32
 *   q_pos   [B, s_q]         int32        RoPE position of each query token
 *   w_k     [G, r, d]        float32      key up-projection, k_{t,g} = c_t . w_k[g]
 *   gamma_q [d], gamma_k [G, d], gamma_qr [d_R]      float32
 *   out: q_tilde [B, s_q, H, r] (cache dtype), alpha_q [B, s_q, H] float32,
 *        q_rope_normed [B, s_q, H, d_R] (cache dtype).
 *   Arithmetic in float32; bfloat16 outputs are rounded to nearest even.
 */
QKN_API int qkn_mla_absorb_query(const qkn_mla_dims* dims, const float* q, const float* q_rope,
                         const int32_t* q_pos, const float* w_k, const float* gamma_q,
                         const float* gamma_k, const float* gamma_qr, void* q_tilde,
                         float* alpha_q, void* q_rope_normed, void* stream);

/*
 * qkn_mla_append -- write new tokens into the paged cache.
 *   Source: QK-Normed MLA summary, "Metodologia" items 2 and 3 (the dynamic
 *   key statistic reduces to one inverse-RMS scalar per token and KV group,
 *   kept in a small scalar cache beside the latent; normalised keys are not
 *   stored) and item 4 (the RoPE key is normalised separately).
 *
 *   Token n (0 <= n < n_tokens) of sequence seq_idx[n] at position pos[n]
 *   goes to page block_table[seq_idx[n]][pos[n] / 64], row pos[n] % 64:
 *     kv_cache[page][row][0:r]     = c_new[n]  (stored in the cache dtype)
 *     kv_cache[page][row][r:r+d_R] = RoPE(gamma_kr * k_rope_new[n] / RMS, pos[n])
 *     alpha_k_cache[page][row][g]  = 1 / sqrt(mean((c . W^K_g)^2) + eps), g < G,
 *   where c is the latent AS STORED (so the scalar matches the cached latent).
 *   The projected key c . W^K_g is formed in registers only.  From 4096
 *   tokens in one call (bf16 cache, d = 32, 64, 128 or 256) the keys of all
 *   tokens are one matrix product per group on the matrix cores (the stored
 *   bf16 latent times W^K_g split into three bf16 words: exact products,
 *   float32 sums); the stored words are formed as for fewer tokens.
 *
 *   c_new [n_tokens, r], k_rope_new [n_tokens, d_R]  float32
 *   seq_idx, pos [n_tokens] int32;  block_table [B, max_pages_per_seq] int32
 *   w_k [G, r, d], gamma_kr [d_R] float32
 *   in/out: kv_cache [num_pages, 64, r + d_R] (cache dtype),
 *           alpha_k_cache [num_pages, 64, G] float32.
 *   err_flag (nullable) int32: a token whose sequence index, position or page
 *   entry is out of range is skipped and QKN_FLAG_INDEX is ORed into *err_flag.
 *   n_tokens == 0 is a no-op.
 */
QKN_API int qkn_mla_append(const qkn_mla_dims* dims, int32_t n_tokens, const float* c_new,
                   const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                   const int32_t* block_table, const float* w_k, const float* gamma_kr,
                   void* kv_cache, float* alpha_k_cache, int32_t* err_flag, void* stream);

/*
 * qkn_mla_decode -- split-KV absorbed-latent attention over the paged cache.
 *   Source: QK-Normed MLA summary, "Metodologia", decode-logit equation (the
 *   content logit (q~ . c_t) alpha^q alpha^k_{t,g(h)}, scalars applied as a
 *   row-column scaling before the softmax) and "Significancia" (the scalars
 *   must be fused into the attention path to avoid extra memory traffic); the
 *   RoPE dot of the shared RoPE key comes from the MQA-absorbed path of the
 *   GQLA summary, section 2.
 *
 *   For every query row (b, i, h) and split p < num_splits, over the visible
 *   tokens t of the split's range [p L, min((p+1) L, T_b)), with
 *   L = 64 * ceil(ceil(T_b / num_splits) / 64):
 *     l_t = softmax_scale * ((q~ . c_t) alpha^q alpha^k_{t,g(h)} + q^R . k^R_t)
 *     o_partial[b,i,h,p,:]  = sum_t softmax(l)_t c_t       (latent space)
 *     lse_partial[b,i,h,p]  = ln sum_t e^{l_t}   (-inf and o = 0 if no token)
 *
 *   q_tilde [B,s_q,H,r], q_rope_normed [B,s_q,H,d_R] (cache dtype);
 *   alpha_q [B,s_q,H] float32; kv_cache, alpha_k_cache as written by append;
 *   block_table [B, max_pages_per_seq], seq_lens [B] int32 (T_b >= s_q).
 *   out: o_partial [B, s_q, H, num_splits, r] (partial dtype, see above),
 *        lse_partial [B, s_q, H, num_splits] float32.
 *   flags: QKN_DECODE_* bits.  err_flag (nullable), bits ORed in:
 *   QKN_FLAG_INDEX when a sequence length exceeds max_pages_per_seq * 64 (it
 *   is clamped) or a page entry is out of range (those tokens are skipped);
 *   QKN_FLAG_PARTIAL_RANGE when a half partial would exceed the half range
 *   (latent entries beyond +-65504 in the cache); it is then stored as +-inf;
 *   QKN_FLAG_RESTART (informational) when a split took the exact restart.
 *   Products run on the matrix cores (bf16 operands, float32 accumulation)
 *   when qkn_mla_decode_kernel_kind() says 1, otherwise on the vector ALUs in
 *   float32.
 */
QKN_API int qkn_mla_decode(const qkn_mla_dims* dims, const void* q_tilde, const float* alpha_q,
                   const void* q_rope_normed, const void* kv_cache,
                   const float* alpha_k_cache, const int32_t* block_table,
                   const int32_t* seq_lens, int32_t num_splits, uint32_t flags,
                   void* o_partial, float* lse_partial, int32_t* err_flag, void* stream);

/*
 * qkn_mla_combine -- merge the split-KV partials of qkn_mla_decode.
 *   Source: the log-sum-exp merge that split-KV decoding over long contexts
 *   needs (GQLA summary, section 1: decode is bound by reading the cached
 *   history; the long-context benchmarks of the QK-Normed MLA summary,
 *   "Resultados", reach 256k tokens).
 *
 *     M = max_p lse_p;  lse = M + ln sum_p e^{lse_p - M};
 *     o_latent = sum_p e^{lse_p - lse} o_p
 *   A row whose splits are all empty gets o_latent = 0 and lse = -inf.
 *   in: o_partial [B,s_q,H,num_splits,r] (partial dtype),
 *       lse_partial [B,s_q,H,num_splits] float32
 *   out: o_latent [B, s_q, H, r] float32, lse [B, s_q, H] float32 (natural log).
 *   qkn_mla_combine_project also applies the value up-projection.
 */
QKN_API int qkn_mla_combine(const qkn_mla_dims* dims, int32_t num_splits, const void* o_partial,
                    const float* lse_partial, float* o_latent, float* lse, void* stream);

/*
 * Chunked prefill on the explicit path: three calls.
 *   Source: QK-Normed MLA summary, "Planteamiento del Problema" (the explicit
 *   path materialises k = c W^K_g and applies the RMSNorm after the
 *   projection) and "Metodologia" item 4 (the RoPE block is normed on its
 *   own).  A chunk of dims->s_q new query tokens per sequence attends
 *   causally to the whole cache, the chunk included (its tokens appended
 *   first with qkn_mla_append): query i of sequence b sits at position
 *   T_b - s_q + i and sees the tokens t <= T_b - s_q + i.
 *   Supported for a bf16 cache with r = 512, d = 128, d_R = 64 and a multiple
 *   of 32 heads per group (QKN_ERR_UNSUPPORTED otherwise).  max_T below is
 *   dims->max_pages_per_seq * 64.  The materialised q_hat, k_hat and v are IEEE
 *   half (fp16): the norm bounds |q_hat_j| by sqrt(d) |gamma_q,j| and |k_hat_j|
 *   likewise, and half keeps three more bits than bf16.
 *
 * qkn_mla_prefill_query: q_hat[b,i,h,:] = gamma_q * q / RMS(q) (fp16) and
 *   q_rope_normed as qkn_mla_absorb_query writes it.
 *   q [B, s_q, H, d], q_rope [B, s_q, H, d_R] float32; q_pos [B, s_q] int32;
 *   out: q_hat [B, s_q, H, d] fp16, q_rope_normed [B, s_q, H, d_R] bf16.
 */
QKN_API int qkn_mla_prefill_query(const qkn_mla_dims* dims, const float* q, const float* q_rope,
                          const int32_t* q_pos, const float* gamma_q, const float* gamma_qr,
                          void* q_hat, void* q_rope_normed, void* stream);

/*
 * qkn_mla_prefill_expand: keys and values of every cached token t < T_b of
 *   every sequence and group, from the stored latent c_t:
 *     k_hat[b,t,g,:] = gamma_k[g] * (c_t W^K_g) * alpha_k_cache[t,g]   (fp16)
 *     v[b,t,g,:]     = c_t W^V_g                                        (fp16)
 *   (alpha^k is 1/RMS of the same projection, so k_hat = RMSNorm(c_t W^K_g)),
 *   as matrix products on the matrix cores with every product exact and
 *   float32 sums.  Rows t >= T_b are written as zeros.
 *   out: k_hat, v [B, max_T, G, d] fp16.  w_k, w_v [G, r, d], gamma_k [G, d]
 *   float32.  err_flag (nullable): a token on an out-of-range page entry is
 *   written as zeros and QKN_FLAG_INDEX is ORed in; a value beyond the half
 *   range (stored as +-inf) ORs QKN_FLAG_PARTIAL_RANGE.
 */
QKN_API int qkn_mla_prefill_expand(const qkn_mla_dims* dims, const void* kv_cache,
                           const float* alpha_k_cache, const int32_t* block_table,
                           const int32_t* seq_lens, const float* w_k, const float* w_v,
                           const float* gamma_k, void* k_hat, void* v, int32_t* err_flag,
                           void* stream);

/*
 * qkn_mla_prefill_attend: for query i of sequence b and head h (group g),
 *   over the keys t <= T_b - s_q + i:
 *     l_t = softmax_scale * (q_hat . k_hat[b,t,g] + q_rope_normed . k^R_t),
 *     o[b,i,h,:] = sum_t softmax(l)_t v[b,t,g,:],  lse[b,i,h] = ln sum_t e^{l_t},
 *   with k^R_t the stored RoPE key of the paged cache.  Flash attention on
 *   the matrix cores: fp16 content and value operands, bf16 RoPE operands,
 *   float32 accumulation, probabilities rounded to fp16 for the P.V product
 *   and normalised by the sum of the same rounded values.
 *   out: o [B, s_q, H, d], lse [B, s_q, H] float32.
 *   err_flag (nullable): T_b < s_q, T_b beyond the page table, or a bad page
 *   entry ORs QKN_FLAG_INDEX (bad pages read as zero RoPE keys).
 */
QKN_API int qkn_mla_prefill_attend(const qkn_mla_dims* dims, const void* q_hat,
                           const void* q_rope_normed, const void* k_hat, const void* v,
                           const void* kv_cache, const int32_t* block_table,
                           const int32_t* seq_lens, float* o, float* lse, int32_t* err_flag,
                           void* stream);

/*
 * qkn_mla_decode_sparse -- selected-token decode (the partials of a split-KV
 * decode over listed cache tokens only).
 *   Source: GQLA summary, section 2, "GQLA Disperso": fine-grained sparse
 *   attention over the latent cache stays on the MQA-absorbed path, whose
 *   decode-logit equation (QK-Normed MLA summary, "Metodologia") it keeps.
 *
 *   Query token (b, i) attends to the cache tokens listed in
 *   indices[b][i][0 .. index_len) (logical positions within sequence b,
 *   shared by every head and group; -1 marks an unused entry).  Logits, the
 *   softmax over the listed tokens (taken as listed: a position listed twice
 *   counts twice), o_p and lse_p are those of qkn_mla_decode, and the partials
 *   have its layout, so qkn_mla_combine (or qkn_mla_combine_project) merges
 *   them.  Split p covers list entries p L .. p L + L - 1, L = index_len / P
 *   rounded up to a multiple of 32.  A split with no valid entry, or a list
 *   with none, gives lse_p = -inf and o_p = 0 (combine then gives o = 0,
 *   lse = -inf).
 *   indices [B, s_q, index_len] int32 (16-byte aligned; may be null when
 *   index_len == 0); the other arguments as for qkn_mla_decode.
 *   err_flag (nullable): an entry that is not -1 and lies outside 0 .. T_b -
 *   s_q + i, or whose page entry is out of range, is skipped and
 *   QKN_FLAG_INDEX is ORed in (as is an out-of-range seq_lens[b]).
 *   Returns QKN_ERR_UNSUPPORTED unless the matrix-core decode takes the dims
 *   with heads a multiple of 128, the cache is under 4 GiB, and a split holds
 *   at most 2048 list entries (raise num_splits for longer lists); and for
 *   QKN_DECODE_FORCE_GENERIC.  QKN_DECODE_NO_ALPHA is accepted.
 */
QKN_API int qkn_mla_decode_sparse(const qkn_mla_dims* dims, const void* q_tilde,
                          const float* alpha_q, const void* q_rope_normed,
                          const void* kv_cache, const float* alpha_k_cache,
                          const int32_t* block_table, const int32_t* seq_lens,
                          const int32_t* indices, int32_t index_len, int32_t num_splits,
                          uint32_t flags, void* o_partial, float* lse_partial,
                          int32_t* err_flag, void* stream);

/*
 * qkn_mla_decode_attend -- qkn_mla_decode followed by qkn_mla_combine, with
 * the split partials in a caller-provided workspace.
 *   Source: as for qkn_mla_decode and qkn_mla_combine.
 *
 *   Writes o_latent [B, s_q, H, r] and lse [B, s_q, H] (float32) with the same
 *   bits as qkn_mla_decode into partials, then qkn_mla_combine of them, for
 *   the same arguments and flags.  `workspace` is a device buffer of
 *   `workspace_bytes` >= qkn_mla_decode_workspace_bytes(dims, num_splits)
 *   bytes, 256-byte aligned, owned by the caller; its contents on entry do not
 *   matter and on return are unspecified.  Two calls that share a workspace
 *   must be ordered on one stream.  A workspace that is too small or
 *   misaligned is rejected (QKN_ERR_INVALID_ARG / QKN_ERR_ALIGNMENT) before
 *   anything is launched.  err_flag as for qkn_mla_decode.
 */
QKN_API int qkn_mla_decode_attend(const qkn_mla_dims* dims, const void* q_tilde,
                          const float* alpha_q, const void* q_rope_normed,
                          const void* kv_cache, const float* alpha_k_cache,
                          const int32_t* block_table, const int32_t* seq_lens,
                          int32_t num_splits, uint32_t flags, void* workspace,
                          size_t workspace_bytes, float* o_latent, float* lse,
                          int32_t* err_flag, void* stream);

/* Bytes of the static device scratch array of qkn_mla_decode_attend_noalloc. */
#define QKN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * qkn_mla_decode_attend_noalloc -- qkn_mla_decode_attend with the split
 * partials in a static device array of the library instead of a caller
 * workspace.  For callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 *   Same arguments, results and bits as qkn_mla_decode_attend without
 *   `workspace` / `workspace_bytes`.  The call allocates nothing: no hipMalloc,
 *   hipFree or allocating library routine.  The partials go to a file-scope
 *   __device__ array of QKN_NOALLOC_SCRATCH_BYTES (64 MiB); every device the
 *   library runs on holds its own copy from the library's first use there
 *   until the process ends.  Its address is looked up once per device, on the
 *   first call made with that device current.
 *   A request whose qkn_mla_decode_workspace_bytes() exceeds
 *   QKN_NOALLOC_SCRATCH_BYTES is rejected with QKN_ERR_SCRATCH before
 *   anything is launched (e.g. 4096 query rows at r = 512 take at most 15
 *   splits).  Every call on one device shares that device's array, which
 *   keeps the last call's contents (nothing in it needs to start at zero):
 *   calls that overlap on one device -- on two streams, or from two host
 *   threads without ordering -- race on it and must not be issued.
 */
QKN_API int qkn_mla_decode_attend_noalloc(const qkn_mla_dims* dims, const void* q_tilde,
                                  const float* alpha_q, const void* q_rope_normed,
                                  const void* kv_cache, const float* alpha_k_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t num_splits, uint32_t flags, float* o_latent,
                                  float* lse, int32_t* err_flag, void* stream);

/* Flags of qkn_mla_combine_project.  o_latent and lse are the same bits in
 * every form; o is within the same bound (the forms divide the reduction
 * among waves differently) and the same bits on every run of one form. */
#define QKN_PROJECT_FUSED 1u    /* one launch (merge and products per block) where
                                   its shape conditions hold, whatever the size */
#define QKN_PROJECT_TWO_PASS 2u /* qkn_mla_combine, then the products */

/*
 * qkn_mla_combine_project -- qkn_mla_combine followed by the value
 * up-projection of every query row.
 *   Source: on the absorbed path the attention-weighted sum is formed in
 *   latent space and the head's value up-projection is applied to it once
 *   (QK-Normed MLA summary, the absorbed form of the problem statement; GQLA
 *   summary, section 2, the absorbed MLA path).
 *
 *     o_latent, lse  exactly as qkn_mla_combine writes them (same bits);
 *     o[b,i,h,:]     = o_latent[b,i,h,:] . W^V_{g(h)}     (d_v = head_dim)
 *   in: o_partial, lse_partial as for qkn_mla_combine;
 *       w_v [G, r, head_dim] float32 (row m of W^V_g maps latent entry m).
 *   out: o_latent [B,s_q,H,r], lse [B,s_q,H], o [B,s_q,H,head_dim], float32.
 *   The products run on the matrix cores with both operands split into
 *   bf16 hi + lo words (each product within 3 * 2^-16 of exact, float32
 *   sums) when r is a multiple of 128 up to 512, head_dim is 32, 64, 128 or
 *   256 and H/G is a multiple of 32; otherwise in float32 on the vector ALUs.
 *   With half partials, at most 16 splits and enough rows (automatic), or with
 *   QKN_PROJECT_FUSED, the merge and the products share one launch; otherwise
 *   qkn_mla_combine runs first.  flags: QKN_PROJECT_* bits.
 */
QKN_API int qkn_mla_combine_project(const qkn_mla_dims* dims, int32_t num_splits,
                            const void* o_partial, const float* lse_partial,
                            const float* w_v, float* o_latent, float* lse, float* o,
                            uint32_t flags, void* stream);

/*
 * The GQA path of GQLA with QK-norm.
 *   Source: GQLA summary, section 2 "Arquitectura" (the GQA path: the latent is
 *   expanded into g groups of keys and values that the cache stores, plus the
 *   shared RoPE key, and the decode is plain grouped-query attention with no
 *   latent expansion per step; the compute-friendly one of two algebraically
 *   equivalent paths over the same weights) and the QK-Normed MLA summary,
 *   "Planteamiento del Problema" (the key is RMS-normed after its
 *   up-projection, so the stored key is the normed one).
 *   Supported for a bf16 latent dtype with d = 128, d_R = 64, r a multiple of
 *   16 and a multiple of 32 heads per group (QKN_ERR_UNSUPPORTED otherwise).
 *
 *   The GQA cache is paged like the latent cache (the same block table and
 *   64-token pages), one row of W = 2 G d + d_R 16-bit words per token:
 *     words [2 d g, 2 d g + d)        the normed key of group g  (IEEE half)
 *     words [2 d g + d, 2 d (g + 1))  the value of group g       (IEEE half)
 *     words [2 d G, 2 d G + d_R)      the normed, rotated RoPE key (bf16)
 *   kvg_cache [num_pages, 64, W], owned by the caller.  The query side is
 *   qkn_mla_prefill_query's q_hat (fp16) and q_rope_normed (bf16).
 */

/*
 * qkn_mla_gqa_append: for each of the n_tokens new tokens (seq_idx[n],
 *   pos[n]), with c the latent rounded to bf16 (the latent cache's stored
 *   value):
 *     key_g   = gamma_k[g] * k / RMS(k),  k = c W^K_g      (half)
 *     value_g = c W^V_g                                    (half)
 *     RoPE key as qkn_mla_append stores it                 (bf16)
 *   into the slot block_table[seq][pos / 64] * 64 + pos % 64.  The products
 *   run on the matrix cores with every product exact and float32 sums.
 *   c_new [N, r], k_rope_new [N, d_R], w_k, w_v [G, r, d], gamma_k [G, d],
 *   gamma_kr [d_R] float32; seq_idx, pos [N] int32.
 *   err_flag (nullable): a token whose sequence, position or page entry is out
 *   of range is skipped and ORs QKN_FLAG_INDEX; a value beyond the half range
 *   (stored as +-inf) ORs QKN_FLAG_PARTIAL_RANGE.  Tokens of one call must
 *   name distinct slots.
 */
QKN_API int qkn_mla_gqa_append(const qkn_mla_dims* dims, int32_t n_tokens, const float* c_new,
                       const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                       const int32_t* block_table, const float* w_k, const float* w_v,
                       const float* gamma_k, const float* gamma_kr, void* kvg_cache,
                       int32_t* err_flag, void* stream);

/*
 * Bytes of device workspace qkn_mla_gqa_attend needs for `num_splits` > 1:
 *   half partials [B, s_q, H, num_splits, d] and float32 lse partials
 *   [B, s_q, H, num_splits], each on a 256-byte boundary.  0 for invalid
 *   dims or num_splits.
 */
QKN_API size_t qkn_mla_gqa_workspace_bytes(const qkn_mla_dims* dims, int32_t num_splits);

/*
 * qkn_mla_gqa_attend: decode over the GQA cache.  For query i of sequence b
 *   and head h (group g), over the visible tokens t <= T_b - s_q + i:
 *     l_t = softmax_scale * (q_hat . key_g[t] + q_rope_normed . kR[t]),
 *     o[b,i,h,:] = sum_t softmax(l)_t value_g[t],  lse[b,i,h] = ln sum_t e^{l_t}.
 *   The keys are split into num_splits partitions of whole pages (split p
 *   covers [p L, min((p + 1) L, T_b)), L = 64 ceil(ceil(T_b / P) / 64), as the
 *   latent decode); each is attended on the matrix cores (fp16 key and value
 *   operands, bf16 RoPE operands, float32 accumulation, probabilities rounded
 *   to fp16 and normalised by the sum of the same rounded values), and with
 *   num_splits > 1 the partials (half, in `workspace`) are merged by the
 *   log-sum-exp combine.  With num_splits == 1 o and lse are written directly
 *   and `workspace` may be null; otherwise `workspace` is a device buffer of
 *   `workspace_bytes` >= qkn_mla_gqa_workspace_bytes(dims, num_splits) bytes,
 *   256-byte aligned, owned by the caller (contents on return unspecified;
 *   calls sharing one must be ordered on one stream).
 *   q_hat [B, s_q, H, d] fp16, q_rope_normed [B, s_q, H, d_R] bf16.
 *   out: o [B, s_q, H, d], lse [B, s_q, H] float32.
 *   err_flag (nullable): T_b < s_q, T_b beyond the page table, or a bad page
 *   entry ORs QKN_FLAG_INDEX (a bad page reads as zero keys and values).
 */
QKN_API int qkn_mla_gqa_attend(const qkn_mla_dims* dims, const void* q_hat,
                       const void* q_rope_normed, const void* kvg_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int32_t num_splits, void* workspace, size_t workspace_bytes,
                       float* o, float* lse, int32_t* err_flag, void* stream);

/*
 * qkn_mla_stream_read -- a plain read-only stream over device memory (not a
 *   step of the method): the achievable HBM read rate on this GPU, against
 *   which the cache-reading kernels are measured besides the published peak.
 *   Every 16-byte word of src is read once with non-temporal loads
 *   (consecutive lanes on consecutive words, four loads in flight per
 *   thread), and the XOR of all the 32-bit words read is XORed into *sink
 *   (so the caller sets *sink beforehand; the result does not depend on
 *   timing).
 *   src (device) 16-byte aligned, bytes a positive multiple of 16;
 *   sink (device) one 4-byte aligned uint32.  Nothing is written but *sink.
 *   QKN_ERR_INVALID_ARG / QKN_ERR_ALIGNMENT before any launch.
 */
QKN_API int qkn_mla_stream_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QKN_MLA_H */
