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

#define QKN_MLA_ABI_VERSION 3
#define QKN_MLA_PAGE_SIZE 64

typedef enum {
  QKN_OK = 0,
  QKN_ERR_INVALID_ARG = -1, /* null pointer, non-positive or inconsistent size */
  QKN_ERR_UNSUPPORTED = -2, /* a size the kernels do not handle (see checks)  */
  QKN_ERR_ALIGNMENT = -3,   /* a pointer not 16-byte aligned                  */
  QKN_ERR_HIP = -4          /* the HIP runtime reported an error on launch    */
} qkn_status;

typedef enum { QKN_F32 = 0, QKN_BF16 = 1 } qkn_dtype;

/* Bits that qkn_mla_append and qkn_mla_decode OR into *err_flag. */
#define QKN_FLAG_INDEX 1         /* an index, position, length or page entry out of range */
#define QKN_FLAG_PARTIAL_RANGE 2 /* a half-precision split partial beyond +-65504 */

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
 * qkn_mla_combine ("partial dtype"): IEEE binary16 (half) when the cache is
 * bfloat16, float32 when it is float32.  A partial is a convex combination of
 * cached latent rows, so half keeps it to within 2^-11 of its own magnitude,
 * eight times finer than the bfloat16 rounding of the latents it is made of,
 * and halves the bytes the split-KV path writes and reads back.
 */

/* QKN_MLA_ABI_VERSION of the loaded library. */
QKN_API int qkn_mla_abi_version(void);

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
 *   (latent entries beyond +-65504 in the cache); it is then stored as +-inf.
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

#ifdef __cplusplus
}
#endif

#endif /* QKN_MLA_H */
