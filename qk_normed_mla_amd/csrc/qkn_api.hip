// extern "C" entry points of libqknmla.so: host-side validation, then launch.
// Every check runs before any HIP call, so a rejected call touches no device.
#include <cmath>
#include <cstdint>

#include "qkn_internal.h"

namespace {

constexpr int kMaxRank = 1024;
constexpr int kMaxHeadDim = 512;
constexpr int kMaxRopeDim = 256;
constexpr int kMaxSplits = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const qkn_mla_dims* d) {
  if (!d) return QKN_ERR_INVALID_ARG;
  if (d->batch < 1 || d->s_q < 1 || d->heads < 1 || d->groups < 1) return QKN_ERR_INVALID_ARG;
  if (d->heads % d->groups != 0) return QKN_ERR_INVALID_ARG;
  if (d->rank < 8 || d->head_dim < 4 || d->rope_dim < 0) return QKN_ERR_INVALID_ARG;
  if (d->max_pages_per_seq < 1 || d->num_pages < 1) return QKN_ERR_INVALID_ARG;
  if (!(std::isfinite(d->eps) && d->eps >= 0.f)) return QKN_ERR_INVALID_ARG;
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale > 0.f)) return QKN_ERR_INVALID_ARG;
  if (!(std::isfinite(d->rope_theta) && d->rope_theta >= 0.f)) return QKN_ERR_INVALID_ARG;
  if (d->cache_dtype != QKN_F32 && d->cache_dtype != QKN_BF16) return QKN_ERR_INVALID_ARG;
  if (d->page_size != QKN_MLA_PAGE_SIZE) return QKN_ERR_UNSUPPORTED;
  if (d->rank % 8 != 0 || d->head_dim % 4 != 0 || d->rope_dim % 8 != 0) return QKN_ERR_UNSUPPORTED;
  if (d->rank > kMaxRank || d->head_dim > kMaxHeadDim || d->rope_dim > kMaxRopeDim)
    return QKN_ERR_UNSUPPORTED;
  // element counts must fit the 32-bit row indices the kernels use per page/row
  const int64_t rows = (int64_t)d->batch * d->s_q * d->heads;
  if (rows > (int64_t)INT32_MAX / 4) return QKN_ERR_UNSUPPORTED;
  if ((int64_t)d->num_pages * QKN_MLA_PAGE_SIZE > (int64_t)INT32_MAX) return QKN_ERR_UNSUPPORTED;
  return QKN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QKN_OK : QKN_ERR_HIP; }

}  // namespace

extern "C" {

int qkn_mla_abi_version(void) { return QKN_MLA_ABI_VERSION; }

const char* qkn_status_string(int status) {
  switch (status) {
    case QKN_OK: return "ok";
    case QKN_ERR_INVALID_ARG: return "invalid argument (null pointer or inconsistent size)";
    case QKN_ERR_UNSUPPORTED: return "unsupported size for these kernels";
    case QKN_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case QKN_ERR_HIP: return "HIP runtime error on launch";
    default: return "unknown status";
  }
}

int qkn_mla_check_dims(const qkn_mla_dims* dims) { return check_dims(dims); }

int qkn_mla_decode_kernel_kind(const qkn_mla_dims* dims, int32_t num_splits, uint32_t flags) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits) return QKN_ERR_INVALID_ARG;
  if (flags & QKN_DECODE_FORCE_GENERIC) return 0;
  return qkn::mfma_decode_supported(*dims) ? 1 : 0;
}

int qkn_mla_absorb_query(const qkn_mla_dims* dims, const float* q, const float* q_rope,
                         const int32_t* q_pos, const float* w_k, const float* gamma_q,
                         const float* gamma_k, const float* gamma_qr, void* q_tilde,
                         float* alpha_q, void* q_rope_normed, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  const bool rope = dims->rope_dim > 0;
  if (!q || !q_pos || !w_k || !gamma_q || !gamma_k || !q_tilde || !alpha_q)
    return QKN_ERR_INVALID_ARG;
  if (rope && (!q_rope || !gamma_qr || !q_rope_normed)) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {q, q_pos, w_k, gamma_q, gamma_k, q_tilde, alpha_q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  if (rope && (!aligned16(q_rope) || !aligned16(gamma_qr) || !aligned16(q_rope_normed)))
    return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_absorb_query(*dims, q, q_rope, q_pos, w_k, gamma_q, gamma_k,
                                             gamma_qr, q_tilde, alpha_q, q_rope_normed,
                                             static_cast<hipStream_t>(stream)));
}

int qkn_mla_append(const qkn_mla_dims* dims, int32_t n_tokens, const float* c_new,
                   const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                   const int32_t* block_table, const float* w_k, const float* gamma_kr,
                   void* kv_cache, float* alpha_k_cache, int32_t* err_flag, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (n_tokens < 0) return QKN_ERR_INVALID_ARG;
  if (n_tokens == 0) return QKN_OK;
  const bool rope = dims->rope_dim > 0;
  if (!c_new || !seq_idx || !pos || !block_table || !w_k || !kv_cache || !alpha_k_cache)
    return QKN_ERR_INVALID_ARG;
  if (rope && (!k_rope_new || !gamma_kr)) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {c_new, seq_idx, pos, block_table, w_k, kv_cache, alpha_k_cache};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  if (rope && (!aligned16(k_rope_new) || !aligned16(gamma_kr))) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_append(*dims, n_tokens, c_new, k_rope_new, seq_idx, pos,
                                       block_table, w_k, gamma_kr, kv_cache, alpha_k_cache,
                                       err_flag, static_cast<hipStream_t>(stream)));
}

int qkn_mla_decode(const qkn_mla_dims* dims, const void* q_tilde, const float* alpha_q,
                   const void* q_rope_normed, const void* kv_cache,
                   const float* alpha_k_cache, const int32_t* block_table,
                   const int32_t* seq_lens, int32_t num_splits, uint32_t flags,
                   void* o_partial, float* lse_partial, int32_t* err_flag, void* stream) {
  int kind = qkn_mla_decode_kernel_kind(dims, num_splits, flags);
  if (kind < 0) return kind;
  if (flags & ~(QKN_DECODE_NO_ALPHA | QKN_DECODE_FORCE_GENERIC)) return QKN_ERR_INVALID_ARG;
  const bool rope = dims->rope_dim > 0;
  if (!q_tilde || !alpha_q || !kv_cache || !alpha_k_cache || !block_table || !seq_lens ||
      !o_partial || !lse_partial)
    return QKN_ERR_INVALID_ARG;
  if (rope && !q_rope_normed) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {q_tilde, alpha_q, kv_cache, alpha_k_cache, block_table, seq_lens,
                        o_partial, lse_partial};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  if (rope && !aligned16(q_rope_normed)) return QKN_ERR_ALIGNMENT;
  qkn::DecodeArgs a{q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache, block_table,
                    seq_lens, o_partial, lse_partial, err_flag, num_splits,
                    (flags & QKN_DECODE_NO_ALPHA) == 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(kind == 1 ? qkn::launch_decode_mfma(*dims, a, s)
                              : qkn::launch_decode_generic(*dims, a, s));
}

int qkn_mla_combine(const qkn_mla_dims* dims, int32_t num_splits, const void* o_partial,
                    const float* lse_partial, float* o_latent, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits) return QKN_ERR_INVALID_ARG;
  if (!o_partial || !lse_partial || !o_latent || !lse) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {o_partial, lse_partial, o_latent, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_combine(*dims, num_splits, o_partial, lse_partial, o_latent, lse,
                                        static_cast<hipStream_t>(stream)));
}

int qkn_mla_combine_project(const qkn_mla_dims* dims, int32_t num_splits, const void* o_partial,
                            const float* lse_partial, const float* w_v, float* o_latent,
                            float* lse, float* o, uint32_t flags, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits) return QKN_ERR_INVALID_ARG;
  if (flags & ~(QKN_PROJECT_FUSED | QKN_PROJECT_TWO_PASS)) return QKN_ERR_INVALID_ARG;
  if (!o_partial || !lse_partial || !w_v || !o_latent || !lse || !o) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {o_partial, lse_partial, w_v, o_latent, lse, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_combine_project(*dims, num_splits, o_partial, lse_partial, w_v,
                                                o_latent, lse, o, flags,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
