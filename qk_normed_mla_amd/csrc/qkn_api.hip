// extern "C" entry points of libqknmla.so: host-side validation, then launch.
// Every check runs before any HIP call, so a rejected call touches no device.
#include <cmath>
#include <cstdint>
#include <mutex>
#include <utility>
#include <vector>

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

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// The partials of one qkn_mla_decode_attend call inside its workspace:
// o_partial at 0, lse_partial at lse_offset, both on 256-byte boundaries.
struct WorkspaceLayout {
  size_t lse_offset, total;
};
WorkspaceLayout workspace_layout(const qkn_mla_dims& d, int num_splits) {
  const size_t rows = (size_t)d.batch * d.s_q * d.heads * num_splits;
  const size_t elem = d.cache_dtype == QKN_BF16 ? 2 : 4;  // the partial dtype
  WorkspaceLayout w;
  w.lse_offset = round256(rows * d.rank * elem);
  w.total = w.lse_offset + round256(rows * 4);
  return w;
}

// The split partials of one qkn_mla_gqa_attend call inside its workspace: half
// o_partial [rows, P, d] at 0, float32 lse_partial [rows, P] at lse_offset.
WorkspaceLayout gqa_workspace_layout(const qkn_mla_dims& d, int num_splits) {
  const size_t rows = (size_t)d.batch * d.s_q * d.heads * num_splits;
  WorkspaceLayout w;
  w.lse_offset = round256(rows * d.head_dim * 2);
  w.total = w.lse_offset + round256(rows * 4);
  return w;
}

// Checks of qkn_mla_decode's arguments (not the partials); returns the kernel
// kind (0 generic, 1 matrix cores) or a negative status.
int check_decode_args(const qkn_mla_dims* dims, const void* q_tilde, const float* alpha_q,
                      const void* q_rope_normed, const void* kv_cache,
                      const float* alpha_k_cache, const int32_t* block_table,
                      const int32_t* seq_lens, int32_t num_splits, uint32_t flags) {
  int kind = qkn_mla_decode_kernel_kind(dims, num_splits, flags);
  if (kind < 0) return kind;
  if (flags & ~(QKN_DECODE_NO_ALPHA | QKN_DECODE_FORCE_GENERIC)) return QKN_ERR_INVALID_ARG;
  const bool rope = dims->rope_dim > 0;
  if (!q_tilde || !alpha_q || !kv_cache || !alpha_k_cache || !block_table || !seq_lens)
    return QKN_ERR_INVALID_ARG;
  if (rope && !q_rope_normed) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {q_tilde, alpha_q, kv_cache, alpha_k_cache, block_table, seq_lens};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  if (rope && !aligned16(q_rope_normed)) return QKN_ERR_ALIGNMENT;
  return kind;
}

hipError_t launch_decode(int kind, const qkn_mla_dims& d, const qkn::DecodeArgs& a,
                         hipStream_t s) {
  return kind == 1 ? qkn::launch_decode_mfma(d, a, s) : qkn::launch_decode_generic(d, a, s);
}

// Decode into the partials laid out in `ws` (workspace_layout), then combine.
int attend_in(int kind, const qkn_mla_dims& d, const void* q_tilde, const float* alpha_q,
              const void* q_rope_normed, const void* kv_cache, const float* alpha_k_cache,
              const int32_t* block_table, const int32_t* seq_lens, int32_t num_splits,
              uint32_t flags, void* ws, float* o_latent, float* lse, int32_t* err_flag,
              hipStream_t s) {
  const WorkspaceLayout w = workspace_layout(d, num_splits);
  void* o_partial = ws;
  float* lse_partial = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + w.lse_offset);
  qkn::DecodeArgs a{q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache, block_table,
                    seq_lens, o_partial, lse_partial, err_flag, num_splits,
                    (flags & QKN_DECODE_NO_ALPHA) == 0};
  if (launch_decode(kind, d, a, s) != hipSuccess) return QKN_ERR_HIP;
  return hip_status(qkn::launch_combine(d, num_splits, o_partial, lse_partial, o_latent, lse, s));
}

}  // namespace

namespace qkn {

hipError_t set_lds_limit_once(const void* fn, int bytes) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;  // (kernel, device)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& k : done)
    if (k.first == fn && k.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(fn, dev);
  return e;
}

}  // namespace qkn

extern "C" {

int qkn_mla_abi_version(void) { return QKN_MLA_ABI_VERSION; }

const char* qkn_status_string(int status) {
  switch (status) {
    case QKN_OK: return "ok";
    case QKN_ERR_INVALID_ARG: return "invalid argument (null pointer or inconsistent size)";
    case QKN_ERR_UNSUPPORTED: return "unsupported size for these kernels";
    case QKN_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case QKN_ERR_HIP: return "HIP runtime error on launch";
    case QKN_ERR_SCRATCH:
      return "request exceeds the static scratch of qkn_mla_decode_attend_noalloc "
             "(QKN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int qkn_mla_check_dims(const qkn_mla_dims* dims) { return check_dims(dims); }

int qkn_mla_partial_dtype(const qkn_mla_dims* dims) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  return dims->cache_dtype == QKN_BF16 ? QKN_F16 : QKN_F32;
}

size_t qkn_mla_decode_workspace_bytes(const qkn_mla_dims* dims, int32_t num_splits) {
  if (check_dims(dims) != QKN_OK || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return workspace_layout(*dims, num_splits).total;
}

int qkn_mla_decode_kernel_kind(const qkn_mla_dims* dims, int32_t num_splits, uint32_t flags) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits) return QKN_ERR_INVALID_ARG;
  if (flags & QKN_DECODE_FORCE_GENERIC) return 0;
  return qkn::mfma_decode_supported(*dims) ? 1 : 0;
}

namespace {
int check_absorb_args(const qkn_mla_dims* dims, const float* q, const float* q_rope,
                      const int32_t* q_pos, const float* w_k, const float* gamma_q,
                      const float* gamma_k, const float* gamma_qr, const void* q_tilde,
                      const float* alpha_q, const void* q_rope_normed) {
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
  return QKN_OK;
}

// n_tokens > 0 here
int check_append_args(const qkn_mla_dims* dims, const float* c_new, const float* k_rope_new,
                      const int32_t* seq_idx, const int32_t* pos, const int32_t* block_table,
                      const float* w_k, const float* gamma_kr, const void* kv_cache,
                      const float* alpha_k_cache) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  const bool rope = dims->rope_dim > 0;
  if (!c_new || !seq_idx || !pos || !block_table || !w_k || !kv_cache || !alpha_k_cache)
    return QKN_ERR_INVALID_ARG;
  if (rope && (!k_rope_new || !gamma_kr)) return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {c_new, seq_idx, pos, block_table, w_k, kv_cache, alpha_k_cache};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  if (rope && (!aligned16(k_rope_new) || !aligned16(gamma_kr))) return QKN_ERR_ALIGNMENT;
  return QKN_OK;
}
}  // namespace

int qkn_mla_absorb_query(const qkn_mla_dims* dims, const float* q, const float* q_rope,
                         const int32_t* q_pos, const float* w_k, const float* gamma_q,
                         const float* gamma_k, const float* gamma_qr, void* q_tilde,
                         float* alpha_q, void* q_rope_normed, void* stream) {
  const int st = check_absorb_args(dims, q, q_rope, q_pos, w_k, gamma_q, gamma_k, gamma_qr,
                                   q_tilde, alpha_q, q_rope_normed);
  if (st != QKN_OK) return st;
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
  st = check_append_args(dims, c_new, k_rope_new, seq_idx, pos, block_table, w_k, gamma_kr,
                         kv_cache, alpha_k_cache);
  if (st != QKN_OK) return st;
  return hip_status(qkn::launch_append(*dims, n_tokens, c_new, k_rope_new, seq_idx, pos,
                                       block_table, w_k, gamma_kr, kv_cache, alpha_k_cache,
                                       err_flag, static_cast<hipStream_t>(stream)));
}

int qkn_mla_decode(const qkn_mla_dims* dims, const void* q_tilde, const float* alpha_q,
                   const void* q_rope_normed, const void* kv_cache,
                   const float* alpha_k_cache, const int32_t* block_table,
                   const int32_t* seq_lens, int32_t num_splits, uint32_t flags,
                   void* o_partial, float* lse_partial, int32_t* err_flag, void* stream) {
  const int kind = check_decode_args(dims, q_tilde, alpha_q, q_rope_normed, kv_cache,
                                     alpha_k_cache, block_table, seq_lens, num_splits, flags);
  if (kind < 0) return kind;
  if (!o_partial || !lse_partial) return QKN_ERR_INVALID_ARG;
  if (!aligned16(o_partial) || !aligned16(lse_partial)) return QKN_ERR_ALIGNMENT;
  qkn::DecodeArgs a{q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache, block_table,
                    seq_lens, o_partial, lse_partial, err_flag, num_splits,
                    (flags & QKN_DECODE_NO_ALPHA) == 0};
  return hip_status(launch_decode(kind, *dims, a, static_cast<hipStream_t>(stream)));
}

int qkn_mla_decode_sparse(const qkn_mla_dims* dims, const void* q_tilde, const float* alpha_q,
                          const void* q_rope_normed, const void* kv_cache,
                          const float* alpha_k_cache, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* indices, int32_t index_len,
                          int32_t num_splits, uint32_t flags, void* o_partial,
                          float* lse_partial, int32_t* err_flag, void* stream) {
  if (flags & QKN_DECODE_FORCE_GENERIC) return QKN_ERR_UNSUPPORTED;
  const int kind = check_decode_args(dims, q_tilde, alpha_q, q_rope_normed, kv_cache,
                                     alpha_k_cache, block_table, seq_lens, num_splits, flags);
  if (kind < 0) return kind;
  if (index_len < 0) return QKN_ERR_INVALID_ARG;
  if (!o_partial || !lse_partial || (index_len > 0 && !indices)) return QKN_ERR_INVALID_ARG;
  if (!aligned16(o_partial) || !aligned16(lse_partial)) return QKN_ERR_ALIGNMENT;
  if (index_len > 0 && !aligned16(indices)) return QKN_ERR_ALIGNMENT;
  const int chk = qkn::sparse_decode_check(*dims, index_len, num_splits);
  if (chk != 0) return chk == -1 ? QKN_ERR_INVALID_ARG : QKN_ERR_UNSUPPORTED;
  qkn::DecodeArgs a{q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache, block_table,
                    seq_lens, o_partial, lse_partial, err_flag, num_splits,
                    (flags & QKN_DECODE_NO_ALPHA) == 0, indices, index_len};
  return hip_status(qkn::launch_decode_sparse(*dims, a, static_cast<hipStream_t>(stream)));
}

int qkn_mla_prefill_query(const qkn_mla_dims* dims, const float* q, const float* q_rope,
                          const int32_t* q_pos, const float* gamma_q, const float* gamma_qr,
                          void* q_hat, void* q_rope_normed, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (!qkn::prefill_supported(*dims)) return QKN_ERR_UNSUPPORTED;
  if (!q || !q_rope || !q_pos || !gamma_q || !gamma_qr || !q_hat || !q_rope_normed)
    return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {q, q_rope, q_pos, gamma_q, gamma_qr, q_hat, q_rope_normed};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_prefill_query(*dims, q, q_rope, q_pos, gamma_q, gamma_qr, q_hat,
                                              q_rope_normed, static_cast<hipStream_t>(stream)));
}

int qkn_mla_prefill_expand(const qkn_mla_dims* dims, const void* kv_cache,
                           const float* alpha_k_cache, const int32_t* block_table,
                           const int32_t* seq_lens, const float* w_k, const float* w_v,
                           const float* gamma_k, void* k_hat, void* v, int32_t* err_flag,
                           void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (!qkn::prefill_supported(*dims)) return QKN_ERR_UNSUPPORTED;
  if (!kv_cache || !alpha_k_cache || !block_table || !seq_lens || !w_k || !w_v || !gamma_k ||
      !k_hat || !v)
    return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {kv_cache, alpha_k_cache, block_table, seq_lens, w_k, w_v, gamma_k, k_hat, v};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_prefill_expand(*dims, kv_cache, alpha_k_cache, block_table,
                                               seq_lens, w_k, w_v, gamma_k, k_hat, v, err_flag,
                                               static_cast<hipStream_t>(stream)));
}

int qkn_mla_prefill_attend(const qkn_mla_dims* dims, const void* q_hat, const void* q_rope_normed,
                           const void* k_hat, const void* v, const void* kv_cache,
                           const int32_t* block_table, const int32_t* seq_lens, float* o,
                           float* lse, int32_t* err_flag, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (!qkn::prefill_supported(*dims)) return QKN_ERR_UNSUPPORTED;
  if (!q_hat || !q_rope_normed || !k_hat || !v || !kv_cache || !block_table || !seq_lens || !o ||
      !lse)
    return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {q_hat, q_rope_normed, k_hat, v, kv_cache, block_table, seq_lens, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_prefill_attend(*dims, q_hat, q_rope_normed, k_hat, v, kv_cache,
                                               block_table, seq_lens, o, lse, err_flag,
                                               static_cast<hipStream_t>(stream)));
}

int qkn_mla_decode_attend(const qkn_mla_dims* dims, const void* q_tilde, const float* alpha_q,
                          const void* q_rope_normed, const void* kv_cache,
                          const float* alpha_k_cache, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t num_splits, uint32_t flags,
                          void* workspace, size_t workspace_bytes, float* o_latent, float* lse,
                          int32_t* err_flag, void* stream) {
  const int kind = check_decode_args(dims, q_tilde, alpha_q, q_rope_normed, kv_cache,
                                     alpha_k_cache, block_table, seq_lens, num_splits, flags);
  if (kind < 0) return kind;
  if (!workspace || !o_latent || !lse) return QKN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QKN_ERR_ALIGNMENT;
  if (!aligned16(o_latent) || !aligned16(lse)) return QKN_ERR_ALIGNMENT;
  if (workspace_bytes < workspace_layout(*dims, num_splits).total) return QKN_ERR_INVALID_ARG;
  return attend_in(kind, *dims, q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache,
                   block_table, seq_lens, num_splits, flags, workspace, o_latent, lse, err_flag,
                   static_cast<hipStream_t>(stream));
}

int qkn_mla_decode_attend_noalloc(const qkn_mla_dims* dims, const void* q_tilde,
                                  const float* alpha_q, const void* q_rope_normed,
                                  const void* kv_cache, const float* alpha_k_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t num_splits, uint32_t flags, float* o_latent,
                                  float* lse, int32_t* err_flag, void* stream) {
  const int kind = check_decode_args(dims, q_tilde, alpha_q, q_rope_normed, kv_cache,
                                     alpha_k_cache, block_table, seq_lens, num_splits, flags);
  if (kind < 0) return kind;
  if (!o_latent || !lse) return QKN_ERR_INVALID_ARG;
  if (!aligned16(o_latent) || !aligned16(lse)) return QKN_ERR_ALIGNMENT;
  if (workspace_layout(*dims, num_splits).total > QKN_NOALLOC_SCRATCH_BYTES) return QKN_ERR_SCRATCH;
  void* scratch = nullptr;
  if (qkn::noalloc_scratch(&scratch) != hipSuccess || !scratch) return QKN_ERR_HIP;
  return attend_in(kind, *dims, q_tilde, alpha_q, q_rope_normed, kv_cache, alpha_k_cache,
                   block_table, seq_lens, num_splits, flags, scratch, o_latent, lse, err_flag,
                   static_cast<hipStream_t>(stream));
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

int qkn_mla_stream_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0) return QKN_ERR_INVALID_ARG;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_stream_read(src, static_cast<size_t>(bytes), sink,
                                            static_cast<hipStream_t>(stream)));
}

size_t qkn_mla_gqa_workspace_bytes(const qkn_mla_dims* dims, int32_t num_splits) {
  if (check_dims(dims) != QKN_OK || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return gqa_workspace_layout(*dims, num_splits).total;
}

int qkn_mla_gqa_append(const qkn_mla_dims* dims, int32_t n_tokens, const float* c_new,
                       const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                       const int32_t* block_table, const float* w_k, const float* w_v,
                       const float* gamma_k, const float* gamma_kr, void* kvg_cache,
                       int32_t* err_flag, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (!qkn::gqa_supported(*dims)) return QKN_ERR_UNSUPPORTED;
  if (n_tokens < 0) return QKN_ERR_INVALID_ARG;
  if (n_tokens == 0) return QKN_OK;
  if (!c_new || !k_rope_new || !seq_idx || !pos || !block_table || !w_k || !w_v || !gamma_k ||
      !gamma_kr || !kvg_cache)
    return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {c_new, k_rope_new, seq_idx, pos, block_table, w_k, w_v, gamma_k, gamma_kr,
                        kvg_cache};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  return hip_status(qkn::launch_gqa_append(*dims, n_tokens, c_new, k_rope_new, seq_idx, pos,
                                           block_table, w_k, w_v, gamma_k, gamma_kr, kvg_cache,
                                           err_flag, static_cast<hipStream_t>(stream)));
}

int qkn_mla_gqa_attend(const qkn_mla_dims* dims, const void* q_hat, const void* q_rope_normed,
                       const void* kvg_cache, const int32_t* block_table, const int32_t* seq_lens,
                       int32_t num_splits, void* workspace, size_t workspace_bytes, float* o,
                       float* lse, int32_t* err_flag, void* stream) {
  int st = check_dims(dims);
  if (st != QKN_OK) return st;
  if (!qkn::gqa_supported(*dims)) return QKN_ERR_UNSUPPORTED;
  if (num_splits < 1 || num_splits > kMaxSplits) return QKN_ERR_INVALID_ARG;
  // workgroups: (sequence, split) pairs padded to a multiple of 8, times the
  // token and head blocks of a pair (at most ceil(s_q / 4) x heads / 32)
  const int64_t pairs = ((int64_t)dims->batch * num_splits + 7) / 8 * 8;
  const int64_t blocks = pairs * ((dims->s_q + 3) / 4) * (dims->heads / 32);
  if (blocks > INT32_MAX) return QKN_ERR_INVALID_ARG;
  if (!q_hat || !q_rope_normed || !kvg_cache || !block_table || !seq_lens || !o || !lse)
    return QKN_ERR_INVALID_ARG;
  const void* ptrs[] = {q_hat, q_rope_normed, kvg_cache, block_table, seq_lens, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QKN_ERR_ALIGNMENT;
  void* o_part = nullptr;
  float* lse_part = nullptr;
  if (num_splits > 1) {
    const WorkspaceLayout w = gqa_workspace_layout(*dims, num_splits);
    if (!workspace || workspace_bytes < w.total) return QKN_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QKN_ERR_ALIGNMENT;
    o_part = workspace;
    lse_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + w.lse_offset);
  }
  return hip_status(qkn::launch_gqa_attend(*dims, q_hat, q_rope_normed, kvg_cache, block_table,
                                           seq_lens, num_splits, o_part, lse_part, o, lse, err_flag,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"
