// qkn_mla_append: write new tokens into the paged latent cache (QK-Normed MLA
// summary, "Metodologia" items 2-4).  For each token: the latent c_t in the
// cache dtype, the RMS-normed and rotated RoPE key, and for every KV group g
// the inverse RMS alpha^k_{t,g} = 1/RMS(c_t W^K_g) of the projected key, which
// is formed in registers from the latent as stored and never written out.
//
// Grid: (token tiles of 16, G).  Every block computes the scalars of its group;
// the group-0 blocks also store the latent and the RoPE key.
#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int TT = 16;  // tokens per block

template <typename CacheT>
__global__ __launch_bounds__(256) void append_kernel(
    int n_tokens, const float* __restrict__ c_new, const float* __restrict__ k_rope_new,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_table, const float* __restrict__ w_k,
    const float* __restrict__ gamma_kr, CacheT* __restrict__ kv, float* __restrict__ alpha_k,
    int32_t* __restrict__ err_flag, int batch, int max_pages, int num_pages, int rank,
    int head_dim, int rope_dim, int groups, float eps, float theta) {
  extern __shared__ float smem[];
  float* cs = smem;                       // [TT][rank]   latent as stored, in float
  __shared__ int slot_row[TT];            // page * 64 + row, or -1
  __shared__ float red[2][4][TT / 2];     // per-wave partial sums of k^2

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int t0 = blockIdx.x * TT;

  if (tid < TT) {
    int n = t0 + tid;
    int sr = -1;
    if (n < n_tokens) {
      int b = seq_idx[n], p = pos[n];
      if (b >= 0 && b < batch && p >= 0 && p < max_pages * QKN_MLA_PAGE_SIZE) {
        int page = block_table[(size_t)b * max_pages + p / QKN_MLA_PAGE_SIZE];
        if (page >= 0 && page < num_pages) sr = page * QKN_MLA_PAGE_SIZE + p % QKN_MLA_PAGE_SIZE;
      }
      if (sr < 0 && err_flag && g == 0) atomicOr(err_flag, 1);
    }
    slot_row[tid] = sr;
  }
  // stage the latents, rounded to the storage type (exact for a float cache)
  for (int e = tid; e < TT * rank; e += 256) {
    int t = e / rank, m = e % rank;
    int n = t0 + t;
    float v = 0.f;
    if (n < n_tokens) {
      v = c_new[(size_t)n * rank + m];
      if (sizeof(CacheT) == 2) v = bf16_to_f32(f32_to_bf16(v));
    }
    cs[t * rank + m] = v;
  }
  __syncthreads();

  const int row_stride = rank + rope_dim;
  if (g == 0) {
    for (int e = tid; e < TT * rank; e += 256) {
      int t = e / rank, m = e % rank;
      int sr = slot_row[t];
      if (sr >= 0) Elem<CacheT>::store(kv, (size_t)sr * row_stride + m, cs[t * rank + m]);
    }
    // RoPE key: one wave per token, normalised over d_R then rotated
    const int wave = tid >> 6, lane = tid & 63;
    for (int t = wave; t < TT && rope_dim > 0; t += 4) {
      int sr = slot_row[t];
      if (sr < 0) continue;
      const int n = t0 + t;
      const float* x = k_rope_new + (size_t)n * rope_dim;
      float ss = 0.f;
      for (int j = lane; j < rope_dim; j += 64) ss = fmaf(x[j], x[j], ss);
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)rope_dim + eps);
      const int half = rope_dim / 2;
      const int p = pos[n];
      CacheT* out = kv + (size_t)sr * row_stride + rank;
      for (int j = lane; j < half; j += 64) {
        float x1 = x[j] * inv * gamma_kr[j];
        float x2 = x[j + half] * inv * gamma_kr[j + half];
        float c = 1.f, s = 0.f;
        if (theta != 0.f) rope_cos_sin(p, j, rope_dim, theta, &c, &s);
        Elem<CacheT>::store(out, j, x1 * c - x2 * s);
        Elem<CacheT>::store(out, j + half, x2 * c + x1 * s);
      }
    }
  }

  // projected key of group g, k[t, j] = sum_m c[t, m] W^K_g[m, j]; only its
  // sum of squares is kept.  Threads 0-127 take tokens 0-7, 128-255 tokens 8-15.
  const int half_id = tid >> 7;
  const int jl = tid & 127;
  const float* wg = w_k + (size_t)g * rank * head_dim;
  float ss[TT / 2] = {};
  for (int j = jl; j < head_dim; j += 128) {
    float acc[TT / 2] = {};
    for (int m = 0; m < rank; ++m) {
      float w = wg[(size_t)m * head_dim + j];
#pragma unroll
      for (int u = 0; u < TT / 2; ++u) acc[u] = fmaf(cs[(half_id * (TT / 2) + u) * rank + m], w, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < TT / 2; ++u) ss[u] = fmaf(acc[u], acc[u], ss[u]);
  }
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < TT / 2; ++u) {
    float v = wave_sum(ss[u]);
    if (lane == 0) red[half_id][wave & 1][u] = v;
  }
  __syncthreads();
  if (tid < TT) {
    int h = tid / (TT / 2), u = tid % (TT / 2);
    int sr = slot_row[tid];
    if (sr >= 0) {
      float tot = red[h][0][u] + red[h][1][u];
      alpha_k[(size_t)sr * groups + g] = 1.0f / sqrtf(tot / (float)head_dim + eps);
    }
  }
}

template <typename CacheT>
hipError_t launch_typed(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                        const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                        const int32_t* block_table, const float* w_k, const float* gamma_kr,
                        void* kv_cache, float* alpha_k_cache, int32_t* err_flag, hipStream_t s) {
  dim3 grid(cdiv(n_tokens, TT), d.groups);
  size_t shmem = (size_t)TT * d.rank * sizeof(float);
  hipLaunchKernelGGL(append_kernel<CacheT>, grid, dim3(256), shmem, s, n_tokens, c_new,
                     k_rope_new, seq_idx, pos, block_table, w_k, gamma_kr,
                     static_cast<CacheT*>(kv_cache), alpha_k_cache, err_flag, d.batch,
                     d.max_pages_per_seq, d.num_pages, d.rank, d.head_dim, d.rope_dim, d.groups,
                     d.eps, d.rope_theta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                         const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                         const int32_t* block_table, const float* w_k, const float* gamma_kr,
                         void* kv_cache, float* alpha_k_cache, int32_t* err_flag, hipStream_t s) {
  if (d.cache_dtype == QKN_BF16)
    return launch_typed<uint16_t>(d, n_tokens, c_new, k_rope_new, seq_idx, pos, block_table, w_k,
                                  gamma_kr, kv_cache, alpha_k_cache, err_flag, s);
  return launch_typed<float>(d, n_tokens, c_new, k_rope_new, seq_idx, pos, block_table, w_k,
                             gamma_kr, kv_cache, alpha_k_cache, err_flag, s);
}

}  // namespace qkn
