// qkn_mla_append: write new tokens into the paged latent cache (QK-Normed MLA
// summary, "Metodologia" items 2-4).  For each token: the latent c_t in the
// cache dtype, the RMS-normed and rotated RoPE key, and for every KV group g
// the inverse RMS alpha^k_{t,g} = 1/RMS(c_t W^K_g) of the projected key, which
// is formed in registers from the latent as stored and never written out.
//
// Grid: one block of 16 waves per (new token, KV group).  Every block forms
// its group's projected key and scalar; the group-0 block also stores the
// latent and the RoPE key.  W^K_g is read once per block in 16-byte pieces:
// thread t takes four columns (t mod d/4) of the key over every RG-th row of
// the latent (RG = 4096 / d row groups), with 16 rows in flight per thread, so
// that a wave's load covers whole rows.  The row groups' partial keys are
// then added in a fixed order, so the result does not depend on timing.
#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int WAVES = 16;
constexpr int UNROLL = 16;  // rows of W^K_g (16 bytes each) in flight per thread
constexpr int MAX_HEAD_DIM = 512;  // columns of W^K_g a block handles (the host checks head_dim)

template <typename CacheT>
__global__ __launch_bounds__(64 * WAVES) void append_kernel(
    const float* __restrict__ c_new, const float* __restrict__ k_rope_new,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_table, const float* __restrict__ w_k,
    const float* __restrict__ gamma_kr, CacheT* __restrict__ kv, float* __restrict__ alpha_k,
    int32_t* __restrict__ err_flag, int batch, int max_pages, int num_pages, int rank,
    int head_dim, int rope_dim, int groups, float eps, float theta) {
  extern __shared__ float cs[];                    // [rank] latent as stored, in float
  __shared__ float part[64 * WAVES * 4];           // [RG][head_dim] partial keys (RG * head_dim <= 4096)
  __shared__ float red[WAVES];
  __shared__ float xn[256];                        // normed RoPE key (d_R <= 256)
  __shared__ int slot_row;                         // page * 64 + row, or -1

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = blockIdx.x;
  const int g = blockIdx.y;

  // This thread's share of the projected key k[j] = sum_m c[m] W^K_g[m, j]:
  // four columns 4 c4 .. 4 c4 + 3 (one 16-byte load per row) over the rows
  // m = rg, rg + RG, ... of the latent (RG row groups).  The first UNROLL of
  // them are loaded before anything else, so that their latency overlaps the
  // page lookup and the latent load.
  const float* wg = w_k + (size_t)g * rank * head_dim;
  const int C4 = head_dim / 4;            // head_dim is a multiple of 4, <= 512
  const int RG = (64 * WAVES) / C4;       // >= 8
  const int c4 = tid % C4, rg = tid / C4;
  const bool proj = rg < RG;              // threads past RG * C4 have no share
  float4 wv[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int m = rg + RG * u;
    wv[u] = (proj && m < rank) ? *reinterpret_cast<const float4*>(wg + (size_t)m * head_dim + 4 * c4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // the RoPE key (wave 0 of the group-0 block): dims lane + 64 k (d_R <= 256)
  const bool rope_wave = g == 0 && wave == 0 && rope_dim > 0;
  float xr[4] = {};
  int xpos = 0;
  if (rope_wave) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (lane + 64 * k < rope_dim) xr[k] = k_rope_new[(size_t)n * rope_dim + lane + 64 * k];
    xpos = pos[n];
  }

  if (tid == 0) {
    int sr = -1;
    const int b = seq_idx[n], p = pos[n];
    if (b >= 0 && b < batch && p >= 0 && p < max_pages * QKN_MLA_PAGE_SIZE) {
      const int page = block_table[(size_t)b * max_pages + p / QKN_MLA_PAGE_SIZE];
      if (page >= 0 && page < num_pages) sr = page * QKN_MLA_PAGE_SIZE + p % QKN_MLA_PAGE_SIZE;
    }
    if (sr < 0 && err_flag && g == 0) atomicOr(err_flag, QKN_FLAG_INDEX);
    slot_row = sr;
  }
  // the latent rounded to the storage type (exact for a float cache)
  for (int m = tid; m < rank; m += 64 * WAVES) {
    float v = c_new[(size_t)n * rank + m];
    if (sizeof(CacheT) == 2) v = bf16_to_f32(f32_to_bf16(v));
    cs[m] = v;
  }
  __syncthreads();
  const int sr = slot_row;
  if (sr < 0) return;  // uniform: nothing is written for a rejected token

  // projected key of group g: this thread's rows, then the row groups' partial
  // keys in LDS
  if (proj) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int u0 = 0; rg + RG * u0 < rank; u0 += UNROLL) {
      if (u0 > 0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int m = rg + RG * (u0 + u);
          wv[u] = m < rank ? *reinterpret_cast<const float4*>(wg + (size_t)m * head_dim + 4 * c4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int m = rg + RG * (u0 + u);
        if (m < rank) {
          const float c = cs[m];
          acc.x = fmaf(c, wv[u].x, acc.x);
          acc.y = fmaf(c, wv[u].y, acc.y);
          acc.z = fmaf(c, wv[u].z, acc.z);
          acc.w = fmaf(c, wv[u].w, acc.w);
        }
      }
    }
    *reinterpret_cast<float4*>(&part[rg * head_dim + 4 * c4]) = acc;
  }

  // the latent as stored and the RoPE key (group-0 block), after the
  // projection so that the W^K_g registers are free
  const int row_stride = rank + rope_dim;
  if (g == 0) {
    for (int m = tid; m < rank; m += 64 * WAVES)
      Elem<CacheT>::store(kv, (size_t)sr * row_stride + m, cs[m]);
    // RoPE key: normalised over d_R, then rotated (dim d and d + d_R / 2
    // are paired, which the normed values reach through LDS)
    if (rope_wave) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) ss = fmaf(xr[k], xr[k], ss);
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)rope_dim + eps);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (lane + 64 * k < rope_dim) xn[lane + 64 * k] = xr[k] * inv * gamma_kr[lane + 64 * k];
      const int half = rope_dim / 2;
      CacheT* out = kv + (size_t)sr * row_stride + rank;
      for (int jj = lane; jj < half; jj += 64) {
        const float x1 = xn[jj], x2 = xn[jj + half];
        float c = 1.f, s = 0.f;
        if (theta != 0.f) rope_cos_sin<std::is_same<CacheT, float>::value>(xpos, jj, rope_dim, theta, &c, &s);
        Elem<CacheT>::store(out, jj, x1 * c - x2 * s);
        Elem<CacheT>::store(out, jj + half, x2 * c + x1 * s);
      }
    }
  }

  __syncthreads();
  float ss = 0.f;
  for (int j = tid; j < head_dim; j += 64 * WAVES) {
    float k = 0.f;
    for (int w = 0; w < RG; ++w) k += part[w * head_dim + j];
    ss = fmaf(k, k, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) tot += red[w];
    alpha_k[(size_t)sr * groups + g] = 1.0f / sqrtf(tot / (float)head_dim + eps);
  }
}

// The stores of the bulk path (bf16 cache): one wave per token for the slot,
// the latent (16-byte stores of 8 bf16 words) and the RoPE key, with the
// operations of append_kernel in the same order; alpha^k comes from
// append_alpha_mfma.
__global__ __launch_bounds__(256) void append_store_bulk(
    const float* __restrict__ c_new, const float* __restrict__ k_rope_new,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_table, const float* __restrict__ gamma_kr,
    uint16_t* __restrict__ kv, int32_t* __restrict__ err_flag, int n_tokens, int batch,
    int max_pages, int num_pages, int rank, int rope_dim, float eps, float theta) {
  __shared__ float xn_all[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + wave;
  if (n >= n_tokens) return;
  int sr = -1;
  const int b = seq_idx[n], p = pos[n];
  if (b >= 0 && b < batch && p >= 0 && p < max_pages * QKN_MLA_PAGE_SIZE) {
    const int page = block_table[(size_t)b * max_pages + p / QKN_MLA_PAGE_SIZE];
    if (page >= 0 && page < num_pages) sr = page * QKN_MLA_PAGE_SIZE + p % QKN_MLA_PAGE_SIZE;
  }
  if (sr < 0) {
    if (lane == 0 && err_flag) atomicOr(err_flag, QKN_FLAG_INDEX);
    return;
  }
  const int row_stride = rank + rope_dim;
  uint16_t* row = kv + (size_t)sr * row_stride;
  for (int m0 = 8 * lane; m0 < rank; m0 += 8 * 64) {
    const float4* src = reinterpret_cast<const float4*>(c_new + (size_t)n * rank + m0);
    const float4 a = src[0], c = src[1];
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    uint4 w;
    uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wp[j] = (uint32_t)f32_to_bf16(v[2 * j]) | ((uint32_t)f32_to_bf16(v[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(row + m0) = w;
  }
  if (rope_dim == 0) return;
  float xr[4] = {};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (lane + 64 * k < rope_dim) xr[k] = k_rope_new[(size_t)n * rope_dim + lane + 64 * k];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) ss = fmaf(xr[k], xr[k], ss);
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)rope_dim + eps);
  float* xn = xn_all[wave];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (lane + 64 * k < rope_dim) xn[lane + 64 * k] = xr[k] * inv * gamma_kr[lane + 64 * k];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const int half = rope_dim / 2;
  uint16_t* out = row + rank;
  for (int jj = lane; jj < half; jj += 64) {
    const float x1 = xn[jj], x2 = xn[jj + half];
    float c = 1.f, s = 0.f;
    if (theta != 0.f) rope_cos_sin<false>(p, jj, rope_dim, theta, &c, &s);
    out[jj] = f32_to_bf16(x1 * c - x2 * s);
    out[jj + half] = f32_to_bf16(x2 * c + x1 * s);
  }
}

template <typename CacheT>
hipError_t launch_typed(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                        const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                        const int32_t* block_table, const float* w_k, const float* gamma_kr,
                        void* kv_cache, float* alpha_k, int32_t* err_flag, hipStream_t s) {
  if (d.head_dim > MAX_HEAD_DIM || d.rope_dim > 256) return hipErrorInvalidValue;
  const size_t shmem = (size_t)d.rank * sizeof(float);
  if (n_tokens >= kBulkMinTokens && append_bulk_applies(d)) {
    // stores and flags per token, then alpha^k of all tokens on the matrix cores
    hipLaunchKernelGGL(append_store_bulk, dim3(cdiv(n_tokens, 4)), dim3(256), 0, s, c_new,
                       k_rope_new, seq_idx, pos, block_table, gamma_kr,
                       static_cast<uint16_t*>(kv_cache), err_flag, n_tokens, d.batch,
                       d.max_pages_per_seq, d.num_pages, d.rank, d.rope_dim, d.eps, d.rope_theta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_append_alpha_bulk(d, n_tokens, c_new, seq_idx, pos, block_table, w_k, alpha_k, s);
  }
  dim3 grid(n_tokens, d.groups);
  hipLaunchKernelGGL(append_kernel<CacheT>, grid, dim3(64 * WAVES), shmem, s, c_new,
                     k_rope_new, seq_idx, pos, block_table, w_k, gamma_kr,
                     static_cast<CacheT*>(kv_cache), alpha_k, err_flag, d.batch,
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
