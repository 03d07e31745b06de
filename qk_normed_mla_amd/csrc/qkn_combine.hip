// qkn_mla_combine: log-sum-exp merge of the split-KV partials.
//   M = max_p lse_p, lse = M + ln sum_p e^{lse_p - M}, o = sum_p e^{lse_p - lse} o_p
// The partials are half (bf16 cache) or float32 (float32 cache); every lane
// loads 16 bytes of a split's row at a time (8 or 4 latents) and accumulates
// in float32.  Each (query row, slice of 64 x 16 bytes of the latent) is served
// by a group of G waves, G = 1, 4, 8 or 16 by the split count (many splits:
// more waves, so that the loads of one row are spread; few: one wave, no
// exchange).
// Every wave forms M and lse over all splits (the lse_p are few bytes); wave k
// of a group then accumulates splits k, k + G, k + 2G, ... (eight splits'
// loads in flight at a time), and the group's first wave adds the G partial
// sums in wave order.  The sums are in a fixed order, so the result does not
// depend on timing.
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int kMaxWaves = 16;  // per block
constexpr int kBatch = 8;     // splits of one wave whose loads are in flight together

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// 16 bytes of partials as float32 values
template <typename PartT>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
};
template <>
struct Chunk<_Float16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const _Float16* p, float (&v)[8]) {
    const f16x8 x = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(x[j]);
  }
};

// group: waves per (row, slice); a block of blockDim.x / 64 waves holds
// blockDim.x / 64 / group of them
template <typename PartT>
__global__ __launch_bounds__(64 * kMaxWaves) void combine_kernel(const PartT* __restrict__ o_part,
                                                                 const float* __restrict__ lse_part,
                                                                 float* __restrict__ o_lat,
                                                                 float* __restrict__ lse_out,
                                                                 int n_rows, int num_splits,
                                                                 int rank, int group) {
  constexpr int N = Chunk<PartT>::N;  // latents per lane
  constexpr int kSlice = 64 * N;
  __shared__ float4 part[kMaxWaves][N / 4][64];
  const int slices = cdiv(rank, kSlice);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = wave % group;  // wave of the group
  const int unit = blockIdx.x * ((int)(blockDim.x >> 6) / group) + wave / group;
  if (unit >= n_rows * slices) return;  // whole groups; a group with work never waits on one without
  const int row = unit / slices, slice = unit % slices;
  const int m0 = slice * kSlice + lane * N;
  const float* lp = lse_part + (size_t)row * num_splits;
  const bool live = m0 < rank;  // rank is a multiple of 8

  // the lse_p of the row, four loads per lane in flight at a time
  float M = -INFINITY;
  for (int p0 = lane; p0 < num_splits; p0 += 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = p0 + 64 * u < num_splits ? lp[p0 + 64 * u] : -INFINITY;
    M = fmaxf(M, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  }
  M = wave_max(M);
  float* out = o_lat + (size_t)row * rank + m0;
  const bool empty = M == -INFINITY;  // every split empty (uniform over the group)
  if (empty) {
    if (sub == 0 && live) {
#pragma unroll
      for (int j = 0; j < N; j += 4) *reinterpret_cast<float4*>(out + j) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (sub == 0 && lane == 0 && slice == 0) lse_out[row] = -INFINITY;
    if (group == 1) return;
  }
  float s = 0.f;
  for (int p0 = lane; p0 < num_splits; p0 += 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = p0 + 64 * u < num_splits ? lp[p0 + 64 * u] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) s += expf(x[u] - M);
  }
  s = wave_sum(s);
  const float lse = M + logf(s);
  if (!empty && sub == 0 && lane == 0 && slice == 0) lse_out[row] = lse;

  const PartT* op = o_part + (size_t)row * num_splits * rank + m0;
  float acc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) acc[j] = 0.f;
  for (int p0 = empty ? num_splits : sub; p0 < num_splits; p0 += group * kBatch) {
    float v[kBatch][N];
    float l[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + group * u;
      l[u] = p < num_splits ? lp[p] : -INFINITY;
      if (p < num_splits && live) {
        Chunk<PartT>::load(op + (size_t)p * rank, v[u]);
      } else {
#pragma unroll
        for (int j = 0; j < N; ++j) v[u][j] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (l[u] == -INFINITY) continue;  // empty split
      const float w = expf(l[u] - lse);
#pragma unroll
      for (int j = 0; j < N; ++j) acc[j] = fmaf(w, v[u][j], acc[j]);
    }
  }
  if (group == 1) {
    if (live) {
#pragma unroll
      for (int j = 0; j < N; j += 4)
        *reinterpret_cast<float4*>(out + j) = make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < N; j += 4) part[wave][j / 4][lane] = make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
  __syncthreads();
  if (sub == 0 && live && !empty) {
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      float4 o = part[wave][j][lane];
      for (int w = 1; w < group; ++w) {
        const float4 t = part[wave + w][j][lane];
        o.x += t.x;
        o.y += t.y;
        o.z += t.z;
        o.w += t.w;
      }
      *reinterpret_cast<float4*>(out + 4 * j) = o;
    }
  }
}

}  // namespace

hipError_t launch_combine_rows(int n_rows, int num_splits, int row_len, bool half_parts,
                               const void* o_part, const float* lse_part, float* o, float* lse,
                               hipStream_t s) {
  const int group = num_splits <= 16 ? 1 : num_splits <= 64 ? 4 : num_splits <= 128 ? 8 : 16;
  const int waves = group < 4 ? 4 : group;  // per block
  const int per_block = waves / group;
  if (half_parts) {
    const int units = n_rows * cdiv(row_len, 64 * Chunk<_Float16>::N);
    hipLaunchKernelGGL(combine_kernel<_Float16>, dim3(cdiv(units, per_block)), dim3(64 * waves), 0,
                       s, static_cast<const _Float16*>(o_part), lse_part, o, lse, n_rows,
                       num_splits, row_len, group);
  } else {
    const int units = n_rows * cdiv(row_len, 64 * Chunk<float>::N);
    hipLaunchKernelGGL(combine_kernel<float>, dim3(cdiv(units, per_block)), dim3(64 * waves), 0, s,
                       static_cast<const float*>(o_part), lse_part, o, lse, n_rows, num_splits,
                       row_len, group);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const qkn_mla_dims& d, int num_splits, const void* o_part,
                          const float* lse_part, float* o_lat, float* lse, hipStream_t s) {
  return launch_combine_rows(d.batch * d.s_q * d.heads, num_splits, d.rank,
                             d.cache_dtype == QKN_BF16, o_part, lse_part, o_lat, lse, s);
}

}  // namespace qkn
