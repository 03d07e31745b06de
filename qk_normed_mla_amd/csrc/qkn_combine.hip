// qkn_mla_combine: log-sum-exp merge of the split-KV partials.
//   M = max_p lse_p, lse = M + ln sum_p e^{lse_p - M}, o = sum_p e^{lse_p - lse} o_p
// Each (query row, 256-float slice of the latent) is served by a group of G
// waves, G = 1, 4 or 8 by the split count (many splits: more waves, so that
// the loads of one row are spread; few: one wave, no exchange).  Every wave
// forms M and lse over all splits (the lse_p are few bytes); wave k of a group
// then accumulates splits k, k + G, k + 2G, ... with each lane owning four
// consecutive latent floats (16-byte loads, eight splits' loads in flight at a
// time), and the group's first wave adds the G partial sums in wave order.
// The sums are in a fixed order, so the result does not depend on timing.
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int kSlice = 256;
constexpr int kMaxWaves = 8;  // per block
constexpr int kBatch = 8;     // splits of one wave whose loads are in flight together

// group: waves per (row, slice); a block of blockDim.x / 64 waves holds
// blockDim.x / 64 / group of them
__global__ __launch_bounds__(64 * kMaxWaves) void combine_kernel(const float* __restrict__ o_part,
                                                                 const float* __restrict__ lse_part,
                                                                 float* __restrict__ o_lat,
                                                                 float* __restrict__ lse_out,
                                                                 int n_rows, int num_splits,
                                                                 int rank, int group) {
  __shared__ float4 part[kMaxWaves][64];
  const int slices = cdiv(rank, kSlice);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = wave % group;  // wave of the group
  const int unit = blockIdx.x * ((int)(blockDim.x >> 6) / group) + wave / group;
  if (unit >= n_rows * slices) return;  // whole groups; a group with work never waits on one without
  const int row = unit / slices, slice = unit % slices;
  const int m0 = slice * kSlice + lane * 4;
  const float* lp = lse_part + (size_t)row * num_splits;

  float M = -INFINITY;
  for (int p = lane; p < num_splits; p += 64) M = fmaxf(M, lp[p]);
  M = wave_max(M);
  float* out = o_lat + (size_t)row * rank;
  const bool empty = M == -INFINITY;  // every split empty (uniform over the group)
  if (empty) {
    if (sub == 0 && m0 < rank) *reinterpret_cast<float4*>(out + m0) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (sub == 0 && lane == 0 && slice == 0) lse_out[row] = -INFINITY;
    if (group == 1) return;
  }
  float s = 0.f;
  for (int p = lane; p < num_splits; p += 64) s += expf(lp[p] - M);
  s = wave_sum(s);
  const float lse = M + logf(s);
  if (!empty && sub == 0 && lane == 0 && slice == 0) lse_out[row] = lse;

  const float* op = o_part + (size_t)row * num_splits * rank + m0;
  const bool live = m0 < rank;  // rank is a multiple of 8
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = empty ? num_splits : sub; p0 < num_splits; p0 += group * kBatch) {
    float4 v[kBatch];
    float l[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + group * u;
      l[u] = p < num_splits ? lp[p] : -INFINITY;
      v[u] = (p < num_splits && live) ? *reinterpret_cast<const float4*>(op + (size_t)p * rank)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (l[u] == -INFINITY) continue;  // empty split
      const float w = expf(l[u] - lse);
      acc.x = fmaf(w, v[u].x, acc.x);
      acc.y = fmaf(w, v[u].y, acc.y);
      acc.z = fmaf(w, v[u].z, acc.z);
      acc.w = fmaf(w, v[u].w, acc.w);
    }
  }
  if (group == 1) {
    if (live) *reinterpret_cast<float4*>(out + m0) = acc;
    return;
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (sub == 0 && live && !empty) {
    float4 o = part[wave][lane];
    for (int w = 1; w < group; ++w) {
      const float4 t = part[wave + w][lane];
      o.x += t.x;
      o.y += t.y;
      o.z += t.z;
      o.w += t.w;
    }
    *reinterpret_cast<float4*>(out + m0) = o;
  }
}

}  // namespace

hipError_t launch_combine(const qkn_mla_dims& d, int num_splits, const float* o_part,
                          const float* lse_part, float* o_lat, float* lse, hipStream_t s) {
  const int n_rows = d.batch * d.s_q * d.heads;
  const int units = n_rows * cdiv(d.rank, kSlice);
  const int group = num_splits <= 16 ? 1 : num_splits <= 64 ? 4 : 8;
  const int waves = group == 8 ? 8 : 4;  // per block
  const int per_block = waves / group;
  hipLaunchKernelGGL(combine_kernel, dim3(cdiv(units, per_block)), dim3(64 * waves), 0, s, o_part,
                     lse_part, o_lat, lse, n_rows, num_splits, d.rank, group);
  return hipGetLastError();
}

}  // namespace qkn
