// qkn_mla_combine: log-sum-exp merge of the split-KV partials.
//   M = max_p lse_p, lse = M + ln sum_p e^{lse_p - M}, o = sum_p e^{lse_p - lse} o_p
// One wave per (query row, 256-float slice of the latent); each lane owns four
// consecutive latent floats, so every partial row is read with 16-byte loads,
// eight splits at a time.
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int kSlice = 256;
constexpr int kBatch = 8;   // splits whose loads are in flight together

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      float* __restrict__ o_lat,
                                                      float* __restrict__ lse_out, int n_rows,
                                                      int num_splits, int rank) {
  const int slices = cdiv(rank, kSlice);
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= n_rows * slices) return;
  const int row = wid / slices;
  const int m0 = (wid % slices) * kSlice + lane * 4;
  const float* lp = lse_part + (size_t)row * num_splits;

  float M = -INFINITY;
  for (int p = lane; p < num_splits; p += 64) M = fmaxf(M, lp[p]);
  M = wave_max(M);
  float* out = o_lat + (size_t)row * rank;
  if (M == -INFINITY) {  // every split empty
    if (m0 < rank) *reinterpret_cast<float4*>(out + m0) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0 && wid % slices == 0) lse_out[row] = -INFINITY;
    return;
  }
  float s = 0.f;
  for (int p = lane; p < num_splits; p += 64) s += expf(lp[p] - M);
  s = wave_sum(s);
  const float lse = M + logf(s);
  if (lane == 0 && wid % slices == 0) lse_out[row] = lse;
  if (m0 >= rank) return;
  const float* op = o_part + (size_t)row * num_splits * rank + m0;
  // splits in groups of kBatch: all loads of a group are issued before any is
  // used; the sum still runs over p = 0, 1, 2, ... in order, skipping empty splits
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < num_splits; p0 += kBatch) {
    float4 v[kBatch];
    float l[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + u;
      l[u] = p < num_splits ? lp[p] : -INFINITY;
      v[u] = p < num_splits ? *reinterpret_cast<const float4*>(op + (size_t)p * rank)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (l[u] == -INFINITY) continue;
      const float w = expf(l[u] - lse);
      acc.x = fmaf(w, v[u].x, acc.x);
      acc.y = fmaf(w, v[u].y, acc.y);
      acc.z = fmaf(w, v[u].z, acc.z);
      acc.w = fmaf(w, v[u].w, acc.w);
    }
  }
  *reinterpret_cast<float4*>(out + m0) = acc;
}

}  // namespace

hipError_t launch_combine(const qkn_mla_dims& d, int num_splits, const float* o_part,
                          const float* lse_part, float* o_lat, float* lse, hipStream_t s) {
  const int n_rows = d.batch * d.s_q * d.heads;
  const int waves = n_rows * cdiv(d.rank, kSlice);
  hipLaunchKernelGGL(combine_kernel, dim3(cdiv(waves, 4)), dim3(256), 0, s, o_part, lse_part,
                     o_lat, lse, n_rows, num_splits, d.rank);
  return hipGetLastError();
}

}  // namespace qkn
