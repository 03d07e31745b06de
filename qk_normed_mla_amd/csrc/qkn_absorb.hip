// qkn_mla_absorb_query: fold the static norm weights into the query and absorb
// W^K_g (QK-Normed MLA summary, "Metodologia" item 1), the per-row inverse RMS
// alpha^q (decode-logit equation) and the separately normed, rotated RoPE query
// (item 4).
//
// Two launches:
//   absorb_gemm   q~[row, m] = sum_j W^K_g[m, j] * (gamma_q[j] gamma_k[g, j] q[row, j])
//                 a float32 GEMM per KV group, [rows_g x d] . [d x r], on the
//                 float32 matrix cores (v_mfma_f32_32x32x2_f32): one wave per
//                 32 x 32 output tile, operands read straight from global memory
//                 as 16-byte rows of 4 head-dim entries.
//   absorb_rows   alpha^q and the RoPE query; one wave per query row, four
//                 heads of one query token per block sharing the rotation
//                 angles, formed once per block.
#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int WAVES_GEMM = 4;  // column tiles per block
constexpr int kMaxHeadDimGemm = 512;  // the host checks head_dim

// Wave tile: rows n0 .. n0 + 31 of group g, latent columns m0 .. m0 + 31.
// Lane l holds row / column l % 32; for each chunk of 8 head-dim entries the
// lanes 0-31 hold entries 0-3 and lanes 32-63 entries 4-7, and the i-th
// product pairs entry i with entry 4 + i (a fixed split of the reduction
// index, the same for both operands).
template <typename OutT>
__global__ __launch_bounds__(64 * WAVES_GEMM) void absorb_gemm(
    const float* __restrict__ q, const float* __restrict__ w_k, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, OutT* __restrict__ q_tilde, int rows_per_group,
    int heads, int heads_per_group, int head_dim, int rank) {
  __shared__ __attribute__((aligned(16))) float gqk[kMaxHeadDimGemm];  // gamma_q * gamma_k[g]
  const int g = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float* gk = gamma_k + (size_t)g * head_dim;
  for (int j = threadIdx.x; j < head_dim; j += 64 * WAVES_GEMM) gqk[j] = gamma_q[j] * gk[j];
  __syncthreads();
  const int n0 = blockIdx.x * 32;
  const int m0 = (blockIdx.y * WAVES_GEMM + wave) * 32;
  if (m0 >= rank) return;  // uniform per wave
  const float* wg = w_k + (size_t)g * rank * head_dim;

  // global row of local row n of group g: n = bi * Hg + hl -> bi * H + g * Hg + hl
  auto global_row = [&](int n) {
    const int bi = n / heads_per_group, hl = n % heads_per_group;
    return (size_t)bi * heads + (size_t)g * heads_per_group + hl;
  };

  const int r = lane & 31, hsel = lane >> 5;
  const int n = n0 + r, m = m0 + r;
  const bool row_ok = n < rows_per_group, col_ok = m < rank;
  // out-of-range rows / columns read row 0 and are zeroed after the load
  const float* qa = q + (row_ok ? global_row(n) : 0) * head_dim;
  const float* wb = wg + (size_t)(col_ok ? m : 0) * head_dim;

  f32x16 acc = {};
  constexpr int CB = 8;  // chunks of 8 head-dim entries whose loads are issued together
  for (int c0 = 0; c0 < head_dim; c0 += 8 * CB) {
    float4 a[CB], bv[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int k = c0 + 8 * u + 4 * hsel;
      const int kc = min(k, head_dim - 4);  // head_dim is a multiple of 4
      a[u] = *reinterpret_cast<const float4*>(qa + kc);
      bv[u] = *reinterpret_cast<const float4*>(wb + kc);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int k = c0 + 8 * u + 4 * hsel;
      const bool ok = k < head_dim;
      const int kc = min(k, head_dim - 4);
      const float4 gf = *reinterpret_cast<const float4*>(gqk + kc);
      const bool ra = ok && row_ok, rb = ok && col_ok;
      const float ax = ra ? a[u].x * gf.x : 0.f, ay = ra ? a[u].y * gf.y : 0.f;
      const float az = ra ? a[u].z * gf.z : 0.f, aw = ra ? a[u].w * gf.w : 0.f;
      const float bx = rb ? bv[u].x : 0.f, by = rb ? bv[u].y : 0.f;
      const float bz = rb ? bv[u].z : 0.f, bw = rb ? bv[u].w : 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ax, bx, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ay, by, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(az, bz, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(aw, bw, acc, 0, 0, 0);
    }
  }
  // D[i][j]: column j = lane % 32, row i = (reg % 4) + 8 (reg / 4) + 4 (lane / 32)
  if (!col_ok) return;
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) {
    const int i = (reg & 3) + 8 * (reg >> 2) + 4 * hsel;
    if (n0 + i < rows_per_group) Elem<OutT>::store(q_tilde, global_row(n0 + i) * rank + m, acc[reg]);
  }
}

// alpha^q = 1/RMS(q) and the normed, rotated RoPE query of four heads of one
// query token; the token's angles are formed once, in double precision.
constexpr int ROWS_HEADS = 4;
constexpr int MAX_HALF = 128;  // rope_dim / 2 <= 128 (the host checks rope_dim)

template <typename OutT>
__global__ __launch_bounds__(256) void absorb_rows(
    const float* __restrict__ q, const float* __restrict__ q_rope,
    const int32_t* __restrict__ q_pos, const float* __restrict__ gamma_qr,
    float* __restrict__ alpha_q, OutT* __restrict__ q_rope_out, int heads,
    int head_dim, int rope_dim, float eps, float theta) {
  __shared__ float cs[MAX_HALF], sn[MAX_HALF];
  const int tok = blockIdx.x;
  const int h0 = blockIdx.y * ROWS_HEADS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = rope_dim / 2;
  for (int j = threadIdx.x; j < half; j += 256) {
    float c = 1.f, s = 0.f;
    if (theta != 0.f) rope_cos_sin(q_pos[tok], j, rope_dim, theta, &c, &s);
    cs[j] = c;
    sn[j] = s;
  }
  __syncthreads();
  const int h = h0 + wave;
  if (h < heads) {
    const size_t row = (size_t)tok * heads + h;
    const float* qr = q + row * head_dim;
    float ss = 0.f;
    for (int j = lane; j < head_dim; j += 64) ss = fmaf(qr[j], qr[j], ss);
    ss = wave_sum(ss);
    if (lane == 0) alpha_q[row] = 1.0f / sqrtf(ss / (float)head_dim + eps);
    if (rope_dim == 0) return;
    const float* x = q_rope + row * rope_dim;
    float sr = 0.f;
    for (int j = lane; j < rope_dim; j += 64) sr = fmaf(x[j], x[j], sr);
    sr = wave_sum(sr);
    const float inv = 1.0f / sqrtf(sr / (float)rope_dim + eps);
    OutT* out = q_rope_out + row * rope_dim;
    for (int j = lane; j < half; j += 64) {
      const float x1 = x[j] * inv * gamma_qr[j];
      const float x2 = x[j + half] * inv * gamma_qr[j + half];
      Elem<OutT>::store(out, j, x1 * cs[j] - x2 * sn[j]);
      Elem<OutT>::store(out, j + half, x2 * cs[j] + x1 * sn[j]);
    }
  }
}

template <typename OutT>
hipError_t launch_typed(const qkn_mla_dims& d, const float* q, const float* q_rope,
                        const int32_t* q_pos, const float* w_k, const float* gamma_q,
                        const float* gamma_k, const float* gamma_qr, void* q_tilde,
                        float* alpha_q, void* q_rope_normed, hipStream_t s) {
  const int hpg = d.heads / d.groups;
  const int rows_per_group = d.batch * d.s_q * hpg;
  dim3 grid(cdiv(rows_per_group, 32), cdiv(d.rank, 32 * WAVES_GEMM), d.groups);
  hipLaunchKernelGGL(absorb_gemm<OutT>, grid, dim3(64 * WAVES_GEMM), 0, s, q, w_k, gamma_q,
                     gamma_k, static_cast<OutT*>(q_tilde), rows_per_group, d.heads, hpg,
                     d.head_dim, d.rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 rgrid(d.batch * d.s_q, cdiv(d.heads, ROWS_HEADS));
  hipLaunchKernelGGL(absorb_rows<OutT>, rgrid, dim3(256), 0, s, q, q_rope, q_pos, gamma_qr,
                     alpha_q, static_cast<OutT*>(q_rope_normed), d.heads, d.head_dim,
                     d.rope_dim, d.eps, d.rope_theta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_query(const qkn_mla_dims& d, const float* q, const float* q_rope,
                               const int32_t* q_pos, const float* w_k, const float* gamma_q,
                               const float* gamma_k, const float* gamma_qr, void* q_tilde,
                               float* alpha_q, void* q_rope_normed, hipStream_t s) {
  if (d.cache_dtype == QKN_BF16)
    return launch_typed<uint16_t>(d, q, q_rope, q_pos, w_k, gamma_q, gamma_k, gamma_qr, q_tilde,
                                  alpha_q, q_rope_normed, s);
  return launch_typed<float>(d, q, q_rope, q_pos, w_k, gamma_q, gamma_k, gamma_qr, q_tilde,
                             alpha_q, q_rope_normed, s);
}

}  // namespace qkn
