// qkn_mla_absorb_query: fold the static norm weights into the query and absorb
// W^K_g (QK-Normed MLA summary, "Metodologia" item 1), the per-row inverse RMS
// alpha^q (decode-logit equation) and the separately normed, rotated RoPE query
// (item 4).
//
// Two launches:
//   absorb_gemm   q~[row, m] = sum_j W^K_g[m, j] * (gamma_q[j] gamma_k[g, j] q[row, j])
//                 a float32 GEMM per KV group, [rows_g x d] . [d x r], on the
//                 float32 matrix cores (v_mfma_f32_32x32x2_f32), 64 x 128 tiles
//                 per block with both operands staged through LDS.
//   absorb_rows   alpha^q and the RoPE query; one wave per query row, four
//                 heads of one query token per block sharing the rotation
//                 angles, formed once per block.
#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TM = 64;    // query rows per block (all of one KV group)
constexpr int TN = 128;   // latent columns per block
constexpr int KC = 32;    // head-dim entries staged per step
constexpr int LDA = KC + 4;  // padded LDS row (floats)

// Block of 4 waves: a 64-row x 128-column tile of q~ for one group.  Wave
// (wr, wc) owns rows 32 wr .. +31 and columns 64 wc .. +63, i.e. two 32 x 32
// tiles of v_mfma_f32_32x32x2_f32.  The folded query rows and the W^K_g rows
// are staged through LDS 32 head-dim entries at a time (the next step's
// global loads are issued before the current step's products).  In a step,
// lane l reads 4 consecutive head-dim entries of its row (lanes 0-31 entries
// 8j .. 8j+3, lanes 32-63 entries 8j+4 .. 8j+7) and the i-th product pairs
// entry 8j+i with 8j+4+i: a fixed split of the reduction index, the same for
// both operands.
template <typename OutT>
__global__ __launch_bounds__(256) void absorb_gemm(
    const float* __restrict__ q, const float* __restrict__ w_k, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, OutT* __restrict__ q_tilde, int rows_per_group,
    int heads, int heads_per_group, int head_dim, int rank) {
  __shared__ __attribute__((aligned(16))) float As[TM * LDA];
  __shared__ __attribute__((aligned(16))) float Bs[TN * LDA];
  const int g = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int n0 = blockIdx.x * TM, m0 = blockIdx.y * TN;
  const float* wg = w_k + (size_t)g * rank * head_dim;
  const float* gk = gamma_k + (size_t)g * head_dim;

  // global row of local row n of group g: n = bi * Hg + hl -> bi * H + g * Hg + hl
  auto global_row = [&](int n) {
    const int bi = n / heads_per_group, hl = n % heads_per_group;
    return (size_t)bi * heads + (size_t)g * heads_per_group + hl;
  };

  // staging assignment: A 64 x 32 floats = 512 float4 (2 per thread), B 128 x 32 = 1024 (4)
  float4 ra[2], rb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u, r = e >> 3, k = k0 + 4 * (e & 7);
      const int n = n0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (n < rows_per_group && k < head_dim) {  // head_dim is a multiple of 4
        v = *reinterpret_cast<const float4*>(q + global_row(n) * head_dim + k);
        v.x *= gamma_q[k] * gk[k];
        v.y *= gamma_q[k + 1] * gk[k + 1];
        v.z *= gamma_q[k + 2] * gk[k + 2];
        v.w *= gamma_q[k + 3] * gk[k + 3];
      }
      ra[u] = v;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u, r = e >> 3, k = k0 + 4 * (e & 7);
      const int m = m0 + r;
      rb[u] = (m < rank && k < head_dim) ? *reinterpret_cast<const float4*>(wg + (size_t)m * head_dim + k)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      *reinterpret_cast<float4*>(&As[(e >> 3) * LDA + 4 * (e & 7)]) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      *reinterpret_cast<float4*>(&Bs[(e >> 3) * LDA + 4 * (e & 7)]) = rb[u];
    }
  };

  f32x16 acc[2] = {};
  const int r = lane & 31, hsel = lane >> 5;
  fetch(0);
  for (int k0 = 0; k0 < head_dim; k0 += KC) {
    __syncthreads();  // every wave is done with the previous step's tiles
    stash();
    __syncthreads();
    if (k0 + KC < head_dim) fetch(k0 + KC);
#pragma unroll
    for (int j = 0; j < KC / 8; ++j) {
      const float4 a = *reinterpret_cast<const float4*>(&As[(32 * wr + r) * LDA + 8 * j + 4 * hsel]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float4 bv = *reinterpret_cast<const float4*>(&Bs[(64 * wc + 32 * t + r) * LDA + 8 * j + 4 * hsel]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bv.x, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bv.y, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bv.z, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bv.w, acc[t], 0, 0, 0);
      }
    }
  }
  // D[i][j]: column j = lane % 32, row i = (reg % 4) + 8 (reg / 4) + 4 (lane / 32)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = m0 + 64 * wc + 32 * t + r;
    if (m >= rank) continue;
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
      const int n = n0 + 32 * wr + (reg & 3) + 8 * (reg >> 2) + 4 * hsel;
      if (n < rows_per_group) Elem<OutT>::store(q_tilde, global_row(n) * rank + m, acc[t][reg]);
    }
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
  dim3 grid(cdiv(rows_per_group, TM), cdiv(d.rank, TN), d.groups);
  hipLaunchKernelGGL(absorb_gemm<OutT>, grid, dim3(256), 0, s, q, w_k, gamma_q,
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
