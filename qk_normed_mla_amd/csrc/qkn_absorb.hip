// qkn_mla_absorb_query: fold the static norm weights into the query and absorb
// W^K_g (QK-Normed MLA summary, "Metodologia" item 1), the per-row inverse RMS
// alpha^q (decode-logit equation) and the separately normed, rotated RoPE query
// (item 4).
//
// Two launches:
//   absorb_gemm   q~[row, m] = sum_j W^K_g[m, j] * (gamma_q[j] gamma_k[g, j] q[row, j])
//                 a float32 tiled GEMM per KV group, [rows_g x d] . [d x r]
//   absorb_rows   alpha^q and the RoPE query, one wave per query row
#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int TM = 64;   // query rows per tile (all of one KV group)
constexpr int TN = 64;   // latent columns per tile
constexpr int TK = 32;   // head-dim chunk staged in LDS

template <typename OutT>
__global__ __launch_bounds__(256) void absorb_gemm(
    const float* __restrict__ q, const float* __restrict__ w_k, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, OutT* __restrict__ q_tilde, int rows_per_group,
    int heads, int heads_per_group, int head_dim, int rank) {
  __shared__ float fs[TK][TM + 4];   // folded query, [j][row]
  __shared__ float ws[TK][TN + 4];   // W^K_g, [j][m]
  const int g = blockIdx.z;
  const int row0 = blockIdx.x * TM;
  const int m0 = blockIdx.y * TN;
  const int tid = threadIdx.x;
  const int tr = tid / 16;  // 16 x 16 threads, 4 x 4 outputs each
  const int tc = tid % 16;
  const float* wg = w_k + (size_t)g * rank * head_dim;
  const float* gk = gamma_k + (size_t)g * head_dim;

  // global row of local row n of group g: n = bi * Hg + hl -> bi * H + g * Hg + hl
  auto global_row = [&](int n) {
    int bi = n / heads_per_group, hl = n % heads_per_group;
    return (size_t)bi * heads + (size_t)g * heads_per_group + hl;
  };

  float acc[4][4] = {};
  for (int j0 = 0; j0 < head_dim; j0 += TK) {
    // stage TM x TK of the folded query and TN x TK of W^K_g (coalesced along j)
    for (int e = tid; e < TM * TK; e += 256) {
      int r = e / TK, j = e % TK;
      int n = row0 + r, jj = j0 + j;
      float v = 0.f;
      if (n < rows_per_group && jj < head_dim)
        v = q[global_row(n) * head_dim + jj] * gamma_q[jj] * gk[jj];
      fs[j][r] = v;
    }
    for (int e = tid; e < TN * TK; e += 256) {
      int m = e / TK, j = e % TK;
      int mm = m0 + m, jj = j0 + j;
      ws[j][m] = (mm < rank && jj < head_dim) ? wg[(size_t)mm * head_dim + jj] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < TK; ++j) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = fs[j][tr * 4 + u];
#pragma unroll
      for (int v = 0; v < 4; ++v) b[v] = ws[j][tc * 4 + v];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int n = row0 + tr * 4 + u;
    if (n >= rows_per_group) continue;
    size_t base = global_row(n) * rank;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int m = m0 + tc * 4 + v;
      if (m < rank) Elem<OutT>::store(q_tilde, base + m, acc[u][v]);
    }
  }
}

// One wave per query row: alpha^q = 1/RMS(q) and the normed, rotated RoPE query.
template <typename OutT>
__global__ __launch_bounds__(256) void absorb_rows(
    const float* __restrict__ q, const float* __restrict__ q_rope,
    const int32_t* __restrict__ q_pos, const float* __restrict__ gamma_qr,
    float* __restrict__ alpha_q, OutT* __restrict__ q_rope_out, int n_rows, int heads,
    int head_dim, int rope_dim, float eps, float theta) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const float* qr = q + (size_t)row * head_dim;
  float ss = 0.f;
  for (int j = lane; j < head_dim; j += 64) ss = fmaf(qr[j], qr[j], ss);
  ss = wave_sum(ss);
  if (lane == 0) alpha_q[row] = 1.0f / sqrtf(ss / (float)head_dim + eps);
  if (rope_dim == 0) return;
  const float* x = q_rope + (size_t)row * rope_dim;
  float sr = 0.f;
  for (int j = lane; j < rope_dim; j += 64) sr = fmaf(x[j], x[j], sr);
  sr = wave_sum(sr);
  const float inv = 1.0f / sqrtf(sr / (float)rope_dim + eps);
  const int pos = q_pos[row / heads];
  const int half = rope_dim / 2;
  OutT* out = q_rope_out + (size_t)row * rope_dim;
  for (int j = lane; j < half; j += 64) {
    float x1 = x[j] * inv * gamma_qr[j];
    float x2 = x[j + half] * inv * gamma_qr[j + half];
    float c = 1.f, s = 0.f;
    if (theta != 0.f) rope_cos_sin(pos, j, rope_dim, theta, &c, &s);
    Elem<OutT>::store(out, j, x1 * c - x2 * s);
    Elem<OutT>::store(out, j + half, x2 * c + x1 * s);
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
  hipLaunchKernelGGL(absorb_gemm<OutT>, grid, dim3(256), 0, s, q, w_k, gamma_q, gamma_k,
                     static_cast<OutT*>(q_tilde), rows_per_group, d.heads, hpg, d.head_dim,
                     d.rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_rows = d.batch * d.s_q * d.heads;
  hipLaunchKernelGGL(absorb_rows<OutT>, dim3(cdiv(n_rows, 4)), dim3(256), 0, s, q, q_rope, q_pos,
                     gamma_qr, alpha_q, static_cast<OutT*>(q_rope_normed), n_rows, d.heads,
                     d.head_dim, d.rope_dim, d.eps, d.rope_theta);
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
