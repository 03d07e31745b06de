// Kernels of the explicit path, where the normed keys are materialised
// (QK-Normed MLA summary, "Planteamiento del Problema": keys k = c W^K_g are
// RMS-normed after the projection; "Metodologia" item 4: the RoPE block is
// normed on its own).  Two users:
//
// Chunked prefill.  A chunk of s_q new query tokens per sequence attends
// causally to its whole cache, the chunk included (its tokens appended first):
//   prefill_query:  q^ = gamma_q * q / RMS(q) per head (IEEE half), and the
//                   normed, rotated RoPE query (bf16, as the absorb call's);
//                   also the query side of the GQA path.
//   prefill_expand: for every cached token and KV group, k^ = gamma_k *
//                   (c W^K_g) * alpha^k (the stored inverse RMS of that same
//                   projection of the stored latent) and v = c W^V_g, as IEEE
//                   half, matrix products on the matrix cores.
// The materialised q^, k^ and v are half, not bf16: the norm bounds |q^_j| by
// sqrt(d) |gamma_q,j| and |k^_j| likewise, and half's three more bits keep the
// explicit path inside the end-to-end tolerance; a value beyond the half range
// is reported (QKN_FLAG_PARTIAL_RANGE).
//   attend:         flash attention of the chunk over the materialised keys
//                   and values, l = scale * (q^ . k^ + q^R . k^R), online
//                   softmax, o = sum p v.
//
// The GQA path of GQLA (GQLA summary, section 2: the latent expanded into g
// groups of keys and values that the cache stores, plus the shared RoPE key;
// the decode is plain grouped attention).  Under QK-norm the stored key is the
// normed one.  The cache is paged like the latent cache, one row per token:
// [G x (k^ (d) | v (d)) half | k^R (d_R) bf16].
//   gqa_append:     for each new token, k^ = gamma_k * k / RMS(k), k = c W^K_g,
//                   and v = c W^V_g from the latent rounded to bf16, and the
//                   normed, rotated RoPE key.
//   attend:         the same attention kernel over the paged cache, split over
//                   the keys (half partials merged by the combine kernel).
#include <math.h>

#include <algorithm>

#include "qkn_internal.h"

namespace qkn {
namespace {

#define LDS_AS __attribute__((address_space(3)))
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// query side: one block per (query token (b, i), 16 heads), d = 128, d_R = 64.
// The RoPE angles depend on the position alone, so the block forms the 32
// cos / sin pairs once; each wave then takes 4 of the heads, all their loads
// in flight: q^ = gamma_q q / RMS(q) as half, the RoPE query normed, rotated
// and rounded to bf16.
// ---------------------------------------------------------------------------
constexpr int PQ_D = 128, PQ_DR = 64, PQ_ROWS = 4;

__global__ __launch_bounds__(256) void prefill_query_kernel(
    const float* __restrict__ q, const float* __restrict__ q_rope, const int32_t* __restrict__ q_pos,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_qr,
    _Float16* __restrict__ q_hat, uint16_t* __restrict__ qr_out, int heads, float eps, float theta) {
  __shared__ float cs[PQ_DR / 2], sn[PQ_DR / 2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int token = blockIdx.x / (heads / 16);
  const int hb = 16 * (blockIdx.x % (heads / 16)) + w;  // this wave's heads: hb + 4 u
  if (threadIdx.x < PQ_DR / 2) {
    float c = 1.f, s = 0.f;
    if (theta != 0.f) rope_cos_sin<false>(q_pos[token], threadIdx.x, PQ_DR, theta, &c, &s);
    cs[threadIdx.x] = c;
    sn[threadIdx.x] = s;
  }
  const float g0 = gamma_q[lane], g1 = gamma_q[lane + 64], gr = gamma_qr[lane];
  __syncthreads();
  const float c = cs[lane & 31], s = sn[lane & 31];
  float x0[PQ_ROWS], x1[PQ_ROWS], xr[PQ_ROWS];
#pragma unroll
  for (int u = 0; u < PQ_ROWS; ++u) {
    const size_t row = (size_t)token * heads + hb + 4 * u;
    x0[u] = q[row * PQ_D + lane];
    x1[u] = q[row * PQ_D + 64 + lane];
    xr[u] = q_rope[row * PQ_DR + lane];
  }
#pragma unroll
  for (int u = 0; u < PQ_ROWS; ++u) {
    const size_t row = (size_t)token * heads + hb + 4 * u;
    const float ss = wave_sum(fmaf(x1[u], x1[u], x0[u] * x0[u]));
    const float inv = 1.0f / sqrtf(ss / (float)PQ_D + eps);
    q_hat[row * PQ_D + lane] = static_cast<_Float16>(x0[u] * inv * g0);
    q_hat[row * PQ_D + 64 + lane] = static_cast<_Float16>(x1[u] * inv * g1);
    const float sr = wave_sum(xr[u] * xr[u]);
    const float ir = 1.0f / sqrtf(sr / (float)PQ_DR + eps);
    const float y = xr[u] * ir * gr;
    const float other = __shfl_xor(y, 32);  // the pair partner j +- d_R / 2
    // first half: y1 c - y2 s; second half: y2 c + y1 s
    const float out = lane < 32 ? y * c - other * s : y * c + other * s;
    qr_out[row * PQ_DR + lane] = f32_to_bf16(out);
  }
}

// ---------------------------------------------------------------------------
// keys and values: K = C W^K_g, V = C W^V_g for 256 tokens of one sequence and
// group and NT column tiles (32 NT of the d columns) per block (blockIdx.z:
// column block * 2 + 0 for keys, + 1 for values).  Wave w owns tokens 32 w ..
// 32 w + 31 (the A rows: the stored bf16 latent words, exact operands) and the
// block's NT column tiles.  W passes through LDS in chunks of KC rows split into
// three bf16 words (hi + mid + lo, exact to 2^-24), read with
// ds_read_b64_tr_b16; every product is exact and the sums are float32.
// ---------------------------------------------------------------------------
constexpr int EX_WAVES = 8;
constexpr int EX_TOK = 32 * EX_WAVES;
constexpr int EX_CHUNK = 8192;  // W values per staged chunk
constexpr int EX_PAD = 16;      // bf16 of padding per staged row
constexpr int ex_chunk_rows(int d) { return EX_CHUNK / d < 128 ? EX_CHUNK / d : 128; }

__device__ __forceinline__ void split3(float4 v, bf16x4& hi, bf16x4& mid, bf16x4& lo) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  hi = __builtin_convertvector(x, bf16x4);
  const f32x4 h = __builtin_convertvector(hi, f32x4);
  f32x4 r1;
#pragma unroll
  for (int j = 0; j < 4; ++j) r1[j] = x[j] - h[j];
  mid = __builtin_convertvector(r1, bf16x4);
  const f32x4 m = __builtin_convertvector(mid, f32x4);
  f32x4 r2;
#pragma unroll
  for (int j = 0; j < 4; ++j) r2[j] = r1[j] - m[j];
  lo = __builtin_convertvector(r2, bf16x4);
}

__device__ __forceinline__ bf16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(const_cast<__bf16*>(p)));
}

template <int NT>
__global__ __launch_bounds__(64 * EX_WAVES) void prefill_expand_kernel(
    const uint16_t* __restrict__ kv, const float* __restrict__ alpha_k,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const float* __restrict__ w_k, const float* __restrict__ w_v,
    const float* __restrict__ gamma_k, _Float16* __restrict__ k_hat, _Float16* __restrict__ v_out,
    int32_t* __restrict__ err_flag, int groups, int rank, int rope_dim, int max_pages,
    int num_pages, int max_T, int width) {
  constexpr int D = NT * 32;  // columns of this block: col0 .. col0 + D - 1 of the width
  constexpr int KC = ex_chunk_rows(D);
  constexpr int PER = KC * D / 4 / (64 * EX_WAVES);  // float4 of a chunk per thread
  constexpr int SPC = KC / 16;                       // 16-row steps per chunk
  constexpr int WROW = D + EX_PAD;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __bf16* W0 = reinterpret_cast<__bf16*>(smem);
  __bf16* W1 = W0 + KC * WROW;
  __bf16* W2 = W1 + KC * WROW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int l16 = lane & 15, G = (lane >> 4) & 1;
  const int b = blockIdx.y / groups, g = blockIdx.y % groups;
  const bool values = blockIdx.z & 1;
  const int col0 = (blockIdx.z >> 1) * D;
  const float* wg = (values ? w_v : w_k) + (size_t)g * rank * width + col0;
  int T = seq_lens[b];
  T = min(max(T, 0), max_pages * QKN_MLA_PAGE_SIZE);
  const int t = blockIdx.x * EX_TOK + 32 * wave + l32;  // token of this lane's A row
  int row = -1;                                          // its cache row
  if (t < T) {
    const int pg = block_table[(size_t)b * max_pages + t / QKN_MLA_PAGE_SIZE];
    if (pg >= 0 && pg < num_pages) row = pg * QKN_MLA_PAGE_SIZE + t % QKN_MLA_PAGE_SIZE;
    else if (err_flag && hh == 0) atomicOr(err_flag, QKN_FLAG_INDEX);
  }
  const uint16_t* crow = kv + (size_t)(row >= 0 ? row : 0) * (rank + rope_dim);

  // the next chunk: W rows k0 .. k0 + KC - 1 and this lane's latents of its
  // SPC steps in the order of the transposed read (4 hh + 0..3, 8 + 4 hh + 0..3)
  float4 wv[PER];
  uint2 av[SPC][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * 64 * EX_WAVES;
      wv[u] = *reinterpret_cast<const float4*>(wg + (size_t)(k0 + e / (D / 4)) * width + 4 * (e % (D / 4)));
    }
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
      const uint16_t* ap = crow + k0 + 16 * st + 4 * hh;
      av[st][0] = row >= 0 ? *reinterpret_cast<const uint2*>(ap) : make_uint2(0u, 0u);
      av[st][1] = row >= 0 ? *reinterpret_cast<const uint2*>(ap + 8) : make_uint2(0u, 0u);
    }
  };
  load(0);

  f32x16 acc[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) acc[ct] = f32x16{};
  const int tr_off = (4 * hh + (l16 >> 2)) * WROW + 16 * G + 4 * (l16 & 3);
  for (int k0 = 0; k0 < rank; k0 += KC) {
    __syncthreads();  // every read of the previous chunk done
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * 64 * EX_WAVES;
      bf16x4 hi, mid, lo;
      split3(wv[u], hi, mid, lo);
      const int at = (e / (D / 4)) * WROW + 4 * (e % (D / 4));
      *reinterpret_cast<bf16x4*>(W0 + at) = hi;
      *reinterpret_cast<bf16x4*>(W1 + at) = mid;
      *reinterpret_cast<bf16x4*>(W2 + at) = lo;
    }
    bf16x8 a[SPC];
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
      const uint4 w4 = {av[st][0].x, av[st][0].y, av[st][1].x, av[st][1].y};
      a[st] = __builtin_bit_cast(bf16x8, w4);  // the stored words of c_t
    }
    if (k0 + KC < rank) load(k0 + KC);  // in flight during this chunk's products
    __syncthreads();
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int off = tr_off + 16 * st * WROW + 32 * ct;
        const bf16x8 b0 = __builtin_shufflevector(tr_read(W0 + off), tr_read(W0 + off + 8 * WROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b1 = __builtin_shufflevector(tr_read(W1 + off), tr_read(W1 + off + 8 * WROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b2 = __builtin_shufflevector(tr_read(W2 + off), tr_read(W2 + off + 8 * WROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        acc[ct] = mfma(a[st], b0, acc[ct]);
        acc[ct] = mfma(a[st], b1, acc[ct]);
        acc[ct] = mfma(a[st], b2, acc[ct]);
      }
    }
  }

  // D[i][j]: lane holds column 32 ct + l32 of tokens i = r % 4 + 8 (r / 4) + 4 hh
  // of the wave; keys are scaled by gamma_k[j] alpha^k of the token.  Tokens
  // past the sequence (or on a bad page) are written as zeros.
  _Float16* out = values ? v_out : k_hat;
  const float* gk = gamma_k + (size_t)g * width + col0;
  float big = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = (r & 3) + 8 * (r >> 2) + 4 * hh;
    const int tt = blockIdx.x * EX_TOK + 32 * wave + i;
    if (tt >= max_T) continue;
    const int row_i = __shfl(row, i);  // lane i holds token i's cache row
    float s = 0.f;
    if (row_i >= 0) s = values ? 1.f : alpha_k[(size_t)row_i * groups + g];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int j = 32 * ct + l32;
      const float x = row_i >= 0 ? acc[ct][r] * s * (values ? 1.f : gk[j]) : 0.f;
      big = fmaxf(big, fabsf(x));
      out[(((size_t)b * max_T + tt) * groups + g) * width + col0 + j] = static_cast<_Float16>(x);
    }
  }
  // a value the half rounds to +-inf
  if (big >= 65520.f && err_flag) atomicOr(err_flag, QKN_FLAG_PARTIAL_RANGE);
}

// ---------------------------------------------------------------------------
// GQA-path append: one block of 16 waves per (32 new tokens, group, keys |
// values).  Wave w computes the 32 x 32 tile of columns 32 (w % 4) .. + 31
// over the latent rows of its quarter of the rank (16-row steps w / 4, w / 4 +
// 4, ...), with every load of its steps issued before its products; the four
// quarters' partial tiles are summed through LDS in a fixed order.  A operand:
// the latent rounded to bf16 (the latent cache's stored words, an exact
// operand); B: W_g columns read 8 rows per lane and split into three bf16
// words (hi + mid + lo, exact to 2^-24), so every product is exact and the
// sums are float32.  Keys: the sums of squares of each token's 128 entries
// (per wave over its 32 lanes, then over the 4 column tiles in LDS) give
// 1 / RMS; the key blocks of group 0 also write the normed, rotated RoPE key.
// Tokens with an out-of-range sequence, position or page are skipped and
// reported.
// ---------------------------------------------------------------------------
constexpr int GA_D = 128, GA_DR = 64;
constexpr int kGqaSmallAppend = 512;  // up to this many tokens: one block per token
constexpr int GA_WAVES = 16;
constexpr int GA_MAX_STEPS = 4;  // 16-row steps of a wave whose loads are in flight together

__global__ __launch_bounds__(64 * GA_WAVES) void gqa_append_kernel(
    const float* __restrict__ c_new, const float* __restrict__ k_rope_new,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_table, const float* __restrict__ w_k,
    const float* __restrict__ w_v, const float* __restrict__ gamma_k,
    const float* __restrict__ gamma_kr, uint16_t* __restrict__ kvg, int32_t* __restrict__ err_flag,
    int n_tokens, int batch, int groups, int rank, int max_pages, int num_pages, float eps,
    float theta) {
  __shared__ f32x4 part[3][4][4][64];  // partial tiles of quarters 1..3: [q - 1][ct][r / 4][lane]
  __shared__ float ssq[4][32];
  __shared__ int slot_of[32];
  __shared__ int pos_of[32];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int ct = w & 3, quarter = w >> 2;
  const int n0 = blockIdx.x * 32;
  const int g = blockIdx.y;
  const bool values = blockIdx.z == 1;
  const int row_words = 2 * GA_D * groups + GA_DR;
  if (tid < 32) {
    const int n = n0 + tid;
    int slot = -1, p = 0;
    if (n < n_tokens) {
      const int b = seq_idx[n];
      p = pos[n];
      if (b >= 0 && b < batch && p >= 0 && p < max_pages * QKN_MLA_PAGE_SIZE) {
        const int pg = block_table[(size_t)b * max_pages + p / QKN_MLA_PAGE_SIZE];
        if (pg >= 0 && pg < num_pages) slot = pg * QKN_MLA_PAGE_SIZE + p % QKN_MLA_PAGE_SIZE;
      }
      if (slot < 0 && err_flag && g == 0 && !values) atomicOr(err_flag, QKN_FLAG_INDEX);
    }
    slot_of[tid] = slot;
    pos_of[tid] = p;
  }

  // ---- this wave's partial tile: tokens n0 + i, columns 32 ct + j ----
  const int tok = n0 + l32;
  const bool tok_ok = tok < n_tokens;
  const float* crow = c_new + (size_t)(tok_ok ? tok : 0) * rank + 8 * hh;
  const float* wcol = (values ? w_v : w_k) + (size_t)g * rank * GA_D + (size_t)(8 * hh) * GA_D + 32 * ct + l32;
  const int steps = rank / 16;
  f32x16 acc = {};
  for (int s0 = quarter; s0 < steps; s0 += 4 * GA_MAX_STEPS) {
    float4 cv[GA_MAX_STEPS][2];
    float wv[GA_MAX_STEPS][8];
#pragma unroll
    for (int u = 0; u < GA_MAX_STEPS; ++u) {
      const int st = s0 + 4 * u;
      const bool live = st < steps;
      const int k0 = 16 * (live ? st : 0);
      cv[u][0] = tok_ok && live ? *reinterpret_cast<const float4*>(crow + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
      cv[u][1] = tok_ok && live ? *reinterpret_cast<const float4*>(crow + k0 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[u][j] = live ? wcol[(size_t)(k0 + j) * GA_D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < GA_MAX_STEPS; ++u) {
      const f32x8 cx = {cv[u][0].x, cv[u][0].y, cv[u][0].z, cv[u][0].w,
                        cv[u][1].x, cv[u][1].y, cv[u][1].z, cv[u][1].w};
      const bf16x8 a = __builtin_convertvector(cx, bf16x8);  // nearest-even, as the latent cache stores it
      bf16x4 h0, m0, lo0, h1, m1, lo1;
      split3(make_float4(wv[u][0], wv[u][1], wv[u][2], wv[u][3]), h0, m0, lo0);
      split3(make_float4(wv[u][4], wv[u][5], wv[u][6], wv[u][7]), h1, m1, lo1);
      acc = mfma(a, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7), acc);
      acc = mfma(a, __builtin_shufflevector(m0, m1, 0, 1, 2, 3, 4, 5, 6, 7), acc);
      acc = mfma(a, __builtin_shufflevector(lo0, lo1, 0, 1, 2, 3, 4, 5, 6, 7), acc);
    }
  }
  if (quarter > 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      part[quarter - 1][ct][q][lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  }
  __syncthreads();  // slot_of, pos_of and the partial tiles
  const bool owner = quarter == 0;  // the wave that finishes column tile ct
  if (owner) {
#pragma unroll
    for (int qt = 0; qt < 3; ++qt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 p = part[qt][ct][q][lane];
        acc[4 * q] += p[0];
        acc[4 * q + 1] += p[1];
        acc[4 * q + 2] += p[2];
        acc[4 * q + 3] += p[3];
      }
    }
  }

  // acc[r]: token i = r % 4 + 8 (r / 4) + 4 hh of the tile, column 32 ct + l32
  if (owner && !values) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float q = acc[r] * acc[r];
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) q += __shfl_xor(q, m, 32);
      if (l32 == 0) ssq[ct][(r & 3) + 8 * (r >> 2) + 4 * hh] = q;
    }
  }
  __syncthreads();  // the column tiles' sums of squares
  if (owner) {
    const int col = 32 * ct + l32;
    const float gk = values ? 1.f : gamma_k[(size_t)g * GA_D + col];
    float big = 0.f;
    const int part_off = 2 * GA_D * g + (values ? GA_D : 0) + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = (r & 3) + 8 * (r >> 2) + 4 * hh;
      const int slot = slot_of[i];
      if (slot < 0) continue;
      float x = acc[r];
      if (!values) {
        const float ss = (ssq[0][i] + ssq[1][i]) + (ssq[2][i] + ssq[3][i]);
        x = x * (1.0f / sqrtf(ss / (float)GA_D + eps)) * gk;
      }
      big = fmaxf(big, fabsf(x));
      const _Float16 hx = static_cast<_Float16>(x);
      kvg[(size_t)slot * row_words + part_off] = __builtin_bit_cast(uint16_t, hx);
    }
    if (big >= 65520.f && err_flag) atomicOr(err_flag, QKN_FLAG_PARTIAL_RANGE);
  }

  // ---- the RoPE key (key blocks of group 0): wave w takes tokens w, w + 16 ----
  if (values || g != 0) return;
  for (int i = w; i < 32; i += GA_WAVES) {
    const int slot = slot_of[i];
    if (slot < 0) continue;  // uniform over the wave
    const float x = k_rope_new[(size_t)(n0 + i) * GA_DR + lane];
    const float ss = wave_sum(fmaf(x, x, 0.f));
    const float inv = 1.0f / sqrtf(ss / (float)GA_DR + eps);
    const float xn = x * inv * gamma_kr[lane];
    const float x2 = __shfl(xn, lane + GA_DR / 2);
    if (lane < GA_DR / 2) {
      float c = 1.f, sn = 0.f;
      if (theta != 0.f) rope_cos_sin<false>(pos_of[i], lane, GA_DR, theta, &c, &sn);
      uint16_t* out = kvg + (size_t)slot * row_words + 2 * GA_D * groups;
      out[lane] = f32_to_bf16(xn * c - x2 * sn);
      out[lane + GA_DR / 2] = f32_to_bf16(x2 * c + xn * sn);
    }
  }
}

// ---------------------------------------------------------------------------
// GQA-path append of a few tokens: one block of 16 waves per (TPB consecutive
// tokens, group, keys | values).  Thread t takes columns 4 (t % 32) .. + 3 over
// the latent rows t / 32, t / 32 + 32, ... (all its weight loads, 16-byte
// pieces, in flight together) and applies each weight row to the TPB tokens'
// latents (staged in LDS), accumulating in float32 with fused multiply-adds;
// the 32 row groups' partial sums are added in a fixed order through LDS.
// Keys: the sum of squares over the 128 entries gives 1 / RMS.  The key block
// of group 0 also writes the normed, rotated RoPE keys.  A token with an
// out-of-range sequence, position or page is skipped and reported.
// ---------------------------------------------------------------------------
constexpr int GS_RG = 32;                  // row groups (d = 128: 32 column quads)
constexpr int GS_MAX_ROWS = 512 / GS_RG;   // rows per thread, all in flight (r <= 512)

template <int TPB>
__global__ __launch_bounds__(1024) void gqa_append_small_kernel(
    const float* __restrict__ c_new, const float* __restrict__ k_rope_new,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_table, const float* __restrict__ w_k,
    const float* __restrict__ w_v, const float* __restrict__ gamma_k,
    const float* __restrict__ gamma_kr, uint16_t* __restrict__ kvg, int32_t* __restrict__ err_flag,
    int n_tokens, int batch, int groups, int rank, int max_pages, int num_pages, float eps,
    float theta) {
  __shared__ float4 part[TPB][GS_RG][GA_D / 4];
  __shared__ float lat[TPB][512];  // the tokens' latents as the latent cache stores them
  __shared__ float red[TPB][2];
  __shared__ int slot_s[TPB], pos_s[TPB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n0 = blockIdx.x * TPB, g = blockIdx.y;
  const bool values = blockIdx.z == 1;
  const int cq = tid % GS_RG, rg = tid / GS_RG;  // column quad, row group
  // this thread's weight loads go out before the latents and slot lookups
  const float* wg = (values ? w_v : w_k) + (size_t)g * rank * GA_D + 4 * cq;
  const int nrows = (rank - rg + GS_RG - 1) / GS_RG;
  float4 wv[GS_MAX_ROWS];
#pragma unroll
  for (int u = 0; u < GS_MAX_ROWS; ++u) {
    const int m = rg + GS_RG * u;
    wv[u] = u < nrows ? *reinterpret_cast<const float4*>(wg + (size_t)m * GA_D) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int e = tid; e < TPB * rank; e += 1024) {
    const int t = e / rank, m = e % rank;
    const float c = n0 + t < n_tokens ? c_new[(size_t)(n0 + t) * rank + m] : 0.f;
    lat[t][m] = static_cast<float>(static_cast<__bf16>(c));  // bf16, nearest-even
  }
  if (tid < TPB) {
    const int n = n0 + tid;
    int slot = -1, p = 0;
    if (n < n_tokens) {
      const int b = seq_idx[n];
      p = pos[n];
      if (b >= 0 && b < batch && p >= 0 && p < max_pages * QKN_MLA_PAGE_SIZE) {
        const int pg = block_table[(size_t)b * max_pages + p / QKN_MLA_PAGE_SIZE];
        if (pg >= 0 && pg < num_pages) slot = pg * QKN_MLA_PAGE_SIZE + p % QKN_MLA_PAGE_SIZE;
      }
      if (slot < 0 && err_flag && g == 0 && !values) atomicOr(err_flag, QKN_FLAG_INDEX);
    }
    slot_s[tid] = slot;
    pos_s[tid] = p;
  }
  __syncthreads();
  float4 acc[TPB];
#pragma unroll
  for (int t = 0; t < TPB; ++t) acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < GS_MAX_ROWS; ++u) {
    const int m = rg + GS_RG * u;
    if (u < nrows) {
#pragma unroll
      for (int t = 0; t < TPB; ++t) {
        const float c = lat[t][m];
        acc[t].x = fmaf(c, wv[u].x, acc[t].x);
        acc[t].y = fmaf(c, wv[u].y, acc[t].y);
        acc[t].z = fmaf(c, wv[u].z, acc[t].z);
        acc[t].w = fmaf(c, wv[u].w, acc[t].w);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TPB; ++t) part[t][rg][cq] = acc[t];
  __syncthreads();
  const int row_words = 2 * GA_D * groups + GA_DR;
  // threads t * 128 + j (t < TPB): column j of token t
  const int tt = tid / GA_D, j = tid % GA_D;
  float x = 0.f;
  if (tt < TPB) {
    const float* pc = reinterpret_cast<const float*>(&part[tt][0][0]) + j;
#pragma unroll
    for (int q = 0; q < GS_RG; ++q) x += pc[q * GA_D];
  }
  if (!values) {  // uniform over the block
    if (tt < TPB) {
      const float ss = wave_sum(x * x);
      if (lane == 0) red[tt][(tid >> 6) & 1] = ss;
    }
    __syncthreads();
  }
  if (tt < TPB) {
    const int slot = slot_s[tt];
    if (slot >= 0) {
      if (!values)
        x = x * (1.0f / sqrtf((red[tt][0] + red[tt][1]) / (float)GA_D + eps)) * gamma_k[(size_t)g * GA_D + j];
      if (fabsf(x) >= 65520.f && err_flag) atomicOr(err_flag, QKN_FLAG_PARTIAL_RANGE);
      const _Float16 hx = static_cast<_Float16>(x);
      kvg[(size_t)slot * row_words + 2 * GA_D * g + (values ? GA_D : 0) + j] = __builtin_bit_cast(uint16_t, hx);
    }
  }
  // the RoPE keys: wave 2 t of the key block of group 0 takes token t (the
  // block has 16 waves, TPB <= 8)
  if (values || g != 0 || (w & 1) || w / 2 >= TPB) return;
  const int t = w / 2, n = n0 + t, slot = slot_s[t];
  if (slot < 0) return;  // uniform over the wave
  const float xr = k_rope_new[(size_t)n * GA_DR + lane];
  const float sr = wave_sum(fmaf(xr, xr, 0.f));
  const float inv = 1.0f / sqrtf(sr / (float)GA_DR + eps);
  const float xn = xr * inv * gamma_kr[lane];
  const float x2 = __shfl(xn, lane + GA_DR / 2);
  if (lane < GA_DR / 2) {
    float c = 1.f, sn = 0.f;
    if (theta != 0.f) rope_cos_sin<false>(pos_s[t], lane, GA_DR, theta, &c, &sn);
    uint16_t* out = kvg + (size_t)slot * row_words + 2 * GA_D * groups;
    out[lane] = f32_to_bf16(xn * c - x2 * sn);
    out[lane + GA_DR / 2] = f32_to_bf16(x2 * c + xn * sn);
  }
}

// ---------------------------------------------------------------------------
// attention: one workgroup per (sequence, key split, 4 consecutive query
// tokens, 32 heads of one group) -- or fewer tokens and more 32-head blocks of
// the group when s_q is small; wave w takes one query token with 32 heads as
// its rows (lane l % 32).  Keys stream in tiles of 32 (k^ 8 KB, k^R 4 KB, v 8 KB)
// through three LDS slots as a software pipeline (the loop below).  Per tile
// and wave:
//   S^T[32 keys x 32 heads] = K^ q^^T + K^R q^R^T (12 products; A a 16-byte
//     key row read per lane, B the queries in registers),
//   online softmax in base 2 against a lazily moved reference (probabilities
//     at most 2^8, rounded to half; the normaliser summed from the same rounded
//     values),
//   O^T[128 x 32 heads] += V^T P^T (8 products; V^T read with
//     ds_read_b64_tr_b16 from the row-major tile).
// Rows of 256 bytes store chunk c of key t at chunk c ^ kswz(t) (RoPE rows:
// c ^ rswz(t)), so the column reads of 32 rows spread over the banks.
// ---------------------------------------------------------------------------
constexpr int AT_D = 128, AT_DR = 64, AT_R = 512;
constexpr int AT_KEYS = 32;
constexpr int AT_K_BYTES = AT_KEYS * AT_D * 2;    // 8192
constexpr int AT_R_BYTES = AT_KEYS * AT_DR * 2;   // 4096
constexpr int AT_TILE = 2 * AT_K_BYTES + AT_R_BYTES;  // 20480
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyLog2 = 8.f;  // probabilities up to 256: far inside the half range

__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Word 3 of a raw buffer descriptor on gfx950 (32-bit data format; offsets
// at or past the size field read as zero).
constexpr int kRsrcWord3 = 0x00020000;

typedef const __attribute__((address_space(4))) int32_t ConstI32;  // read through the scalar cache

// Chunk swizzles for the 64 four-byte LDS banks.  Chunk c of a 256-byte key
// or value row t is stored at c ^ kswz(t): kswz is a bijection on 16 rows (so
// the 16-byte reads of 16 rows at one chunk, the QK operand, meet 64 banks)
// whose rows 4k .. 4k + 3 differ in bits 2-3 (so the 8-byte transposed reads
// of 4 rows at 4 neighbouring chunks, the PV operand, do too).  Chunk c of a
// 128-byte RoPE row t is stored at c ^ rswz(t): rows 2j and 2j + 1 fall on the
// two halves of the banks, so rswz must differ over the even (and the odd)
// rows of 16.
// compile-time unrolled loop: f(integral_constant<int, i>) for i in [B, E)
template <int B, int E>
struct Unroll {
  template <typename F>
  __device__ __forceinline__ static void run(F&& f) {
    f(std::integral_constant<int, B>{});
    Unroll<B + 1, E>::run(f);
  }
};
template <int E>
struct Unroll<E, E> {
  template <typename F>
  __device__ __forceinline__ static void run(F&&) {}
};

__device__ __forceinline__ int kswz(int t) { return 4 * (t & 3) + ((t >> 2) & 3); }
__device__ __forceinline__ int rswz(int t) { return (t >> 1) & 7; }

struct AttendArgs {
  const _Float16* q_hat;
  const uint16_t* q_rope;
  // GQA: the paged cache (rows of row_words 16-bit words); prefill: k^ and v
  // [B, max_T, G, d] and the latent cache (its RoPE keys)
  const uint16_t* kvg;
  const _Float16* k_hat;
  const _Float16* v;
  const uint16_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* o;               // [rows, d] float32 when num_splits == 1
  float* lse;             // [rows]
  _Float16* o_part;       // [rows, P, d] half when num_splits > 1
  float* lse_part;        // [rows, P]
  int32_t* err_flag;
  // a workgroup: tpw query tokens x 4 / tpw blocks of 32 heads (one group)
  int batch, s_q, heads, groups, max_pages, num_pages, max_T, tpw, token_groups, head_groups, num_splits;
  int row_words, rank;
  float scale;
};

// Consecutive workgroup ids go to the 8 XCDs in turn; this renumbering gives
// each XCD a contiguous run of logical ids, so the head blocks that read the
// same keys share one L2.
__device__ __forceinline__ int xcd_local(int id, int n) {
  const int full = n & ~7;
  if (id >= full) return id;
  return (id & 7) * (full >> 3) + (id >> 3);
}

// IDLE: s_q is not a multiple of the query tokens per workgroup, so some waves
// have no query token (they then only move tiles); otherwise every wave works
// and the loop has no branch for it.
template <bool GQA, bool IDLE>
__global__ __launch_bounds__(256, 1) void attend_kernel(const AttendArgs A) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * AT_TILE];
  const int tid = threadIdx.x;
  // the wave index is uniform over the wave: held in a scalar register, the
  // heads, group and query token derived from it are too, and so are the
  // tile descriptors built from them
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int s_q = A.s_q, heads = A.heads, groups = A.groups, max_pages = A.max_pages;
  const int head_groups = A.head_groups, token_groups = A.token_groups, tpw = A.tpw;
  int hg, tg, sp, b;
  const int items = token_groups * head_groups;  // workgroups of one (sequence, split) pair
  bool ragged = false;
  int tl = 0;  // length of sequence `lane` (GQA, batch <= 64)
  if (GQA && A.batch <= 64) {
    tl = lane < A.batch ? A.seq_lens[lane] : 0;
    const int t0 = __builtin_amdgcn_readfirstlane(tl);
    ragged = __ballot(lane < A.batch && tl != t0) != 0;
  }
  if (ragged) {
    // The (sequence, split) pairs in order of length (longest first, ties by
    // index) are dealt round robin over the 8 XCDs (block 8 j + x is the j-th
    // of XCD x), the token and head blocks of a pair together: they read the
    // same keys and share an L2, and every XCD holds the same mix of lengths,
    // longest first.  Blocks past the last pair exit.
    const int pos = blockIdx.x >> 3;
    const int v = pos % items;
    const int k = (pos / items) * 8 + (blockIdx.x & 7);
    if (k >= A.batch * A.num_splits) return;
    const int o = k / A.num_splits;
    sp = k - o * A.num_splits;
    hg = v % head_groups;
    tg = v / head_groups;
    int rank = 0;  // place of sequence `lane` in the order
    for (int j = 0; j < A.batch; ++j) {
      const int tj = __builtin_amdgcn_readlane(tl, j);
      rank += (tj > tl || (tj == tl && j < lane)) ? 1 : 0;
    }
    // the ranks are a permutation of 0 .. batch - 1: exactly one lane has rank o
    b = static_cast<int>(__builtin_ctzll(__ballot(lane < A.batch && rank == o)));
  } else if (GQA) {
    // equal lengths (or more than 64 sequences): XCD x takes the x-th eighth
    // of the workgroups in order, so that the splits and blocks of one
    // sequence share an L2 (the grid may hold more blocks: they exit)
    const int n_items = A.batch * A.num_splits * items;
    const int per_xcd = (n_items + 7) / 8;
    if ((int)(blockIdx.x >> 3) >= per_xcd) return;
    const int lid = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (lid >= n_items) return;
    hg = lid % head_groups;
    tg = (lid / head_groups) % token_groups;
    sp = (lid / items) % A.num_splits;
    b = lid / (items * A.num_splits);
  } else {
    const int lid = xcd_local(blockIdx.x, gridDim.x);
    hg = lid % head_groups;
    tg = (lid / head_groups) % token_groups;
    sp = (lid / (head_groups * token_groups)) % A.num_splits;
    b = lid / (head_groups * token_groups * A.num_splits);
  }
  const int h0 = 32 * ((4 / tpw) * hg + w / tpw);  // this wave's heads
  const int g = h0 / (heads / groups);              // the same for every wave
  const int i = tpw * tg + w % tpw;                 // this wave's query token
  const bool active = i < s_q;
  int T = A.seq_lens[b];
  int err = 0;
  if (T < s_q || T > max_pages * QKN_MLA_PAGE_SIZE) {
    err = 1;
    T = min(max(T, s_q), max_pages * QKN_MLA_PAGE_SIZE);
  }
  // this split's keys [lo, hi): whole pages (the decode's split rule)
  const int L = split_len(T, A.num_splits);
  const int lo = min(sp * L, T), hi = min(sp * L + L, T);  // lo < hi: lo a multiple of 64
  const int vis = active ? T - s_q + i + 1 : 0;                        // keys of this wave
  const int vis_max = T - s_q + min(tpw * tg + tpw - 1, s_q - 1) + 1;  // keys of the block
  const int kt_lo = lo / AT_KEYS;
  const int kt_hi = lo < hi ? (min(hi, vis_max) + AT_KEYS - 1) / AT_KEYS : kt_lo;

  // queries as the B operand: lane holds head l32, entries 16 kk + 8 hh .. + 7
  const size_t qrow = ((size_t)b * s_q + (active ? i : 0)) * heads + h0 + l32;
  f16x8 qb[AT_D / 16];
  bf16x8 qrb[AT_DR / 16];
#pragma unroll
  for (int kk = 0; kk < AT_D / 16; ++kk)
    qb[kk] = *reinterpret_cast<const f16x8*>(A.q_hat + qrow * AT_D + 16 * kk + 8 * hh);
#pragma unroll
  for (int kk = 0; kk < AT_DR / 16; ++kk)
    qrb[kk] = *reinterpret_cast<const bf16x8*>(A.q_rope + qrow * AT_DR + 16 * kk + 8 * hh);

  // tile loads: thread e < 512 of K^ / V takes row e / 16, chunk e % 16 (two
  // each); thread e < 256 of K^R row e / 8, chunk e % 8.  Buffer loads
  // through a descriptor per tile whose size ends at the last visible row (a
  // bad page: size 0), so rows past it read as zeros with no branch.
  uint4 nk[2], nv[2], nr;
  // a 32-key tile lies in one 64-token page.  The block table is read through
  // the scalar (constant) cache: it does not change during the kernel, and a
  // scalar load does not count among the vector loads the tile waits on.  The
  // page of the next tile is loaded a tile ahead.
  const ConstI32* pages = (const ConstI32*)(A.block_table) + (size_t)b * max_pages;
  int pg_next = kt_lo < kt_hi ? pages[kt_lo * AT_KEYS / QKN_MLA_PAGE_SIZE] : 0;
  // tiles are fetched in order; one at or past kt_hi reads nothing (size 0)
  // and its registers hold zeros, so the loop needs no branch for it
  auto fetch = [&](int kt) {
    const bool real = kt < kt_hi;
    const int pg = pg_next;
    pg_next = pages[min(kt + 1, kt_hi - 1) * AT_KEYS / QKN_MLA_PAGE_SIZE];
    const bool page_ok = pg >= 0 && pg < A.num_pages;
    if (real && !page_ok) err = 1;
    const int nvalid = real ? min(AT_KEYS, vis_max - kt * AT_KEYS) : 0;
    const size_t row0 = (size_t)(page_ok ? pg : 0) * QKN_MLA_PAGE_SIZE + kt * AT_KEYS % QKN_MLA_PAGE_SIZE;
    if (GQA) {
      const uint32_t rb = 2u * A.row_words;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(A.kvg + row0 * A.row_words), 0, page_ok ? nvalid * rb : 0, kRsrcWord3);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = tid + 256 * u, rr = e >> 4, c = e & 15;
        const uint32_t off = rr * rb + 4u * AT_D * g + 16u * c;
        nk[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        nv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 2u * AT_D, 0, 0));
      }
      const int rr = tid >> 3, c = tid & 7;
      nr = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rs, rr * rb + 4u * AT_D * groups + 16u * c, 0, 0));
    } else {
      const uint32_t stride = 2u * AT_D * groups;
      const size_t first = ((size_t)b * A.max_T + kt * AT_KEYS) * groups + g;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<_Float16*>(A.k_hat + first * AT_D), 0, nvalid * stride, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<_Float16*>(A.v + first * AT_D), 0, nvalid * stride, kRsrcWord3);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = tid + 256 * u, rr = e >> 4, c = e & 15;
        nk[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, rr * stride + 16u * c, 0, 0));
        nv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, rr * stride + 16u * c, 0, 0));
      }
      const uint32_t rb = 2u * (A.rank + AT_DR);
      const __amdgpu_buffer_rsrc_t rr_ = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(A.kv + row0 * (A.rank + AT_DR)), 0, page_ok ? nvalid * rb : 0, kRsrcWord3);
      const int rr = tid >> 3, c = tid & 7;
      nr = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rr_, rr * rb + 2u * A.rank + 16u * c, 0, 0));
    }
  };
  auto stash = [&](int slot) {
    uint8_t* buf = smem + slot * AT_TILE;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u, rr = e >> 4, c = e & 15;
      const int at = rr * 256 + ((c ^ kswz(rr)) << 4);
      *reinterpret_cast<uint4*>(buf + at) = nk[u];
      *reinterpret_cast<uint4*>(buf + AT_K_BYTES + AT_R_BYTES + at) = nv[u];
    }
    const int rr = tid >> 3, c = tid & 7;
    *reinterpret_cast<uint4*>(buf + AT_K_BYTES + rr * 128 + ((c ^ rswz(rr)) << 4)) = nr;
  };

  // per-lane read offsets.  QK: key row l32, chunk 2 kk + hh.  PV (V^T, the
  // transposed read of the decode's P.C): within a 16-lane group G16, row
  // t0 = 4 hh + l16 / 4 (and t0 + 8), chunk 4 om + 2 G16 + (l16 % 4) / 2,
  // byte 8 (l16 % 2); rows + 16 ks.
  const int l16 = lane & 15, G16 = (lane >> 4) & 1;
  const int t0 = 4 * hh + (l16 >> 2), c_lo = 2 * G16 + ((l16 & 3) >> 1);
  const uint32_t pv0 = static_cast<uint32_t>(t0 * 256 + 8 * (l16 & 1) + ((c_lo ^ kswz(t0)) << 4));
  const uint32_t pv1 =
      static_cast<uint32_t>((t0 + 8) * 256 + 8 * (l16 & 1) + ((c_lo ^ kswz(t0 + 8)) << 4));

  f32x16 acc[AT_D / 32];
#pragma unroll
  for (int om = 0; om < AT_D / 32; ++om) acc[om] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = A.scale * kLog2e;
  const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};

  // per-lane LDS offsets within a slot: the QK operands (8 normed-key and 4
  // RoPE-key reads) and the PV operands (two transposed reads per product)
  constexpr int NQ = AT_D / 16 + AT_DR / 16, QK_AHEAD = 4;
  uint32_t qk_off[NQ], pv_off[2][AT_D / 32];
#pragma unroll
  for (int n = 0; n < NQ; ++n)
    qk_off[n] = n < AT_D / 16 ? l32 * 256 + (((2 * n + hh) ^ kswz(l32)) << 4)
                              : AT_K_BYTES + l32 * 128 + (((2 * (n - AT_D / 16) + hh) ^ rswz(l32)) << 4);
#pragma unroll
  for (int om = 0; om < AT_D / 32; ++om) {
    pv_off[0][om] = AT_K_BYTES + AT_R_BYTES + (pv0 ^ (64u * om));
    pv_off[1][om] = AT_K_BYTES + AT_R_BYTES + (pv1 ^ (64u * om));
  }
  const LDS_AS uint8_t* lds = (const LDS_AS uint8_t*)smem;

  // S^T of the tile in slot SLOT: 8 products over the normed keys, then 4
  // over the RoPE keys, operands read QK_AHEAD products ahead; fill(n) runs
  // after product n (the softmax of the previous tile)
  auto qk = [&](auto SLOT, auto&& fill) {
    constexpr uint32_t base = decltype(SLOT)::value * AT_TILE;
    auto rd = [&](int n) { return *reinterpret_cast<const LDS_AS f16x8*>(lds + base + qk_off[n]); };
    f16x8 ab[QK_AHEAD];
#pragma unroll
    for (int n = 0; n < QK_AHEAD; ++n) ab[n] = rd(n);
    f32x16 s_ = {};
    Unroll<0, NQ>::run([&](auto N) {
      constexpr int n = decltype(N)::value;
      const f16x8 a = ab[n % QK_AHEAD];
      if constexpr (n + QK_AHEAD < NQ) ab[n % QK_AHEAD] = rd(n + QK_AHEAD);
      if constexpr (n < AT_D / 16)
        s_ = mfma(a, qb[n], s_);
      else
        s_ = mfma(__builtin_bit_cast(bf16x8, a), qrb[n - AT_D / 16], s_);
      fill(N);
      __builtin_amdgcn_sched_barrier(0);
    });
    return s_;
  };
  // O^T += V^T P^T over the tile in slot SLOT
  auto pv = [&](auto SLOT, const f16x8 (&pb)[2]) {
    constexpr uint32_t base = decltype(SLOT)::value * AT_TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int om = 0; om < AT_D / 32; ++om) {
        // the transposed read moves 16-bit words; the words are halves here
        const f16x4 lo4 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(lds + base + 4096u * ks + pv_off[0][om])));
        const f16x4 hi4 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(lds + base + 4096u * ks + pv_off[1][om])));
        const f16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[om] = mfma(a, pb[ks], acc[om]);
      }
    }
  };

  // Software pipeline over three LDS slots (slot of tile kt: (kt - kt_lo) mod
  // 3).  Iteration kt: the loads of tile kt + 2 go out; the QK products of
  // tile kt + 1 run with the softmax of tile kt between them; then the PV
  // products of tile kt; tile kt + 2 is stored into the slot of tile kt - 1
  // and one barrier ends the iteration.  Every active wave takes every tile
  // of the block: a tile past this wave's keys is masked whole, which leaves
  // its max, sum and accumulators as they were; a wave past the last query
  // token only loads and stores tiles.
  if (kt_lo < kt_hi) {
    fetch(kt_lo);  // in flight together with the query loads
    stash(0);
    fetch(kt_lo + 1);
    // the queries are in registers before the tile loop: otherwise the wait
    // for them inside the loop would also wait for the next tile's loads
#pragma unroll
    for (int kk = 0; kk < AT_D / 16; ++kk) asm volatile("" ::"v"(qb[kk]));
#pragma unroll
    for (int kk = 0; kk < AT_DR / 16; ++kk) asm volatile("" ::"v"(qrb[kk]));
    __syncthreads();
    f32x16 sc = {};
    if (!IDLE || active) sc = qk(std::integral_constant<int, 0>{}, [](auto) {});
    stash(1);
    __syncthreads();

    auto iteration = [&](auto SLOT, int kt) {
      constexpr int P = decltype(SLOT)::value;
      fetch(kt + 2);
      // ---- softmax of tile kt (mask, running max, probabilities) between
      // the QK products of tile kt + 1 ----
      float mx = -INFINITY, mc = 0.f;
      f16x8 pb[2];
      auto soft = [&](auto N) {
        constexpr int n = decltype(N)::value;
        if constexpr (n == 0) {
          // register r holds key kt * 32 + r % 4 + 8 (r / 4) + 4 hh
          if (kt * AT_KEYS + AT_KEYS > vis) {  // the tile reaches past this wave's keys
            const int lim = vis - kt * AT_KEYS - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if ((r & 3) + 8 * (r >> 2) >= lim) sc[r] = -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
        } else if constexpr (n == 1) {
          mx = pair_max(mx);
          // the reference m_run moves only when the tile's maximum passes it
          // by more than 2^kLazyLog2 in probability (always on a row's first
          // key): probabilities stay at most 2^kLazyLog2, and the rescale of
          // the accumulators is rare after the first tiles
          const float m_new = fmaxf(m_run, mx);
          if ((m_new - m_run) * c2 > kLazyLog2) {
            if (m_run != -INFINITY) {
              const float al = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
              l_run *= al;
#pragma unroll
              for (int om = 0; om < AT_D / 32; ++om)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[om][r] *= al;
            }
            m_run = m_new;
          }
          mc = m_run == -INFINITY ? 0.f : m_run * c2;
        } else if constexpr (n >= 2 && n < 10) {
          constexpr int r = 2 * (n - 2);
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[r + 1], c2, -mc));
          const f16x2 pr = __builtin_convertvector((f32x2){p0, p1}, f16x2);
          pb[r >> 3][r & 7] = pr[0];
          pb[r >> 3][(r & 7) + 1] = pr[1];
          l_run = __builtin_amdgcn_fdot2(pr, ones, l_run, false);
        }
      };
      // the two waves on a SIMD (two workgroups per CU): the one issuing
      // products goes first, the other's vector work fills the gaps
      if (!IDLE || active) {  // a wave past the last query token only moves tiles
        __builtin_amdgcn_s_setprio(1);
        const f32x16 sc_next = qk(std::integral_constant<int, (P + 1) % 3>{}, soft);
        pv(std::integral_constant<int, P>{}, pb);
        __builtin_amdgcn_s_setprio(0);
        sc = sc_next;
      }
      // tile kt + 2 goes to the slot of tile kt - 1, which every wave
      // finished reading before the previous barrier
      stash((P + 2) % 3);
      __syncthreads();
    };
    for (int kt = kt_lo;;) {
      iteration(std::integral_constant<int, 0>{}, kt);
      if (++kt >= kt_hi) break;
      iteration(std::integral_constant<int, 1>{}, kt);
      if (++kt >= kt_hi) break;
      iteration(std::integral_constant<int, 2>{}, kt);
      if (++kt >= kt_hi) break;
    }
  }

  // ---- o = acc / l (lane: head l32, entries 32 om + r % 4 + 8 (r / 4) + 4 hh);
  // a split with no visible key gives o = 0, lse = -inf ----
  if (active) {
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float ls = l_tot > 0.f ? m_run * A.scale + log2f(l_tot) * kLn2 : -INFINITY;
    const size_t orow = ((size_t)b * s_q + i) * heads + h0 + l32;
    if (A.num_splits == 1) {
#pragma unroll
      for (int om = 0; om < AT_D / 32; ++om) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 x = {acc[om][4 * qd] * inv, acc[om][4 * qd + 1] * inv,
                           acc[om][4 * qd + 2] * inv, acc[om][4 * qd + 3] * inv};
          *reinterpret_cast<f32x4*>(A.o + orow * AT_D + 32 * om + 8 * qd + 4 * hh) = x;
        }
      }
      if (hh == 0) A.lse[orow] = ls;
    } else {
      // a partial is a convex combination of half values: it stays in range
      const size_t prow = orow * A.num_splits + sp;
#pragma unroll
      for (int om = 0; om < AT_D / 32; ++om) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 x = {acc[om][4 * qd] * inv, acc[om][4 * qd + 1] * inv,
                           acc[om][4 * qd + 2] * inv, acc[om][4 * qd + 3] * inv};
          *reinterpret_cast<f16x4*>(A.o_part + prow * AT_D + 32 * om + 8 * qd + 4 * hh) =
              __builtin_convertvector(x, f16x4);
        }
      }
      if (hh == 0) A.lse_part[prow] = ls;
    }
  }
  if (err && A.err_flag && lane == 0) atomicOr(A.err_flag, QKN_FLAG_INDEX);
}

// ---------------------------------------------------------------------------
// combine of the GQA path's half partials (rows of d = 128): 16 lanes per row,
// 4 rows per wave.  M = max_p lse_p, lse = M + ln sum_p e^{lse_p - M},
// o = sum_p e^{lse_p - lse} o_p; every split empty gives o = 0, lse = -inf.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gqa_combine_kernel(const _Float16* __restrict__ o_part,
                                                          const float* __restrict__ lse_part,
                                                          float* __restrict__ o, float* __restrict__ lse,
                                                          int n_rows, int num_splits) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int row = (blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  if (row >= n_rows) return;  // whole 16-lane groups
  const float* lp = lse_part + (size_t)row * num_splits;
  float M = -INFINITY;
  for (int p = l16; p < num_splits; p += 16) M = fmaxf(M, lp[p]);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 16));
  float* out = o + (size_t)row * AT_D + 8 * l16;
  if (M == -INFINITY) {
    *reinterpret_cast<float4*>(out) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(out + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (l16 == 0) lse[row] = -INFINITY;
    return;
  }
  float sum = 0.f;
  for (int p = l16; p < num_splits; p += 16) sum += expf(lp[p] - M);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) sum += __shfl_xor(sum, m, 16);
  const float L = M + logf(sum);
  if (l16 == 0) lse[row] = L;
  const _Float16* op = o_part + (size_t)row * num_splits * AT_D + 8 * l16;
  float acc[8] = {};
  for (int p0 = 0; p0 < num_splits; p0 += 4) {
    f16x8 v[4];
    float wgt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u;
      const float l = p < num_splits ? lp[p] : -INFINITY;
      wgt[u] = l == -INFINITY ? 0.f : expf(l - L);
      v[u] = p < num_splits ? *reinterpret_cast<const f16x8*>(op + (size_t)p * AT_D) : f16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(wgt[u], static_cast<float>(v[u][j]), acc[j]);
  }
  *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// The same merge for many splits: one wave per row; its four 16-lane groups
// take the splits p = 4 k + group, and their sums are added across the
// groups at the end.
__global__ __launch_bounds__(256) void gqa_combine_wide_kernel(const _Float16* __restrict__ o_part,
                                                               const float* __restrict__ lse_part,
                                                               float* __restrict__ o,
                                                               float* __restrict__ lse, int n_rows,
                                                               int num_splits) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, sub = lane >> 4;
  const int row = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (row >= n_rows) return;  // whole waves
  const float* lp = lse_part + (size_t)row * num_splits;
  float M = -INFINITY;
  for (int p = lane; p < num_splits; p += 64) M = fmaxf(M, lp[p]);
  M = wave_max(M);
  float* out = o + (size_t)row * AT_D + 8 * l16;
  if (M == -INFINITY) {
    if (sub == 0) {
      *reinterpret_cast<float4*>(out) = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(out + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (lane == 0) lse[row] = -INFINITY;
    return;
  }
  float sum = 0.f;
  for (int p = lane; p < num_splits; p += 64) sum += expf(lp[p] - M);
  sum = wave_sum(sum);
  const float L = M + logf(sum);
  if (lane == 0) lse[row] = L;
  const _Float16* op = o_part + (size_t)row * num_splits * AT_D + 8 * l16;
  float acc[8] = {};
  for (int p0 = sub; p0 < num_splits; p0 += 16) {
    f16x8 v[4];
    float wgt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + 4 * u;
      const float l = p < num_splits ? lp[p] : -INFINITY;
      wgt[u] = l == -INFINITY ? 0.f : expf(l - L);
      v[u] = p < num_splits ? *reinterpret_cast<const f16x8*>(op + (size_t)p * AT_D) : f16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(wgt[u], static_cast<float>(v[u][j]), acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] += __shfl_xor(acc[j], 16);
    acc[j] += __shfl_xor(acc[j], 32);
  }
  if (sub == 0) {
    *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

template <int NT>
hipError_t launch_expand_nt(const qkn_mla_dims& d, const void* kv, const float* alpha_k,
                            const int32_t* block_table, const int32_t* seq_lens, const float* w_k,
                            const float* w_v, const float* gamma_k, void* k_hat, void* v,
                            int32_t* err_flag, hipStream_t s) {
  constexpr int D = NT * 32;
  constexpr int KC = ex_chunk_rows(D);
  const int lds = 3 * KC * (D + EX_PAD) * 2;
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&prefill_expand_kernel<NT>), lds);
  if (e != hipSuccess) return e;
  const int max_T = d.max_pages_per_seq * QKN_MLA_PAGE_SIZE;
  // blocks of NT column tiles: (token block, sequence and group, column block and keys | values)
  hipLaunchKernelGGL(prefill_expand_kernel<NT>,
                     dim3(cdiv(max_T, EX_TOK), d.batch * d.groups, 2 * (d.head_dim / D)),
                     dim3(64 * EX_WAVES), lds, s, static_cast<const uint16_t*>(kv), alpha_k,
                     block_table, seq_lens, w_k, w_v, gamma_k, static_cast<_Float16*>(k_hat),
                     static_cast<_Float16*>(v), err_flag, d.groups, d.rank, d.rope_dim,
                     d.max_pages_per_seq, d.num_pages, max_T, d.head_dim);
  return hipGetLastError();
}

// Query tokens per workgroup: 4, or fewer when s_q is smaller and the heads of
// one group fill the other waves (so no wave idles at s_q = 1 or 2).
void set_shape(const qkn_mla_dims& d, AttendArgs& A) {
  const int blocks_per_group = d.heads / d.groups / 32;
  int tpw = 4;
  while (tpw > 1 && tpw / 2 >= d.s_q && blocks_per_group % (8 / tpw) == 0) tpw /= 2;
  A.tpw = tpw;
  A.token_groups = cdiv(d.s_q, tpw);
  A.head_groups = d.heads / 32 / (4 / tpw);
}

}  // namespace

bool prefill_supported(const qkn_mla_dims& d) {
  return d.cache_dtype == QKN_BF16 && d.head_dim == AT_D && d.rope_dim == AT_DR && d.rank == AT_R &&
         (d.heads / d.groups) % 32 == 0;
}

hipError_t launch_prefill_query(const qkn_mla_dims& d, const float* q, const float* q_rope,
                                const int32_t* q_pos, const float* gamma_q, const float* gamma_qr,
                                void* q_hat, void* q_rope_normed, hipStream_t s) {
  hipLaunchKernelGGL(prefill_query_kernel, dim3(d.batch * d.s_q * (d.heads / 16)), dim3(256), 0, s,
                     q, q_rope, q_pos,
                     gamma_q, gamma_qr, static_cast<_Float16*>(q_hat),
                     static_cast<uint16_t*>(q_rope_normed), d.heads, d.eps, d.rope_theta);
  return hipGetLastError();
}

hipError_t launch_prefill_expand(const qkn_mla_dims& d, const void* kv, const float* alpha_k,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const float* w_k, const float* w_v, const float* gamma_k,
                                 void* k_hat, void* v, int32_t* err_flag, hipStream_t s) {
  // 64 columns per block: twice the blocks of whole-width ones (256 for two
  // 8192-token sequences), each staging half of W_g
  return launch_expand_nt<2>(d, kv, alpha_k, block_table, seq_lens, w_k, w_v, gamma_k,
                                     k_hat, v, err_flag, s);
}

hipError_t launch_prefill_attend(const qkn_mla_dims& d, const void* q_hat, const void* q_rope_normed,
                                 const void* k_hat, const void* v, const void* kv,
                                 const int32_t* block_table, const int32_t* seq_lens, float* o,
                                 float* lse, int32_t* err_flag, hipStream_t s) {
  AttendArgs A{};
  A.q_hat = static_cast<const _Float16*>(q_hat);
  A.q_rope = static_cast<const uint16_t*>(q_rope_normed);
  A.k_hat = static_cast<const _Float16*>(k_hat);
  A.v = static_cast<const _Float16*>(v);
  A.kv = static_cast<const uint16_t*>(kv);
  A.block_table = block_table;
  A.seq_lens = seq_lens;
  A.o = o;
  A.lse = lse;
  A.err_flag = err_flag;
  A.batch = d.batch;
  A.s_q = d.s_q;
  A.heads = d.heads;
  A.groups = d.groups;
  A.max_pages = d.max_pages_per_seq;
  A.num_pages = d.num_pages;
  A.max_T = d.max_pages_per_seq * QKN_MLA_PAGE_SIZE;
  set_shape(d, A);
  A.num_splits = 1;
  A.rank = d.rank;
  A.scale = d.softmax_scale;
  auto kernel = d.s_q % A.tpw ? attend_kernel<false, true> : attend_kernel<false, false>;
  hipLaunchKernelGGL(kernel, dim3(d.batch * A.token_groups * A.head_groups), dim3(256),
                     0, s, A);
  return hipGetLastError();
}

bool gqa_supported(const qkn_mla_dims& d) {
  return d.cache_dtype == QKN_BF16 && d.head_dim == AT_D && d.rope_dim == AT_DR && d.rank % 16 == 0 &&
         (d.heads / d.groups) % 32 == 0;
}

int gqa_row_words(const qkn_mla_dims& d) { return 2 * d.head_dim * d.groups + d.rope_dim; }

hipError_t launch_gqa_append(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                             const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                             const int32_t* block_table, const float* w_k, const float* w_v,
                             const float* gamma_k, const float* gamma_kr, void* kvg,
                             int32_t* err_flag, hipStream_t s) {
  if (n_tokens <= kGqaSmallAppend && d.rank <= GS_RG * GS_MAX_ROWS) {
    // tokens per block: each block streams all of its W_g once, so several
    // tokens share it once there are more blocks than CUs
    const int tpb = n_tokens >= 256 ? 4 : n_tokens >= 128 ? 2 : 1;
    auto kernel = tpb == 4 ? gqa_append_small_kernel<4>
                : tpb == 2 ? gqa_append_small_kernel<2> : gqa_append_small_kernel<1>;
    hipLaunchKernelGGL(kernel, dim3(cdiv(n_tokens, tpb), d.groups, 2), dim3(1024), 0, s, c_new,
                       k_rope_new, seq_idx, pos, block_table, w_k, w_v, gamma_k, gamma_kr,
                       static_cast<uint16_t*>(kvg), err_flag, n_tokens, d.batch, d.groups, d.rank,
                       d.max_pages_per_seq, d.num_pages, d.eps, d.rope_theta);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gqa_append_kernel, dim3(cdiv(n_tokens, 32), d.groups, 2), dim3(64 * GA_WAVES), 0, s, c_new,
                     k_rope_new, seq_idx, pos, block_table, w_k, w_v, gamma_k, gamma_kr,
                     static_cast<uint16_t*>(kvg), err_flag, n_tokens, d.batch, d.groups, d.rank,
                     d.max_pages_per_seq, d.num_pages, d.eps, d.rope_theta);
  return hipGetLastError();
}

hipError_t launch_gqa_attend(const qkn_mla_dims& d, const void* q_hat, const void* q_rope_normed,
                             const void* kvg, const int32_t* block_table, const int32_t* seq_lens,
                             int num_splits, void* o_part, float* lse_part, float* o, float* lse,
                             int32_t* err_flag, hipStream_t s) {
  AttendArgs A{};
  A.q_hat = static_cast<const _Float16*>(q_hat);
  A.q_rope = static_cast<const uint16_t*>(q_rope_normed);
  A.kvg = static_cast<const uint16_t*>(kvg);
  A.block_table = block_table;
  A.seq_lens = seq_lens;
  A.o = o;
  A.lse = lse;
  A.o_part = static_cast<_Float16*>(o_part);
  A.lse_part = lse_part;
  A.err_flag = err_flag;
  A.batch = d.batch;
  A.s_q = d.s_q;
  A.heads = d.heads;
  A.groups = d.groups;
  A.max_pages = d.max_pages_per_seq;
  A.num_pages = d.num_pages;
  A.max_T = d.max_pages_per_seq * QKN_MLA_PAGE_SIZE;
  set_shape(d, A);
  A.num_splits = num_splits;
  A.row_words = gqa_row_words(d);
  A.rank = d.rank;
  A.scale = d.softmax_scale;
  // (sequence, split) pairs padded to a multiple of 8 (one per XCD), each
  // with its token and head blocks
  const long long blocks = 8LL * cdiv(d.batch * num_splits, 8) * A.token_groups * A.head_groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  auto kernel = d.s_q % A.tpw ? attend_kernel<true, true> : attend_kernel<true, false>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || num_splits == 1) return e;
  const int rows = d.batch * d.s_q * d.heads;
  if (num_splits >= 32) {  // a wave per row: the walk over many partials in four lane groups
    hipLaunchKernelGGL(gqa_combine_wide_kernel, dim3(cdiv(rows, 4)), dim3(256), 0, s,
                       static_cast<const _Float16*>(o_part), lse_part, o, lse, rows, num_splits);
  } else {
    hipLaunchKernelGGL(gqa_combine_kernel, dim3(cdiv(rows, 16)), dim3(256), 0, s,
                       static_cast<const _Float16*>(o_part), lse_part, o, lse, rows, num_splits);
  }
  return hipGetLastError();
}

}  // namespace qkn
