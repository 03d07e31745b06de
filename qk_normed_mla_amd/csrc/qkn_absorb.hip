// qkn_mla_absorb_query: fold the static norm weights into the query and absorb
// W^K_g (QK-Normed MLA summary, "Metodologia" item 1), the per-row inverse RMS
// alpha^q (decode-logit equation) and the separately normed, rotated RoPE query
// (item 4).
//
// q~[row, m] = sum_j W^K_g[m, j] * (gamma_q[j] gamma_k[g, j] q[row, j]) is a
// GEMM per KV group, [rows_g x d] . [d x r], in 64 x 128 tiles with both
// operands staged through LDS.
//   bf16 q~ (absorb_split, one launch): every float32 operand x is split into
//     bf16 words hi = bf16(x), lo = bf16(x - hi), and the product is taken as
//     hi.hi + hi.lo + lo.hi on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
//     float32 accumulate).  The dropped lo.lo term and the rounding of lo are
//     about 2^-17 of the product, far below the bf16 storage step of q~, at a
//     sixteenth of the float32 matrix cost per product.  The same blocks (8
//     waves) also form alpha^q and the RoPE query of a share of their rows,
//     while the first operand loads are in flight.
//   float32 q~ (absorb_gemm + absorb_rows): the float32 matrix cores
//     (v_mfma_f32_32x32x2_f32); then alpha^q and the RoPE query, one wave per
//     query row, four heads of one query token per block.
#include <algorithm>

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


// ---------------------------------------------------------------------------
// split-bf16 GEMM with the row work folded in (bf16 q~)
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int SK = 128;       // head-dim entries staged per step (all of d <= 128 at once)
constexpr int SLD = SK + 8;   // LDS row of bf16 words (272 B: 16 rows hit distinct banks)
constexpr int SPLIT_LDS = (2 * TM + 2 * TN) * SLD * 2 + SK * 4 + 2 * TM * 4;  // bytes

// hi/lo bf16 words of four floats
__device__ __forceinline__ void split4(float4 v, bf16x4& hi, bf16x4& lo) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  hi = __builtin_convertvector(x, bf16x4);
  const f32x4 r = x - __builtin_convertvector(hi, f32x4);
  lo = __builtin_convertvector(r, bf16x4);
}

// Row work of one wave: alpha^q and the normed, rotated RoPE query of up to
// four global query rows (rows[u] < 0: none).  load() issues every load of the
// batch; finish() does the arithmetic and the stores.  The angles of token
// angle_tok for dims lane and lane + 64 are kept and formed again only when
// the token changes (double precision: at positions of 2^18 a float angle is
// off by ~1e-2 rad).
constexpr int QR_BATCH = 4;
struct QueryRows {
  int row[QR_BATCH], tok[QR_BATCH], pos[QR_BATCH];
  float qv[QR_BATCH][8];             // head_dim <= 512
  float xa[QR_BATCH][2], xb[QR_BATCH][2];  // dims j and j + d_R / 2, j = lane + 64 k
  float ga[2], gb[2];                      // gamma_qR at those dims

  __device__ __forceinline__ void load(const float* __restrict__ q, const float* __restrict__ q_rope,
                                       const int32_t* __restrict__ q_pos,
                                       const float* __restrict__ gamma_qr, int head_dim, int rope_dim,
                                       int lane) {
    const int half = rope_dim / 2;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = lane + 64 * k;
      ga[k] = j < half ? gamma_qr[j] : 0.f;
      gb[k] = j < half ? gamma_qr[j + half] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < QR_BATCH; ++u) {
      const size_t r = row[u] >= 0 ? (size_t)row[u] : 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = lane + 64 * k;
        qv[u][k] = (row[u] >= 0 && j < head_dim) ? q[r * head_dim + j] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int j = lane + 64 * k;
        const bool ok = row[u] >= 0 && j < half;
        xa[u][k] = ok ? q_rope[r * rope_dim + j] : 0.f;
        xb[u][k] = ok ? q_rope[r * rope_dim + j + half] : 0.f;
      }
      pos[u] = (row[u] >= 0 && rope_dim > 0) ? q_pos[tok[u]] : 0;
    }
  }

  __device__ __forceinline__ void finish(float* __restrict__ alpha_q,
                                         uint16_t* __restrict__ q_rope_out, int& angle_tok,
                                         float (&cs)[2], float (&sn)[2], int head_dim, int rope_dim,
                                         float eps, float theta, int lane) {
    const int half = rope_dim / 2;
#pragma unroll
    for (int u = 0; u < QR_BATCH; ++u) {
      if (row[u] < 0) continue;  // uniform
      const size_t r = (size_t)row[u];
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) ss = fmaf(qv[u][k], qv[u][k], ss);
      ss = wave_sum(ss);
      if (lane == 0) alpha_q[r] = 1.0f / sqrtf(ss / (float)head_dim + eps);
      if (rope_dim == 0) continue;
      if (tok[u] != angle_tok) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int j = lane + 64 * k;
          cs[k] = 1.f;
          sn[k] = 0.f;
          if (j < half && theta != 0.f) rope_cos_sin<false>(pos[u], j, rope_dim, theta, &cs[k], &sn[k]);
        }
        angle_tok = tok[u];
      }
      float sr = 0.f;
#pragma unroll
      for (int k = 0; k < 2; ++k) sr = fmaf(xa[u][k], xa[u][k], fmaf(xb[u][k], xb[u][k], sr));
      sr = wave_sum(sr);
      const float inv = 1.0f / sqrtf(sr / (float)rope_dim + eps);
      uint16_t* out = q_rope_out + r * rope_dim;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int j = lane + 64 * k;
        if (j < half) {
          const float x1 = xa[u][k] * inv * ga[k];
          const float x2 = xb[u][k] * inv * gb[k];
          out[j] = f32_to_bf16(x1 * cs[k] - x2 * sn[k]);
          out[j + half] = f32_to_bf16(x2 * cs[k] + x1 * sn[k]);
        }
      }
    }
  }
};

// Block of 8 waves: 64-row x 128-column tiles of q~ for one group, wave
// (wr, wc) = (w / 4, w % 4) owning rows 32 wr .. +31 and columns 32 wc .. +31
// (one 32 x 32 tile) of each.  A block takes `tiles` consecutive row tiles of
// its column block: with d <= 128 the W^K_g tile is split into hi/lo words in
// LDS once and kept, and the next row tile's query loads are issued before the
// current tile's products.  Per step of 128 head-dim entries the query rows
// (times gamma_q gamma_k) are split into hi/lo words as they are stored to LDS.
// Block (x, y) of group g also forms alpha^q and the RoPE query of its share of
// each tile's rows (rows y * share .. of the tile), so every query row is done
// once; those loads go out ahead of the arithmetic that needs them.  A
// finished tile is written back through LDS in 16-byte pieces.
constexpr int SW = 8;  // waves per block
template <bool KEEP>  // d <= 128: one step, the W^K_g tile kept across row tiles
__global__ __launch_bounds__(64 * SW) void absorb_split(
    const float* __restrict__ q, const float* __restrict__ q_rope,
    const int32_t* __restrict__ q_pos, const float* __restrict__ w_k,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_k,
    const float* __restrict__ gamma_qr, uint16_t* __restrict__ q_tilde,
    float* __restrict__ alpha_q, uint16_t* __restrict__ q_rope_out, int rows_per_group,
    int heads, int heads_per_group, int head_dim, int rank, int rope_dim, float eps,
    float theta, int tiles) {
  constexpr int NT = 64 * SW;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint16_t* Ah = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Al = Ah + TM * SLD;
  uint16_t* Bh = Al + TM * SLD;
  uint16_t* Bl = Bh + TN * SLD;
  float* fold = reinterpret_cast<float*>(Bl + TN * SLD);  // gamma_q gamma_k of the step
  const int g = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;
  const int m0 = blockIdx.y * TN;
  const float* wg = w_k + (size_t)g * rank * head_dim;
  const float* gk = gamma_k + (size_t)g * head_dim;
  const int t_lo = blockIdx.x * tiles;
  const int t_hi = min(cdiv(rows_per_group, TM), t_lo + tiles);

  // global row and query token of group row n (n < rows_per_group, else -1)
  auto grow_of = [&](int n) {
    const int bi = n / heads_per_group, hl = n % heads_per_group;
    return n < rows_per_group ? bi * heads + g * heads_per_group + hl : -1;
  };

  // the block's share of each tile's row work, in batches of SW * QR_BATCH rows
  const int share = cdiv(TM, gridDim.y);
  const int r_lo = min(TM, (int)blockIdx.y * share), r_hi = min(TM, r_lo + share);
  QueryRows qr;
  auto pick_rows = [&](int n0, int base) {
#pragma unroll
    for (int u = 0; u < QR_BATCH; ++u) {
      const int lr = base + wave + SW * u;
      qr.row[u] = lr < r_hi ? grow_of(n0 + lr) : -1;
      qr.tok[u] = lr < r_hi ? (n0 + lr) / heads_per_group : 0;
    }
  };

  // operands of a step: A 64 x 128 floats = 2048 float4 (4 per thread), B 128 x 128 (8)
  constexpr int NA = TM * SK / 4 / NT, NB = TN * SK / 4 / NT;
  float4 ra[NA], rb[NB];
  auto fetch_a = [&](int n0, int k0) {
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int e = tid + NT * u, r = e >> 5, k = k0 + 4 * (e & 31);
      const int gr = grow_of(n0 + r);
      ra[u] = (gr >= 0 && k < head_dim) ? *reinterpret_cast<const float4*>(q + (size_t)gr * head_dim + k)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto fetch_b = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int e = tid + NT * u, r = e >> 5, k = k0 + 4 * (e & 31);
      const int m = m0 + r;
      rb[u] = (m < rank && k < head_dim) ? *reinterpret_cast<const float4*>(wg + (size_t)m * head_dim + k)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < SK) fold[tid] = k0 + tid < head_dim ? gamma_q[k0 + tid] * gk[k0 + tid] : 0.f;
  };
  auto stash_a = [&]() {
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int e = tid + NT * u, c = 4 * (e & 31), o = (e >> 5) * SLD + c;
      float4 v = ra[u];
      v.x *= fold[c];
      v.y *= fold[c + 1];
      v.z *= fold[c + 2];
      v.w *= fold[c + 3];
      bf16x4 hi, lo;
      split4(v, hi, lo);
      *reinterpret_cast<bf16x4*>(&Ah[o]) = hi;
      *reinterpret_cast<bf16x4*>(&Al[o]) = lo;
    }
  };
  auto stash_b = [&]() {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int e = tid + NT * u, o = (e >> 5) * SLD + 4 * (e & 31);
      bf16x4 hi, lo;
      split4(rb[u], hi, lo);
      *reinterpret_cast<bf16x4*>(&Bh[o]) = hi;
      *reinterpret_cast<bf16x4*>(&Bl[o]) = lo;
    }
  };

  if (t_lo >= t_hi) return;  // uniform: no tile for this block
  pick_rows(t_lo * TM, r_lo);
  qr.load(q, q_rope, q_pos, gamma_qr, head_dim, rope_dim, lane);
  fetch_a(t_lo * TM, 0);
  fetch_b(0);
  int angle_tok = -1;
  float cs[2], sn[2];
  const int r = lane & 31, kh = lane >> 5;
  for (int t = t_lo; t < t_hi; ++t) {
    const int n0 = t * TM;
    qr.finish(alpha_q, q_rope_out, angle_tok, cs, sn, head_dim, rope_dim, eps, theta, lane);
    // further batches when the share is larger than one batch (few column blocks)
    for (int base = r_lo + SW * QR_BATCH; base < r_hi; base += SW * QR_BATCH) {
      pick_rows(n0, base);
      qr.load(q, q_rope, q_pos, gamma_qr, head_dim, rope_dim, lane);
      qr.finish(alpha_q, q_rope_out, angle_tok, cs, sn, head_dim, rope_dim, eps, theta, lane);
    }
    f32x16 acc = {};
    for (int k0 = 0; k0 < (KEEP ? SK : head_dim); k0 += SK) {
      if (k0 > 0) {
        __syncthreads();  // every wave is done with the previous step's tiles
        fetch_a(n0, k0);
        fetch_b(k0);
      }
      __syncthreads();  // the fold factors are visible; the previous tile left LDS
      stash_a();
      if (!KEEP || t == t_lo) stash_b();
      __syncthreads();
      if (KEEP && t + 1 < t_hi) {
        // the next tile's operand and row-work loads, in flight during the products
        fetch_a(n0 + TM, 0);
        pick_rows(n0 + TM, r_lo);
        qr.load(q, q_rope, q_pos, gamma_qr, head_dim, rope_dim, lane);
      }
#pragma unroll
      for (int ks = 0; ks < SK / 16; ++ks) {
        if (k0 + 16 * ks >= head_dim) break;  // uniform
        // A operand: row 32 wr + r, entries 16 ks + 8 kh .. + 7; B operand: W^K row (column of q~)
        const int ao = (32 * wr + r) * SLD + 16 * ks + 8 * kh;
        const int bo = (32 * wc + r) * SLD + 16 * ks + 8 * kh;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Ah[ao]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Al[ao]);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Bh[bo]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Bl[bo]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
      }
    }
    // The tile goes out through LDS (in the place of the A operand words) as
    // whole 16-byte pieces of q~ rows.  D[i][j]: column j = lane % 32, row
    // i = (reg % 4) + 8 (reg / 4) + 4 (lane / 32).
    __syncthreads();  // every wave is done with the operands
    uint16_t* T = Ah;  // [TM][SLD]
#pragma unroll
    for (int reg = 0; reg < 16; ++reg)
      T[(32 * wr + (reg & 3) + 8 * (reg >> 2) + 4 * kh) * SLD + 32 * wc + r] = f32_to_bf16(acc[reg]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TM * TN / 8 / NT; ++u) {
      const int e = tid + NT * u, row = e >> 4, c = 8 * (e & 15);
      const int gr = grow_of(n0 + row);
      if (gr >= 0 && m0 + c < rank)  // rank is a multiple of 8
        *reinterpret_cast<uint4*>(q_tilde + (size_t)gr * rank + m0 + c) =
            *reinterpret_cast<const uint4*>(&T[row * SLD + c]);
    }
  }
}

// Wave-independent variant for d = 128, rank a multiple of 128 and d_R a
// multiple of 32 up to 128 (the workloads' shapes).  A block of 8 waves (one
// block per CU) stages one 128-column block of W^K_g, times gamma_q gamma_k,
// as hi/lo bf16 words in LDS (69.6 KB) and needs no barrier after that: each
// wave takes whole 32-row tiles of q~ on its own.  The product is taken transposed,
// q~^T = W . q^T, so that the W rows are the first operand (read from LDS)
// and the query rows the second one, loaded straight from HBM into the
// operand layout (lane l: row l % 32, head-dim entries 16 s + 8 (l / 32) ..
// + 7 of step s) and split in registers; the accumulator then holds, per lane,
// runs of four consecutive q~ columns of one row, and the two lanes of a row
// trade halves to store 16-byte pieces.  The next tile's query loads go out
// step by step as the current tile's operand words are formed.  alpha^q comes
// from the same registers (the two lanes of a row hold its two halves); the
// RoPE query of a share of each tile's rows (per column block) is formed four
// rows per wave step, 16 lanes on a row, its loads issued with the tile's
// first products.
constexpr int WCB = 128;          // q~ columns per block
constexpr int WLD = 128 + 8;      // LDS row of bf16 words (272 B: as SLD)
constexpr int WAVE_LDS = 2 * WCB * WLD * 2;  // bytes: hi and lo words
constexpr int WROWS = 32;         // query rows per wave tile
constexpr int RCH = 8;            // RoPE rows per chunk
constexpr int WW = 8;             // waves per block (one block per CU)

__global__ __launch_bounds__(64 * WW) __attribute__((amdgpu_waves_per_eu(2, 2))) void absorb_wave(
    const float* __restrict__ q, const float* __restrict__ q_rope,
    const int32_t* __restrict__ q_pos, const float* __restrict__ w_k,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_k,
    const float* __restrict__ gamma_qr, uint16_t* __restrict__ q_tilde,
    float* __restrict__ alpha_q, uint16_t* __restrict__ q_rope_out, int rows_per_group,
    int heads, int heads_per_group, int rank, int rope_dim, float eps, float theta) {
  constexpr int D = 128;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint16_t* Wh = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Wl = Wh + WCB * WLD;
  const int g = blockIdx.z, cb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int m0 = cb * WCB;
  const int n_tiles = cdiv(rows_per_group, WROWS);
  const int t_step = gridDim.x * WW;
  const int t0 = blockIdx.x * WW + wave;

  auto grow_of = [&](int n) {  // global query row of group row n, -1 past the end
    const int bi = n / heads_per_group, hl = n - bi * heads_per_group;
    return n < rows_per_group ? bi * heads + g * heads_per_group + hl : -1;
  };
  // Query operand of tile t, lane (r, h): row r of the tile, entries
  // 16 s + 8 h .. + 7 of step s.  A row past the end reads row 0 instead: a
  // q~ row depends on its own query row only, and such rows are not stored.
  auto row_ptr = [&](int t) {
    const int gr = grow_of(t * WROWS + r);
    return q + (size_t)(gr >= 0 ? gr : 0) * D + 8 * h;
  };
  float4 raw[8][2];
  const float* qp = row_ptr(t0 < n_tiles ? t0 : 0);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    raw[s][0] = *reinterpret_cast<const float4*>(qp + 16 * s);
    raw[s][1] = *reinterpret_cast<const float4*>(qp + 16 * s + 4);
  }

  // stage W^K_g rows m0 .. m0 + 127 times gamma_q gamma_k as hi/lo words
  {
    const float* wg = w_k + ((size_t)g * rank + m0) * D;
    const float* gk = gamma_k + (size_t)g * D;
    const int k4 = 4 * (tid & 31);
    const float4 f = make_float4(gamma_q[k4] * gk[k4], gamma_q[k4 + 1] * gk[k4 + 1],
                                 gamma_q[k4 + 2] * gk[k4 + 2], gamma_q[k4 + 3] * gk[k4 + 3]);
    constexpr int NW = WCB * D / 4 / (64 * WW);  // float4 of the block's W rows per thread
    float4 wv[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u)
      wv[u] = *reinterpret_cast<const float4*>(wg + (size_t)((tid >> 5) + 2 * WW * u) * D + k4);
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      float4 v = wv[u];
      v.x *= f.x;
      v.y *= f.y;
      v.z *= f.z;
      v.w *= f.w;
      bf16x4 hi, lo;
      split4(v, hi, lo);
      const int o = ((tid >> 5) + 2 * WW * u) * WLD + k4;
      *reinterpret_cast<bf16x4*>(&Wh[o]) = hi;
      *reinterpret_cast<bf16x4*>(&Wl[o]) = lo;
    }
  }
  __syncthreads();  // the only barrier: from here on the waves are independent

  // RoPE rows of each tile for this column block: rows rr_lo .. rr_hi - 1,
  // four per wave step.  Lane (rq, jj) = (lane / 16, lane % 16) takes row
  // rq of the step and the pairs (j, j + d_R / 2), j = jj + 16 p, p < d_R / 32;
  // the row's sum of squares is reduced over its 16 lanes.  A lane keeps the
  // angles of the query token of its last row and forms them again when the
  // token changes.
  const int share = cdiv(WROWS, (int)gridDim.y);
  const int rr_lo = min(WROWS, cb * share), rr_hi = min(WROWS, rr_lo + share);
  const int half = rope_dim / 2;
  const int np_ = half / 16;  // pairs per lane, 1 .. 4 (d_R a multiple of 32, at most 128)
  const int rq = lane >> 4, jj = lane & 15;
  float ga[4], gb[4], cs[4], sn[4];
  double om[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int j = jj + 16 * pp;
    const bool ok = pp < np_;
    ga[pp] = ok ? gamma_qr[j] : 0.f;
    gb[pp] = ok ? gamma_qr[j + half] : 0.f;
    om[pp] = (ok && theta != 0.f) ? rope_omega(j, rope_dim, theta) : 0.0;
    cs[pp] = 1.f;
    sn[pp] = 0.f;
  }
  int angle_tok = -1;
  constexpr int RST = RCH / 4;  // wave steps per chunk
  float xa[RST][4], xb[RST][4];
  auto rope_load = [&](int n0, int c0) {
#pragma unroll
    for (int u = 0; u < RST; ++u) {
      const int lr = min(c0 + 4 * u + rq, WROWS - 1);
      const int gr = lr < rr_hi ? grow_of(n0 + lr) : -1;
      const float* x = q_rope + (size_t)(gr >= 0 ? gr : 0) * rope_dim;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int j = pp < np_ ? jj + 16 * pp : 0;
        xa[u][pp] = x[j];
        xb[u][pp] = x[j + half];
      }
    }
  };
  auto rope_finish = [&](int n0, int c0) {
#pragma unroll
    for (int u = 0; u < RST; ++u) {
      const int lr = c0 + 4 * u + rq;
      const int gr = lr < rr_hi ? grow_of(n0 + lr) : -1;
      float ss = 0.f;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
        if (pp < np_) ss = fmaf(xa[u][pp], xa[u][pp], fmaf(xb[u][pp], xb[u][pp], ss));
      // the 16 lanes of a row: quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror
      ss += dpp_partner<0xB1>(ss);
      ss += dpp_partner<0x4E>(ss);
      ss += dpp_partner<0x141>(ss);
      ss += dpp_partner<0x140>(ss);
      const float inv = 1.0f / sqrtf(ss / (float)rope_dim + eps);
      if (gr >= 0) {
        const int tok = (n0 + lr) / heads_per_group;
        if (tok != angle_tok) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
            if (pp < np_ && theta != 0.f) rope_cos_sin_at<false>(q_pos[tok], om[pp], &cs[pp], &sn[pp]);
          angle_tok = tok;
        }
        uint16_t* out = q_rope_out + (size_t)gr * rope_dim;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          if (pp < np_) {
            const int j = jj + 16 * pp;
            const float x1 = xa[u][pp] * inv * ga[pp], x2 = xb[u][pp] * inv * gb[pp];
            out[j] = f32_to_bf16(x1 * cs[pp] - x2 * sn[pp]);
            out[j + half] = f32_to_bf16(x2 * cs[pp] + x1 * sn[pp]);
          }
        }
      }
    }
  };
  const bool has_rope = rope_dim > 0 && rr_lo < rr_hi;

  for (int t = t0; t < n_tiles; t += t_step) {
    // the W words are read from LDS again for every tile (hoisted out of the
    // loop they would need 256 registers)
    asm volatile("" ::: "memory");
    const int n0 = t * WROWS;
    const int gr = grow_of(n0 + r);
    if (has_rope) rope_load(n0, rr_lo);
    // the next tile's rows (on the last tile: this tile's again, unused)
    const float* np = row_ptr(t + t_step < n_tiles ? t + t_step : t);
    f32x16 acc[4] = {};
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 a0 = raw[s][0], a1 = raw[s][1];
      ss = fmaf(a0.x, a0.x, fmaf(a0.y, a0.y, fmaf(a0.z, a0.z, fmaf(a0.w, a0.w, ss))));
      ss = fmaf(a1.x, a1.x, fmaf(a1.y, a1.y, fmaf(a1.z, a1.z, fmaf(a1.w, a1.w, ss))));
      bf16x4 h0, l0, h1, l1;
      split4(a0, h0, l0);
      split4(a1, h1, l1);
      const bf16x8 bh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 bl = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
      raw[s][0] = *reinterpret_cast<const float4*>(np + 16 * s);
      raw[s][1] = *reinterpret_cast<const float4*>(np + 16 * s + 4);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int o = (32 * ct + r) * WLD + 16 * s + 8 * h;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Wh[o]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Wl[o]);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[ct], 0, 0, 0);
      }
    }
    // alpha^q of row r: the lanes r and r + 32 hold its two halves
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
      const float tot = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
      if (cb == 0 && h == 0 && gr >= 0) alpha_q[gr] = 1.0f / sqrtf(tot / (float)D + eps);
    }
    // D[c][row]: lane (r, h), register 4 a + b holds column 32 ct + 8 a + 4 h + b
    // of row r.  For a = 2 p, 2 p + 1 the two lanes of a row trade halves
    // (v_permlane32_swap), so that lane (r, h) holds columns 16 p + 8 h .. + 7
    // and stores them as one 16-byte piece.
    {
      uint16_t* out = q_tilde + (size_t)(gr >= 0 ? gr : 0) * rank + m0 + 8 * h;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const f32x4 v0 = {acc[ct][8 * p], acc[ct][8 * p + 1], acc[ct][8 * p + 2], acc[ct][8 * p + 3]};
          const f32x4 v1 = {acc[ct][8 * p + 4], acc[ct][8 * p + 5], acc[ct][8 * p + 6], acc[ct][8 * p + 7]};
          const bf16x4 w0 = __builtin_convertvector(v0, bf16x4), w1 = __builtin_convertvector(v1, bf16x4);
          const uint2 x = __builtin_bit_cast(uint2, w0), y = __builtin_bit_cast(uint2, w1);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
          if (gr >= 0)
            *reinterpret_cast<uint4*>(out + 32 * ct + 16 * p) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
    }
    if (has_rope) {
      rope_finish(n0, rr_lo);
      for (int c0 = rr_lo + RCH; c0 < rr_hi; c0 += RCH) {  // shares larger than one chunk
        rope_load(n0, c0);
        rope_finish(n0, c0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 path
// ---------------------------------------------------------------------------
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
    if (theta != 0.f) rope_cos_sin<std::is_same<OutT, float>::value>(q_pos[tok], j, rope_dim, theta, &c, &s);
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
  if (d.cache_dtype == QKN_BF16) {
    if (d.rope_dim / 2 > 128) return hipErrorInvalidValue;
    const int hpg = d.heads / d.groups;
    const int rows_per_group = d.batch * d.s_q * hpg;
    const int wave_cols = d.rank / WCB, n_tiles = cdiv(rows_per_group, WROWS);
    if (d.head_dim == 128 && d.rank % WCB == 0 && d.rope_dim % 32 == 0 && d.rope_dim <= 128 &&
        (long)rows_per_group * wave_cols * d.groups >= 65536) {
      // Enough 32-row tiles for every wave (one 8-wave block per CU) to take
      // about two (from 16384 query rows at r = 512); below that the 8-wave
      // 64-row tiles keep more waves busy.  The column blocks of one row range
      // sit on one XCD (block ids that differ by a multiple of 8) and share
      // its L2.
      int nb = std::max(1, std::min(cdiv(n_tiles, WW), (2048 / WW) / (wave_cols * d.groups)));
      if (nb >= 8) nb -= nb % 8;
      const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&absorb_wave), WAVE_LDS);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(absorb_wave, dim3(nb, wave_cols, d.groups), dim3(64 * WW), WAVE_LDS, s, q,
                         q_rope, q_pos, w_k, gamma_q, gamma_k, gamma_qr,
                         static_cast<uint16_t*>(q_tilde), alpha_q,
                         static_cast<uint16_t*>(q_rope_normed), rows_per_group, d.heads, hpg,
                         d.rank, d.rope_dim, d.eps, d.rope_theta);
      return hipGetLastError();
    }
    // about one block per CU: a block takes several row tiles when there are
    // more (the W^K_g tile is staged once per block when d <= 128)
    const int row_tiles = cdiv(rows_per_group, TM), col_blocks = cdiv(d.rank, TN);
    const bool keep = d.head_dim <= SK;
    const int tiles = keep ? std::max(1, row_tiles * col_blocks * d.groups / 256) : 1;
    dim3 grid(cdiv(row_tiles, tiles), col_blocks, d.groups);
    const void* fn = keep ? reinterpret_cast<const void*>(&absorb_split<true>)
                          : reinterpret_cast<const void*>(&absorb_split<false>);
    const hipError_t e = set_lds_limit_once(fn, SPLIT_LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(keep ? absorb_split<true> : absorb_split<false>, grid, dim3(64 * SW), SPLIT_LDS,
                       s, q, q_rope, q_pos, w_k, gamma_q,
                       gamma_k, gamma_qr, static_cast<uint16_t*>(q_tilde), alpha_q,
                       static_cast<uint16_t*>(q_rope_normed), rows_per_group, d.heads, hpg,
                       d.head_dim, d.rank, d.rope_dim, d.eps, d.rope_theta, tiles);
    return hipGetLastError();
  }
  return launch_typed<float>(d, q, q_rope, q_pos, w_k, gamma_q, gamma_k, gamma_qr, q_tilde,
                             alpha_q, q_rope_normed, s);
}

}  // namespace qkn
