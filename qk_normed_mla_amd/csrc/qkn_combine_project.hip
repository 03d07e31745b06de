// qkn_mla_combine_project: the log-sum-exp merge of the split-KV partials
// followed by the value up-projection o = o^lat W^V_g of every query row.  On
// the absorbed path the attention-weighted sum stays in latent space and the
// group's value up-projection is applied once per row afterwards (QK-Normed MLA
// summary, the absorbed form of the problem statement; GQLA summary, section 2).
//
// Matrix-core kernel (project_mfma): r a multiple of 128 and <= 512,
// d_v = d in {32, 64, 128, 256}, H/G a multiple of 32.  One block of 8 waves per
// 32 consecutive query rows (one (b, i) and one group g).
//   rows     either merged here from the half partials (fused form: wave w
//            merges rows 4w .. 4w+3 exactly as the combine kernel does for up to
//            16 splits, one wave per row, splits in order) or read back from
//            o_latent after the combine kernel (two-pass form).  They go to LDS
//            as float32, 32 x r, rows padded by 16 bytes so that the operand
//            reads below spread over the banks.
//   project  O[32 x d_v] = L[32 x r] . W^V_g[r x d_v] on v_mfma_f32_32x32x16_bf16.
//            Both operands are split into bf16 words, x = hi + lo + e with
//            |e| <= 2^-16 |x|, and each step takes hi.hi + hi.lo + lo.hi: every
//            product is within 3 * 2^-16 of exact, the sum is float32.
//            W^V_g passes through LDS in chunks of kc rows (16-byte loads, split
//            into hi and lo words on the way, kept row-major); the next chunk's
//            loads are in flight while the current chunk is multiplied.  The
//            W operand is read with ds_read_b64_tr_b16, which hands each lane
//            one column over four rows, so the reduction index of a step runs
//            4 hh + (0..3) and 8 + 4 hh + (0..3); the rows' operand is read from
//            LDS in the same order.  Wave w owns the 32-column tile
//            w mod (d_v / 32) and every KS-th step, KS = 8 / (d_v / 32); the
//            waves' tiles are added in a fixed order through LDS, so the result
//            does not depend on timing, and the tile leaves as 16-byte stores.
//            In the two-pass form, when the row tiles alone would not fill the
//            chip, the d_v columns are split over 2 or 4 blocks per tile (each
//            streams only its columns of W^V_g).
// 128-row fused kernel (project_gemm): the fused form when d_v = 128, r is a
// multiple of 64, there are at most 4 splits and a group has a multiple of 128
// heads; the same merge and the same split products, but over 128 rows per
// block with the merge done chunk by chunk of the latent, so W^V_g is streamed
// once per 128 rows.
// Generic kernel (every other shape): one block per query row, the row from
// o_latent in LDS, o_j = sum_m L_m W^V_g[m, j] in float32 in index order.
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

constexpr int WAVES = 8;
constexpr int ROWS = 32;           // query rows per block
constexpr int RMAX = 512;          // largest latent rank of the matrix-core kernel
constexpr int LSTRIDE = RMAX + 4;  // floats per LDS row
constexpr int L_BYTES = ROWS * LSTRIDE * 4;
constexpr int WCHUNK = 16384;      // W^V_g values staged in LDS at a time (at most)
constexpr int KC_MAX = 256;        // W^V_g rows staged at a time (at most)
constexpr int W_PAD = 16;          // bf16 of padding per staged row (rows 4 apart: distinct banks)
constexpr int PER = WCHUNK / 4 / (64 * WAVES);  // float4 of a chunk per thread
constexpr int kBatch = 8;          // splits whose loads are in flight together (merge)
constexpr int kFuseMaxSplits = 16; // the fused form keeps the combine's one-wave order
constexpr int kFuseMinTiles = 512; // below this many blocks the combine kernel merges faster
constexpr int kFillBlocks = 256;   // blocks that fill the chip (one per compute unit)

#define LDS_AS __attribute__((address_space(3)))
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// hi/lo bf16 words of four floats
__device__ __forceinline__ void split4(float4 v, bf16x4& hi, bf16x4& lo) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  hi = __builtin_convertvector(x, bf16x4);
  const f32x4 h = __builtin_convertvector(hi, f32x4);
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = x[j] - h[j];
  lo = __builtin_convertvector(r, bf16x4);
}

// 4 x 16 bf16 of LDS transposed across each 16-lane group: lane i of a group
// gets column i of the four rows its group addressed (8 bytes per lane)
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (LDS_AS bf16x4*)(const_cast<__bf16*>(p)));
}

// hi/lo bf16 words of eight floats
__device__ __forceinline__ void split8(f32x8 x, bf16x8& hi, bf16x8& lo) {
  hi = __builtin_convertvector(x, bf16x8);
  const f32x8 h = __builtin_convertvector(hi, f32x8);
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = x[j] - h[j];
  lo = __builtin_convertvector(r, bf16x8);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Merge of one row by one wave (half partials, lanes hold latents 8 lane ..
// 8 lane + 7): the same operations in the same order as the combine kernel's
// one-wave groups, so the two agree bit for bit.
__device__ __forceinline__ void merge_row(const _Float16* __restrict__ o_part,
                                          const float* __restrict__ lse_part, int row,
                                          int num_splits, int rank, int lane, float (&acc)[8],
                                          float& lse) {
  const int m0 = lane * 8;
  const bool live = m0 < rank;
  const float* lp = lse_part + (size_t)row * num_splits;
  float M = -INFINITY;
  for (int p0 = lane; p0 < num_splits; p0 += 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = p0 + 64 * u < num_splits ? lp[p0 + 64 * u] : -INFINITY;
    M = fmaxf(M, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  }
  M = wave_max(M);
  float s = 0.f;
  for (int p0 = lane; p0 < num_splits; p0 += 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = p0 + 64 * u < num_splits ? lp[p0 + 64 * u] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) s += expf(x[u] - M);
  }
  s = wave_sum(s);
  const bool empty = M == -INFINITY;
  lse = empty ? -INFINITY : M + logf(s);
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if (empty) return;
  const _Float16* op = o_part + (size_t)row * num_splits * rank + m0;
  for (int p0 = 0; p0 < num_splits; p0 += kBatch) {
    f16x8 v[kBatch];
    float l[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + u;
      l[u] = p < num_splits ? lp[p] : -INFINITY;
      v[u] = (p < num_splits && live) ? *reinterpret_cast<const f16x8*>(op + (size_t)p * rank)
                                      : f16x8{};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (l[u] == -INFINITY) continue;  // empty split
      const float w = expf(l[u] - lse);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, static_cast<float>(v[u][j]), acc[j]);
    }
  }
}

// A float32 operand of a step: L[l32][k0 + 4 hh + (j % 4) + 8 (j / 4)], j < 8 (the
// reduction-index order that the transposed LDS read below gives the other operand)
template <bool MERGE>
__global__ __launch_bounds__(64 * WAVES) void project_mfma(
    const _Float16* __restrict__ o_part, const float* __restrict__ lse_part,
    const float* __restrict__ w_v, float* __restrict__ o_lat, float* __restrict__ lse_out,
    float* __restrict__ o_out, int num_splits, int rank, int dv, int heads, int groups, int kc,
    int dvb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* L = reinterpret_cast<float*>(smem);
  const int col0 = blockIdx.y * dvb;  // this block's output columns col0 .. col0 + dvb - 1
  const int wrow = dvb + W_PAD;       // bf16 per staged W^V row
  __bf16* Wh = reinterpret_cast<__bf16*>(smem + L_BYTES);
  __bf16* Wl = Wh + kc * wrow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int l16 = lane & 15, G = (lane >> 4) & 1;
  const int row0 = blockIdx.x * ROWS;
  const int g = (row0 % heads) / (heads / groups);

  // W^V_g chunks of kc rows: 16-byte loads into registers, then hi/lo words
  // into LDS (row-major, rows padded by W_PAD)
  const float* wg = w_v + (size_t)g * rank * dv;
  const int c4n = dvb / 4;
  const int chunk4 = kc * c4n;  // float4 per chunk
  float4 wv[PER];
  auto wload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * 64 * WAVES;
      wv[u] = e < chunk4 ? *reinterpret_cast<const float4*>(wg + (size_t)(k0 + e / c4n) * dv + col0 + 4 * (e % c4n))
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto wstore = [&]() {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * 64 * WAVES;
      if (e < chunk4) {
        bf16x4 hi, lo;
        split4(wv[u], hi, lo);
        const int at = (e / c4n) * wrow + 4 * (e % c4n);
        *reinterpret_cast<bf16x4*>(Wh + at) = hi;
        *reinterpret_cast<bf16x4*>(Wl + at) = lo;
      }
    }
  };
  wload(0);

  // the 32 rows, as float32 in LDS
#pragma unroll
  for (int k = 0; k < ROWS / WAVES; ++k) {
    const int lr = (ROWS / WAVES) * wave + k;
    const int row = row0 + lr;
    const int m0 = lane * 8;
    float acc[8];
    if (MERGE) {
      float lse;
      merge_row(o_part, lse_part, row, num_splits, rank, lane, acc, lse);
      if (lane == 0) lse_out[row] = lse;
      if (m0 < rank) {
        float4* gp = reinterpret_cast<float4*>(o_lat + (size_t)row * rank + m0);
        gp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        gp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    } else if (m0 < rank) {
      const float4* gp = reinterpret_cast<const float4*>(o_lat + (size_t)row * rank + m0);
      const float4 a = gp[0], b = gp[1];
      acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
      acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
    }
    if (m0 < rank) {
      float4* lp = reinterpret_cast<float4*>(&L[lr * LSTRIDE + m0]);
      lp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      lp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }

  // this wave's share: columns ct*32 .. +31, steps ks, ks + KS, ... of every chunk
  const int n_ct = dvb / 32;
  const int KS = WAVES / n_ct;
  const int ct = wave % n_ct, ks = wave / n_ct;
  const int spc = kc / 16;
  // transposed read of staged rows 4 hh + l16 / 4 (+ 8), columns ct*32 + 16 G + 4 (l16 % 4)
  const int tr_off = (4 * hh + (l16 >> 2)) * wrow + ct * 32 + 16 * G + 4 * (l16 & 3);
  f32x16 acc = {};
  for (int k0 = 0; k0 < rank; k0 += kc) {
    __syncthreads();  // rows in L; every read of the previous chunk done
    wstore();
    if (k0 + kc < rank) wload(k0 + kc);  // in flight during this chunk's products
    __syncthreads();
    for (int st = ks; st < spc; st += KS) {
      const int kl = 16 * st;
      const float* ap = &L[l32 * LSTRIDE + k0 + kl + 4 * hh];
      const float4 a0 = *reinterpret_cast<const float4*>(ap);
      const float4 a1 = *reinterpret_cast<const float4*>(ap + 8);
      const f32x8 av = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const int off = tr_off + kl * wrow;
      const bf16x8 bh = __builtin_shufflevector(lds_read_tr(Wh + off), lds_read_tr(Wh + off + 8 * wrow),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 bl = __builtin_shufflevector(lds_read_tr(Wl + off), lds_read_tr(Wl + off + 8 * wrow),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      bf16x8 ah, al;
      split8(av, ah, al);
      acc = mfma(ah, bh, acc);
      acc = mfma(ah, bl, acc);
      acc = mfma(al, bh, acc);
    }
  }

  // slices 1 .. KS-1 hand their tiles to slice 0 (W area); slice 0 adds them in
  // order and puts the tile into the L area as [32][d_v]; then 16-byte stores
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem + L_BYTES);
  if (ks > 0) {
    float* rp = part + ((ks - 1) * n_ct + ct) * 1024;
#pragma unroll
    for (int r = 0; r < 16; ++r) rp[r * 64 + lane] = acc[r];
  }
  __syncthreads();
  if (ks == 0) {
    for (int k2 = 1; k2 < KS; ++k2) {
      const float* rp = part + ((k2 - 1) * n_ct + ct) * 1024;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += rp[r * 64 + lane];
    }
    // D[m][n]: m = r % 4 + 8 (r / 4) + 4 hh, n = l32
#pragma unroll
    for (int r = 0; r < 16; ++r) L[((r & 3) + 8 * (r >> 2) + 4 * hh) * dvb + ct * 32 + l32] = acc[r];
  }
  __syncthreads();
  for (int e = tid; e < ROWS * c4n; e += 64 * WAVES) {
    const int m = e / c4n, c = e % c4n;
    *reinterpret_cast<float4*>(o_out + (size_t)(row0 + m) * dv + col0 + 4 * c) =
        *reinterpret_cast<const float4*>(&L[m * dvb + 4 * c]);
  }
}

// Fused form for 128-row tiles within one group (d_v = 128, r a multiple of 64,
// at most 4 splits): one block of 8 waves per 128 query rows, the latent taken
// in chunks of GK = 64.  First every wave forms the log-sum-exp statistics of
// 16 rows exactly as merge_row does (the same loads, reductions and weights),
// keeping each split's weight (and whether it is empty) in LDS.  Then per
// chunk: thread t merges latents 8 (t % 8) .. + 7 of rows t / 8 and t / 8 + 64
// from the half partials, splits in order, as merge_row does (so o_latent is
// the combine kernel's bits), writes them to o_latent, and stores their bf16
// hi/lo words in LDS in the reduction order of the products; the chunk of
// W^V_g goes to LDS as hi/lo words the same way the 32-row kernel stages it.
// Wave w computes the 32 x 32 output tiles (w / 2, 2 (w % 2)) and (w / 2,
// 2 (w % 2) + 1) with hi.hi + hi.lo + lo.hi per step.  The next chunk's
// partial and W^V_g loads are in flight during the current chunk's products.
// W^V_g is streamed once per 128 rows (four times less than 32-row blocks).
constexpr int GT = 128;  // rows per block
constexpr int GK = 64;   // latents per chunk
constexpr int GD = 128;  // output columns (d_v)
constexpr int G_MAXP = 4;
constexpr int GA_ROW = GK + 8;    // bf16 per staged row of the rows' words (16 bytes of padding)
constexpr int GW_ROW = GD + W_PAD;
constexpr size_t G_LDS = 2 * (size_t)GT * GA_ROW * 2 + 2 * (size_t)GK * GW_ROW * 2 + (size_t)GT * G_MAXP * 4 + GT * 4;

// position of latent k (within its chunk) among the staged words: in each
// 16-group the order is k 0-3, 8-11, 4-7, 12-15, so that lane half hh reads the
// 8 entries 4 hh + (0..3), 8 + 4 hh + (0..3) of a step as one 16-byte piece
__device__ __forceinline__ int gpos(int k) { return (k & ~15) | (k & 3) | ((k & 8) >> 1) | ((k & 4) << 1); }

__global__ __launch_bounds__(64 * WAVES) void project_gemm(
    const _Float16* __restrict__ o_part, const float* __restrict__ lse_part,
    const float* __restrict__ w_v, float* __restrict__ o_lat, float* __restrict__ lse_out,
    float* __restrict__ o_out, int num_splits, int rank, int heads, int groups) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __bf16* Ah = reinterpret_cast<__bf16*>(smem);
  __bf16* Al = Ah + GT * GA_ROW;
  __bf16* Wh = Al + GT * GA_ROW;
  __bf16* Wl = Wh + GK * GW_ROW;
  float* wgt = reinterpret_cast<float*>(Wl + GK * GW_ROW);  // [GT][G_MAXP] split weights
  int* skip = reinterpret_cast<int*>(wgt + GT * G_MAXP);    // [GT] bit p: split p empty
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int l16 = lane & 15, G = (lane >> 4) & 1;
  const int row0 = blockIdx.x * GT;
  const int g = (row0 % heads) / (heads / groups);
  const int P = num_splits;

  // ---- statistics of 16 rows per wave (merge_row's first part) ----
  {
    float x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = row0 + 16 * wave + q;
      x[q] = lane < P ? lse_part[(size_t)row * P + lane] : -INFINITY;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int lr = 16 * wave + q;
      // lanes 64 u + lane hold split p0 + 64 u: with P <= 64 only u = 0 is live
      const float M = wave_max(fmaxf(fmaxf(fmaxf(x[q], -INFINITY), -INFINITY), -INFINITY));
      float sl = 0.f;
      sl += expf(x[q] - M);
      sl += expf(-INFINITY - M);
      sl += expf(-INFINITY - M);
      sl += expf(-INFINITY - M);
      const float s = wave_sum(sl);
      const bool empty = M == -INFINITY;
      const float lse = empty ? -INFINITY : M + logf(s);
      if (lane == 0) lse_out[row0 + lr] = lse;
      const bool skip_p = empty || x[q] == -INFINITY;
      const unsigned long long sk = __ballot(lane < P && skip_p);
      if (lane < P) wgt[lr * G_MAXP + lane] = skip_p ? 0.f : expf(x[q] - lse);
      if (lane == 0) skip[lr] = static_cast<int>(sk & 0xF);
    }
  }

  // ---- chunk loads: partials of items (row t / 8 + 64 u, latents 8 (t % 8)
  // .. + 7) and W^V_g rows k0 .. k0 + GK - 1 (16 floats per thread) ----
  const int it_row = tid >> 3, it_c = 8 * (tid & 7);
  f16x8 pv[2][G_MAXP];
  float4 wv[GK * GD / 4 / (64 * WAVES)];
  const float* wg = w_v + (size_t)g * rank * GD;
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = row0 + it_row + 64 * u;
#pragma unroll
      for (int p = 0; p < G_MAXP; ++p)
        pv[u][p] = p < P ? *reinterpret_cast<const f16x8*>(o_part + ((size_t)row * P + p) * rank + k0 + it_c)
                         : f16x8{};
    }
#pragma unroll
    for (int u = 0; u < GK * GD / 4 / (64 * WAVES); ++u) {
      const int e = tid + u * 64 * WAVES;
      wv[u] = *reinterpret_cast<const float4*>(wg + (size_t)(k0 + e / (GD / 4)) * GD + 4 * (e % (GD / 4)));
    }
  };

  const int rt = wave >> 1, ct0 = 2 * (wave & 1);
  const int tr_off = (4 * hh + (l16 >> 2)) * GW_ROW + 16 * G + 4 * (l16 & 3);
  f32x16 acc[2] = {};
  __syncthreads();  // the weights are in LDS
  load(0);
  for (int k0 = 0; k0 < rank; k0 += GK) {
    // merge, o_latent, the rows' words
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int lr = it_row + 64 * u;
      const int sk = skip[lr];
      float a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = 0.f;
#pragma unroll
      for (int p = 0; p < G_MAXP; ++p) {
        if (p >= P || ((sk >> p) & 1)) continue;
        const float w = wgt[lr * G_MAXP + p];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = fmaf(w, static_cast<float>(pv[u][p][j]), a[j]);
      }
      float4* gp = reinterpret_cast<float4*>(o_lat + (size_t)(row0 + lr) * rank + k0 + it_c);
      gp[0] = make_float4(a[0], a[1], a[2], a[3]);
      gp[1] = make_float4(a[4], a[5], a[6], a[7]);
      bf16x4 h0, l0, h1, l1;
      split4(make_float4(a[0], a[1], a[2], a[3]), h0, l0);
      split4(make_float4(a[4], a[5], a[6], a[7]), h1, l1);
      const int at0 = lr * GA_ROW + gpos(it_c), at1 = lr * GA_ROW + gpos(it_c + 4);
      *reinterpret_cast<bf16x4*>(Ah + at0) = h0;
      *reinterpret_cast<bf16x4*>(Al + at0) = l0;
      *reinterpret_cast<bf16x4*>(Ah + at1) = h1;
      *reinterpret_cast<bf16x4*>(Al + at1) = l1;
    }
#pragma unroll
    for (int u = 0; u < GK * GD / 4 / (64 * WAVES); ++u) {
      const int e = tid + u * 64 * WAVES;
      bf16x4 hi, lo;
      split4(wv[u], hi, lo);
      const int at = (e / (GD / 4)) * GW_ROW + 4 * (e % (GD / 4));
      *reinterpret_cast<bf16x4*>(Wh + at) = hi;
      *reinterpret_cast<bf16x4*>(Wl + at) = lo;
    }
    if (k0 + GK < rank) load(k0 + GK);  // in flight during this chunk's products
    __syncthreads();
#pragma unroll
    for (int st = 0; st < GK / 16; ++st) {
      const int ao = (32 * rt + l32) * GA_ROW + 16 * st + 8 * hh;
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Ah + ao);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(Al + ao);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int off = tr_off + 16 * st * GW_ROW + 32 * (ct0 + c);
        const bf16x8 bh = __builtin_shufflevector(lds_read_tr(Wh + off), lds_read_tr(Wh + off + 8 * GW_ROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 bl = __builtin_shufflevector(lds_read_tr(Wl + off), lds_read_tr(Wl + off + 8 * GW_ROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        acc[c] = mfma(ah, bh, acc[c]);
        acc[c] = mfma(ah, bl, acc[c]);
        acc[c] = mfma(al, bh, acc[c]);
      }
    }
    __syncthreads();  // every read of this chunk's words done
  }
  // D[m][n]: m = r % 4 + 8 (r / 4) + 4 hh, n = l32
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      o_out[(size_t)(row0 + 32 * rt + (r & 3) + 8 * (r >> 2) + 4 * hh) * GD + 32 * (ct0 + c) + l32] = acc[c][r];
}

// one block per query row
__global__ __launch_bounds__(256) void project_generic(const float* __restrict__ o_lat,
                                                       const float* __restrict__ w_v,
                                                       float* __restrict__ o_out, int rank,
                                                       int dv, int heads, int groups) {
  extern __shared__ float lrow[];
  const int row = blockIdx.x;
  const int g = (row % heads) / (heads / groups);
  for (int m = threadIdx.x; m < rank; m += blockDim.x) lrow[m] = o_lat[(size_t)row * rank + m];
  __syncthreads();
  const float* wg = w_v + (size_t)g * rank * dv;
  for (int j = threadIdx.x; j < dv; j += blockDim.x) {
    float s = 0.f;
    for (int m = 0; m < rank; ++m) s = fmaf(lrow[m], wg[(size_t)m * dv + j], s);
    o_out[(size_t)row * dv + j] = s;
  }
}

}  // namespace

namespace {
int chunk_rows(int dv) { return WCHUNK / dv < KC_MAX ? WCHUNK / dv : KC_MAX; }
size_t project_lds_bytes(int dv) { return L_BYTES + 2 * (size_t)chunk_rows(dv) * (dv + W_PAD) * 2; }
// the largest of the supported widths' LDS needs
size_t project_lds_max() {
  size_t m = 0;
  for (int dv = 32; dv <= 256; dv *= 2) m = project_lds_bytes(dv) > m ? project_lds_bytes(dv) : m;
  return m;
}
template <bool MERGE>
hipError_t set_lds_limit() {
  return set_lds_limit_once(reinterpret_cast<const void*>(&project_mfma<MERGE>),
                            (int)project_lds_max());
}
}  // namespace

// a block width the matrix-core kernel takes
static bool width_ok(int rank, int w) {
  return (w == 32 || w == 64 || w == 128 || w == 256) && rank % chunk_rows(w) == 0;
}

bool project_mfma_applies(const qkn_mla_dims& d) {
  return d.rank % 128 == 0 && d.rank <= RMAX && width_ok(d.rank, d.head_dim) &&
         (d.heads / d.groups) % 32 == 0;
}

hipError_t launch_combine_project(const qkn_mla_dims& d, int num_splits, const void* o_part,
                                  const float* lse_part, const float* w_v, float* o_lat,
                                  float* lse, float* o, uint32_t flags, hipStream_t s) {
  const int n_rows = d.batch * d.s_q * d.heads;
  const bool mfma_ok = project_mfma_applies(d);
  const int tiles = n_rows / ROWS;
  const bool fuse_ok = mfma_ok && d.cache_dtype == QKN_BF16 && num_splits <= kFuseMaxSplits;
  bool fuse = fuse_ok && tiles >= kFuseMinTiles;
  if (flags & QKN_PROJECT_FUSED) fuse = fuse_ok;
  if (flags & QKN_PROJECT_TWO_PASS) fuse = false;
  // the two-pass form splits the output columns over up to 4 blocks per row
  // tile until the grid fills the chip; the fused form keeps one (its merge
  // is not repeated)
  int cs = 1;
  while (!fuse && cs < 4 && tiles * cs < kFillBlocks && width_ok(d.rank, d.head_dim / (2 * cs)))
    cs *= 2;
  const int dvb = d.head_dim / cs;
  const int kc = chunk_rows(dvb);
  const size_t lds = project_lds_bytes(dvb);
  if (fuse && d.head_dim == GD && d.rank % GK == 0 && num_splits <= G_MAXP &&
      (d.heads / d.groups) % GT == 0) {
    const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&project_gemm), (int)G_LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(project_gemm, dim3(n_rows / GT), dim3(64 * WAVES), G_LDS, s,
                       static_cast<const _Float16*>(o_part), lse_part, w_v, o_lat, lse, o,
                       num_splits, d.rank, d.heads, d.groups);
    return hipGetLastError();
  }
  if (fuse) {
    hipError_t e = set_lds_limit<true>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(project_mfma<true>, dim3(tiles), dim3(64 * WAVES), lds, s,
                       static_cast<const _Float16*>(o_part), lse_part, w_v, o_lat, lse, o,
                       num_splits, d.rank, d.head_dim, d.heads, d.groups, kc, dvb);
    return hipGetLastError();
  }
  hipError_t e = launch_combine(d, num_splits, o_part, lse_part, o_lat, lse, s);
  if (e != hipSuccess) return e;
  if (mfma_ok) {
    e = set_lds_limit<false>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(project_mfma<false>, dim3(tiles, cs), dim3(64 * WAVES), lds, s, nullptr,
                       nullptr, w_v, o_lat, nullptr, o, num_splits, d.rank, d.head_dim, d.heads,
                       d.groups, kc, dvb);
  } else {
    hipLaunchKernelGGL(project_generic, dim3(n_rows), dim3(256), (size_t)d.rank * sizeof(float), s,
                       o_lat, w_v, o, d.rank, d.head_dim, d.heads, d.groups);
  }
  return hipGetLastError();
}

}  // namespace qkn
