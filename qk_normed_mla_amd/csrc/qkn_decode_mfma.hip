// Matrix-core split-KV decode for gfx950 (MI355X): bf16 latent cache, r = 512,
// d_R = 64, heads per KV group a multiple of 16.
//
// What it computes (QK-Normed MLA summary, "Metodologia", decode-logit
// equation; the RoPE dot of the shared RoPE key from the MQA-absorbed path of
// the GQLA summary, section 2): for query row (b, i, h) and split p, over the
// visible tokens t of the split,
//   l_t = scale * ((q~ . c_t) alpha^q alpha^k_{t,g(h)} + q^R . k^R_t)
//   o_p = sum_t softmax(l)_t c_t,   lse_p = ln sum_t e^{l_t}
// The inverse-RMS factors are applied to the content logits in registers as a
// row (alpha^q, one per head) by column (alpha^k, one per token) scaling before
// the RoPE dot is accumulated; nothing extra is read or written for them beyond
// the 4 bytes per token and group of the scalar cache.
//
// Work decomposition
//   one workgroup (4 waves, 1 per SIMD) per (sequence b, split p, block of 128
//   query rows); wave w owns 32 query rows = 32 heads of one query token, all
//   in one KV group.  Every 64-token page of the split is read from HBM once
//   and shared by the 4 waves through LDS.  A wave keeps q~ (128 registers) in
//   VGPRs and its 32 x 512 latent accumulator (256 registers) in the AGPR file.
//
// Per page (one pipeline stage), in two 32-token halves:
//   HBM -> LDS   73 LDS-DMA loads of 16 B per lane (buffer_load ... lds), issued
//                two pages ahead into a double buffer.  The buffer descriptor of
//                a page ends at the last valid token, so a partial page reads
//                zeros beyond it; an invalid page entry reads zeros throughout.
//   QK           S^T[32 tok x 32 heads] = C[32 x 512] . q~^T  (v_mfma_f32_32x32x16_bf16,
//                A = latent rows from LDS, B = q~ in registers for the whole
//                kernel), then S *= alpha^q alpha^k, then += K^R . q^R^T.
//   softmax      base 2 against a per-head reference fixed at the first
//                visible tokens of the split, so the accumulator is never
//                rescaled inside the loop.  QK-norm bounds the logits, so the
//                probabilities stay far below the 2^96 headroom allowed; should
//                a later logit exceed it, the workgroup restarts the split with
//                the larger reference (exact; never seen with normalised
//                logits).  A head's tokens sit in lanes l and l^32.
//   PV           O^T[512 x 32 heads] += C^T . P^T, the C^T operand read with
//                ds_read_b64_tr_b16 straight from the row-major page in LDS; the
//                token order inside each 16-token step follows the register
//                layout of S^T (both operands use the same permutation of the
//                reduction index, which leaves the sum unchanged).
// LDS layout of a staged page (bytes): content [64][1024] with the 16-byte
// chunk c of token t stored at chunk position c ^ f(t) (f below), RoPE keys
// [64][128] with chunk c of token t at c ^ ((t >> 1) & 7), then alpha^k [64][G].
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int R = 512;                    // latent rank
constexpr int DR = 64;                    // RoPE dim
constexpr int PAGE = QKN_MLA_PAGE_SIZE;   // 64 tokens per page = per stage
constexpr int ROW_BYTES = (R + DR) * 2;   // 1152
constexpr int CONTENT_BYTES = PAGE * R * 2;       // 65536
constexpr int ROPE_BYTES = PAGE * DR * 2;         // 8192
constexpr int ALPHA_BYTES = PAGE * 16 * 4;        // room for G <= 16
constexpr int STAGE_BYTES = CONTENT_BYTES + ROPE_BYTES + ALPHA_BYTES;  // 77824
constexpr int LDS_BYTES = 2 * STAGE_BYTES;        // 155648
constexpr int WAVES = 4;
constexpr int HEADS_PER_WAVE = 32;
constexpr int ROWS_PER_WG = WAVES * HEADS_PER_WAVE;  // 128
constexpr int kMaxGroups = 16;
constexpr int QK_AHEAD = 3;                      // LDS reads in flight ahead of the MFMAs
constexpr int PV_AHEAD = 3;
constexpr float kMaxExp2 = 96.0f;                 // headroom of p = 2^(y - ref), log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// content chunk position of chunk c of token t: c ^ f(t mod 16)
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 7; }

// raw buffer descriptor: base, byte size (reads at or past it return 0)
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffff));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// One LDS-DMA load: 16 bytes per lane from rsrc + voff to LDS (M0 + 16 * lane).
// The whole offset is in the vector operand, which is what the descriptor's
// range check covers (reads at or past the descriptor size return zeros).
// Issued through asm so that the compiler does not hold every LDS read until
// all DMA in flight has landed; completion is awaited explicitly (vmcnt)
// before the barrier that publishes a page.  The s_nop covers the wait states
// the hardware needs after M0 and descriptor SGPRs are written.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ bf16x8 lds_read16(const LDS_AS uint8_t* p) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(p);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<LDS_AS bf16x4*>(const_cast<LDS_AS uint8_t*>(p)));
}

// The lane index, re-materialised where it is used: the empty volatile asm
// keeps per-lane offsets derived from it from being hoisted out of the page
// loop and held in registers for the whole kernel.
__device__ __forceinline__ int fresh_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// PV product into an accumulator tile kept in the AGPR file (the 512-wide
// accumulator of a wave fills it exactly).  Issued through asm so that the
// compiler never parks another MFMA result in an AGPR and spills a tile to
// make room.  Hazards the compiler cannot see through asm: 2 wait states
// before the MFMA reads operands written by the vector ALU (s_nop 1), and
// wait_acc_results() before anything reads the accumulator back.
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+a"(acc) : "v"(a), "v"(b));
}
// wait states between an MFMA writing registers and a vector instruction
// reading them (covers the longest MFMA; 3 x 8)
__device__ __forceinline__ void wait_acc_results() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ __forceinline__ float pair_sum(float v) { return v + __shfl_xor(v, 32, 64); }

template <bool USE_ALPHA>
__global__ __launch_bounds__(64 * WAVES, 1) void decode_mfma_kernel(
    const uint16_t* __restrict__ q_tilde, const float* __restrict__ alpha_q,
    const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ kv,
    const float* __restrict__ alpha_k, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ err_flag, int s_q, int heads,
    int groups, int max_pages, int num_pages, int num_splits, int row_blocks, int n_work,
    int per_xcd, float scale) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // blocks are dealt to the 8 XCDs round-robin; give consecutive work items
  // (the row blocks and splits of one sequence) to the same XCD and L2
  const int wg = blockIdx.x;
  const int work = (wg & 7) * per_xcd + (wg >> 3);
  if (work >= n_work) return;
  const int rb = work % row_blocks;
  const int p = (work / row_blocks) % num_splits;
  const int b = work / (row_blocks * num_splits);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;   // which 8-wide half of a 16-long reduction step
  int err = 0;

  int T = seq_lens[b];
  if (T < 0 || T > max_pages * PAGE) {
    err = 1;
    T = min(max(T, 0), max_pages * PAGE);
  }
  const int L = split_len(max(T, 1), num_splits);
  const int lo = p * L;
  const int hi = min(lo + L, T);
  const int first_page = lo / PAGE;
  const int n_st = hi > lo ? (hi - lo + PAGE - 1) / PAGE : 0;

  // this wave's 32 query rows: query token i, heads h0 .. h0 + 31, group g
  const int rows_total = s_q * heads;
  const int row0 = rb * ROWS_PER_WG + w * HEADS_PER_WAVE;
  const bool wave_active = row0 < rows_total;
  const int i = wave_active ? row0 / heads : 0;
  const int h0 = wave_active ? row0 % heads : 0;
  const int g = h0 / (heads / groups);
  const int hi_w = min(hi, T - s_q + i + 1);  // visible end for this query token
  // row of this lane's head (an idle wave uses row 0 and discards its results)
  const size_t my_row = ((size_t)b * s_q + i) * heads + h0 + l32;

  // q~ as the B operand of QK: lane holds q~[head l32][16 kk + 8 hh .. +8]
  bf16x8 qb[R / 16];
  bf16x8 qrb[DR / 16];
  {
    const bf16x8* qt = reinterpret_cast<const bf16x8*>(q_tilde + my_row * R) + hh;
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) qb[kk] = qt[2 * kk];
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_rope + my_row * DR) + hh;
#pragma unroll
    for (int kk = 0; kk < DR / 16; ++kk) qrb[kk] = qr[2 * kk];
  }
  const float aq = USE_ALPHA ? alpha_q[my_row] : 1.f;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query operands are in registers

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS uint8_t*)smem));
  const int alpha_bytes_per_wave = PAGE * groups * 4 / WAVES;  // 64 G

  // page index of stage s (-1 when the entry is out of range)
  auto page_of = [&](int s) -> int {
    int pg = block_table[(size_t)b * max_pages + first_page + s];
    return (pg >= 0 && pg < num_pages) ? pg : -1;
  };

  // issue the 19 loads of this wave for stage s into buffer (s & 1):
  // 16 content rows, 2 RoPE blocks, 1 slice of alpha^k
  auto issue = [&](int s) {
    const int ln = fresh_lane();
    const int pg = page_of(s);
    const int tok0 = lo + s * PAGE;
    const int nv = pg >= 0 ? min(PAGE, T - tok0) : 0;   // valid rows of the page
    const uint8_t* page_ptr = reinterpret_cast<const uint8_t*>(kv) +
                              (size_t)(pg >= 0 ? pg : 0) * PAGE * ROW_BYTES;
    const i32x4 rs = buffer_rsrc(page_ptr, nv * ROW_BYTES);
    const uint32_t buf = lds_base + (s & 1) * STAGE_BYTES;
#pragma unroll
    for (int k = 0; k < 16; ++k) {  // content: token t = w + 4k, lane -> chunk lane ^ f(t)
      const int t = w + 4 * k;
      dma16(buf + t * 1024, t * ROW_BYTES + ((ln ^ swz(t & 15)) << 4), rs);
    }
    // RoPE keys of tokens 8r .. 8r + 7 for r = w, w + 4: token 8 r + lane / 8,
    // chunk (lane % 8) ^ f_R(token), and f_R = (4 r + lane / 16) mod 8 is the same for both
    const uint32_t rope_lane = (ln >> 3) * ROW_BYTES + R * 2 +
                               (((ln & 7) ^ ((4 * w + (ln >> 4)) & 7)) << 4);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = w + 4 * k;
      dma16(buf + CONTENT_BYTES + r * 1024, r * 8 * ROW_BYTES + rope_lane, rs);
    }
    {  // alpha^k of the page: 64 * G floats, a quarter per wave
      const float* ap = alpha_k + (size_t)(pg >= 0 ? pg : 0) * PAGE * groups;
      const i32x4 ra = buffer_rsrc(ap, nv * groups * 4);
      if (ln * 16 < alpha_bytes_per_wave)
        dma16(buf + CONTENT_BYTES + ROPE_BYTES + w * alpha_bytes_per_wave,
              w * alpha_bytes_per_wave + ln * 16, ra);
    }
  };

  f32x16 acc[R / 32];
  float m_ref = -INFINITY;   // reference of the exponent for this lane's head (logit units)
  float m_seen = -INFINITY;  // largest logit of this head seen so far
  float l_run = 0.f;         // this lane's share of the softmax denominator
  const float c2 = scale * kLog2e;  // logits -> log2 units

  bool again;
  do {
    again = false;
#pragma unroll
    for (int om = 0; om < R / 32; ++om) acc[om] = f32x16{};
    l_run = 0.f;
    if (n_st > 0) issue(0);
    if (n_st > 1) issue(1);

    for (int s = 0; s < n_st; ++s) {
      if (s + 1 < n_st) {
        asm volatile("s_waitcnt vmcnt(19)" ::: "memory");  // the next page's 19 loads may fly
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      const uint32_t stage_off = (s & 1) * STAGE_BYTES;
      const LDS_AS uint8_t* lds0 = (LDS_AS uint8_t*)smem;
      const LDS_AS float* st_alpha = (const LDS_AS float*)(lds0 + stage_off + CONTENT_BYTES + ROPE_BYTES);
      const int tok0 = lo + s * PAGE;
      const bool page_ok = page_of(s) >= 0;
      if (!page_ok) err = 1;
      // rows r of this page with r < lim are visible to this wave
      const int lim = page_ok ? hi_w - tok0 : 0;
      int overflow = 0;

      if (wave_active) {
        // Per-lane LDS byte offsets inside the staged page.  The XOR swizzle only
        // touches the low 4 bits of a chunk index, and a chunk index splits into
        // disjoint bit fields, so every read is (per-lane base) XOR (constant)
        // plus a compile-time offset above those bits (stage bases are multiples
        // of 1024 and commute with the XORs):
        //  QK row read, token 32 mt + l32, chunk 2 kk + hh:
        //    [l32*1024 + ((hh ^ f(l32)) << 4)] ^ (32 (kk % 8)) + 256 (kk / 8) + 32768 mt
        //  RoPE row read, chunk 2 kk + hh (kk < 4):
        //    [l32*128 + ((hh ^ f_R(l32)) << 4)] ^ (32 kk) + 4096 mt
        //  PV transposed read: 16-lane group G = lane / 16 reads 4 rows
        //  t0 = 4 (G / 2) + (lane % 16) / 4 of the step (and t0 + 8), latents
        //  32 om + 16 (G % 2) + 4 (lane % 4) .. +3, i.e. chunk 4 om + c0 with
        //  c0 = 2 (G % 2) + (lane % 4) / 2, byte 8 (lane % 2) of the chunk:
        //    [t*1024 + 8 (lane % 2) + ((c0 ^ f(t)) << 4)] ^ (64 (om % 4)) + 256 (om / 4) + 1024 (16 ks + 32 mt)
        uint32_t qk_b, rp_b, pv_a, pv_bb;
        {
          const int ln = fresh_lane();
          const int lt = ln & 31, lh = ln >> 5;
          qk_b = lt * 1024 + ((lh ^ swz(lt & 15)) << 4) + stage_off;
          rp_b = lt * 128 + ((lh ^ swz_rope(lt)) << 4) + stage_off + CONTENT_BYTES;
          const int G = ln >> 4, k16 = ln & 15;
          const int t0 = 4 * (G >> 1) + (k16 >> 2);
          const int c0 = 2 * (G & 1) + ((k16 & 3) >> 1);
          const int inner = 8 * (k16 & 1);
          pv_a = t0 * 1024 + inner + ((c0 ^ swz(t0)) << 4) + stage_off;
          pv_bb = (t0 + 8) * 1024 + inner + ((c0 ^ swz(t0 + 8)) << 4) + stage_off;
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          // ---- QK for 32 tokens: content, alpha scaling, RoPE ----
          // 32 reduction steps kk = 8 kh + k8, operands read QK_AHEAD steps ahead
          f32x16 sc = f32x16{};
          {
            constexpr int NK = R / 16;
            bf16x8 abuf[QK_AHEAD];
            auto rd = [&](int n) {  // step n in issue order: k8 = n / 4, kh = n % 4
              const int k8 = n >> 2, kh = n & 3;
              return lds_read16(lds0 + (qk_b ^ (32u * k8)) + 256 * kh + 32768 * mt);
            };
#pragma unroll
            for (int n = 0; n < QK_AHEAD; ++n) abuf[n] = rd(n);
#pragma unroll
            for (int n = 0; n < NK; ++n) {
              const bf16x8 a = abuf[n % QK_AHEAD];
              if (n + QK_AHEAD < NK) abuf[n % QK_AHEAD] = rd(n + QK_AHEAD);
              sc = mfma(a, qb[8 * (n & 3) + (n >> 2)], sc);
            }
          }
          if (USE_ALPHA) {
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
              const int t = 32 * mt + 8 * jg + 4 * hh;  // rows of registers 4 jg .. 4 jg + 3
#pragma unroll
              for (int e = 0; e < 4; ++e) sc[4 * jg + e] *= aq * st_alpha[(t + e) * groups + g];
            }
          }
#pragma unroll
          for (int kk = 0; kk < DR / 16; ++kk) {
            const bf16x8 a = lds_read16(lds0 + (rp_b ^ (32u * kk)) + 4096 * mt);
            sc = mfma(a, qrb[kk], sc);
          }
          // ---- mask rows past the visible end (tail page, causal window, bad page)
          if (lim < 32 * mt + 32) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (32 * mt + 8 * (j >> 2) + 4 * hh + (j & 3) >= lim) sc[j] = -INFINITY;
          }
          // ---- probabilities against the fixed reference ----
          float mx = sc[0];
#pragma unroll
          for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sc[j]);
          mx = pair_max(mx);
          m_seen = fmaxf(m_seen, mx);
          if (m_ref == -INFINITY) m_ref = mx;  // first visible tokens of the split
          if ((mx - m_ref) * c2 > kMaxExp2) overflow = 1;
          const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
          bf16x8 pb[2];  // P^T of the two 16-token steps
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const __bf16 pr = static_cast<__bf16>(exp2f(fmaf(sc[j], c2, -mc)));
            pb[j >> 3][j & 7] = pr;
            l_run += static_cast<float>(pr);
          }
          // ---- PV: O^T[512 x 32] += C^T[512 x 32 tok] . P^T ----
          // 32 products (o4, ks, oh) in that order, operands read PV_AHEAD ahead
          {
            constexpr int NP = 4 * 2 * (R / 128);
            bf16x8 abuf[PV_AHEAD];
            auto rd = [&](int n) {
              const int o4 = n >> 3, ks = (n >> 2) & 1, oh = n & 3;
              const int imm = 256 * oh + 1024 * (16 * ks + 32 * mt);
              const bf16x4 lo4 = lds_read_tr(lds0 + (pv_a ^ (64u * o4)) + imm);
              const bf16x4 hi4 = lds_read_tr(lds0 + (pv_bb ^ (64u * o4)) + imm);
              return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            };
#pragma unroll
            for (int n = 0; n < PV_AHEAD; ++n) abuf[n] = rd(n);
#pragma unroll
            for (int n = 0; n < NP; ++n) {
              const bf16x8 a = abuf[n % PV_AHEAD];
              if (n + PV_AHEAD < NP) abuf[n % PV_AHEAD] = rd(n + PV_AHEAD);
              mfma_acc(acc[4 * (n & 3) + (n >> 3)], a, pb[(n >> 2) & 1]);
            }
          }
        }
      }
      // all waves done with this buffer; did any head outgrow its reference?
      if (__syncthreads_or(overflow)) {
        again = true;
        break;
      }
      if (s + 2 < n_st) issue(s + 2);
    }
    if (again) {
      // restart the split with the largest logit seen as the reference
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      m_ref = m_seen;
    }
  } while (again);

  // ---- epilogue: o_p = acc / l, lse_p = scale * m_ref + ln l ----
  wait_acc_results();
  if (wave_active) {
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* out = o_part + (my_row * num_splits + p) * R;
#pragma unroll
    for (int om = 0; om < R / 32; ++om) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[om][4 * jg + e] * inv;
        *reinterpret_cast<f32x4*>(out + 32 * om + 8 * jg + 4 * hh) = v;
      }
    }
    if (hh == 0) {
      lse_part[my_row * num_splits + p] =
          l_tot > 0.f ? m_ref * scale + log2f(l_tot) * kLn2 : -INFINITY;
    }
  }
  if (err && err_flag && lane == 0) atomicOr(err_flag, 1);
}

template <bool USE_ALPHA>
hipError_t launch_typed(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mfma_kernel<USE_ALPHA>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int row_blocks = cdiv(d.s_q * d.heads, ROWS_PER_WG);
  const int n_work = d.batch * a.num_splits * row_blocks;
  const int per_xcd = cdiv(n_work, 8);
  dim3 grid(per_xcd * 8);
  hipLaunchKernelGGL(decode_mfma_kernel<USE_ALPHA>, grid, dim3(64 * WAVES), LDS_BYTES, s,
                     static_cast<const uint16_t*>(a.q_tilde), a.alpha_q,
                     static_cast<const uint16_t*>(a.q_rope), static_cast<const uint16_t*>(a.kv),
                     a.alpha_k, a.block_table, a.seq_lens, a.o_part, a.lse_part, a.err_flag, d.s_q,
                     d.heads, d.groups, d.max_pages_per_seq, d.num_pages, a.num_splits, row_blocks,
                     n_work, per_xcd, d.softmax_scale);
  return hipGetLastError();
}

}  // namespace

bool mfma_decode_supported(const qkn_mla_dims& d) {
  return d.cache_dtype == QKN_BF16 && d.rank == R && d.rope_dim == DR && d.groups <= kMaxGroups &&
         (d.heads / d.groups) % HEADS_PER_WAVE == 0;
}

hipError_t launch_decode_mfma(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s) {
  return a.use_alpha ? launch_typed<true>(d, a, s) : launch_typed<false>(d, a, s);
}

}  // namespace qkn
