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
//   one workgroup (8 waves, 2 per SIMD) per (sequence b, split p, block of 128
//   query rows); wave w owns 16 query rows = 16 heads of one query token, all
//   in one KV group.  Every token of the split is read from HBM once and
//   shared by the 8 waves through LDS.  A wave keeps q~ (72 registers) and its
//   16 x 512 latent accumulator (128 registers) for the whole kernel, within
//   the 256 registers that let two waves share a SIMD, so one wave's softmax
//   overlaps the other's MFMAs.
//
// Per 32-token stage (half a page):
//   HBM -> LDS   LDS-DMA loads of 16 B per lane (buffer_load ... lds) into a
//                ring of 4 stage buffers, 3 stages in flight, so that about
//                115 KB per CU is always on its way from HBM.  The buffer
//                descriptor of a stage ends at its last valid token, so a
//                partial page reads zeros beyond it; an invalid page entry
//                reads zeros throughout.
//   QK           S^T[16 tok x 16 heads] = C[16 x 512] . q~^T  (v_mfma_f32_16x16x32_bf16,
//                A = latent rows from LDS, B = q~ in registers for the whole
//                kernel), then S *= alpha^q alpha^k, then += K^R . q^R^T.
//   softmax      base 2 against a per-head reference fixed at the first
//                visible tokens of the split, so the accumulator is never
//                rescaled inside the loop.  QK-norm bounds the logits, so the
//                probabilities stay far below the 2^96 headroom allowed; should
//                a later logit exceed it, the workgroup restarts the split with
//                the larger reference (exact; never seen with normalised
//                logits).  A head's tokens sit in lanes l, l^16, l^32, l^48.
//   PV           O^T[512 x 16 heads] += C^T . P^T over the 32 tokens, the C^T
//                operand read with ds_read_b64_tr_b16 straight from the
//                row-major stage in LDS; the token order inside the step
//                follows the register layout of two S^T tiles (both operands
//                use the same permutation of the reduction index, which leaves
//                the sum unchanged).
// LDS layout of a stage (bytes): content [32][1024] with the 16-byte chunk c of
// token t stored at chunk position c ^ f(t) (f below), RoPE keys [32][128] with
// chunk c of token t at c ^ ((t >> 1) & 7), then alpha^k [32][G].  The
// swizzles spread the row reads of QK and the transposed reads of PV over
// the LDS banks.
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int R = 512;                    // latent rank
constexpr int DR = 64;                    // RoPE dim
constexpr int PAGE = QKN_MLA_PAGE_SIZE;   // 64 tokens per page
constexpr int ST = 32;                    // tokens per pipeline stage
constexpr int NSTAGE = 4;                 // stage buffers in LDS
constexpr int ROW_BYTES = (R + DR) * 2;   // 1152
constexpr int CONTENT_BYTES = ST * R * 2;         // 32768
constexpr int ROPE_BYTES = ST * DR * 2;           // 4096
constexpr int ALPHA_BYTES = ST * 16 * 4;          // room for G <= 16
constexpr int STAGE_BYTES = CONTENT_BYTES + ROPE_BYTES + ALPHA_BYTES;  // 38912
constexpr int FLAG_OFFSET = NSTAGE * STAGE_BYTES; // the workgroup's restart flag
constexpr int LDS_BYTES = FLAG_OFFSET + 16;       // 155664
constexpr int WAVES = 8;
constexpr int HEADS_PER_WAVE = 16;
constexpr int ROWS_PER_WG = WAVES * HEADS_PER_WAVE;  // 128
constexpr int kMaxGroups = 16;
constexpr int QK_AHEAD = 3;                      // LDS reads in flight ahead of the MFMAs
constexpr int PV_AHEAD = 3;
constexpr float kMaxExp2 = 96.0f;                 // headroom of p = 2^(y - ref), log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// content chunk position of chunk c of token t: c ^ f(t mod 16), f the
// linear map over GF(2)^4 with f(1) = 2, f(2) = 15, f(4) = 8, f(8) = 9.
// Measured on gfx950: LDS b128 reads run at full rate when lanes 0-7 of a
// 16-lane group stay in one 128-byte half of the 64 banks and lanes 8-15 in
// the other, which the QK row read (16 tokens x one chunk) meets when f's top
// bit follows t's top bit; among such maps this one also keeps the
// transposed 8-byte reads of PV (4 tokens x 2 chunks per 16 lanes) near
// their best rate.  A search over all invertible maps picked it.
__device__ __forceinline__ int swz(int t) {
  return static_cast<int>((0xce3146b957a8df20ull >> (4 * (t & 15))) & 15);
}
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

// the value, hidden from the optimiser so that it recomputes what derives from it
// instead of keeping those results live in registers
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the four lanes l, l^16, l^32, l^48 that hold one head.
// v_permlane16_swap / v_permlane32_swap with both operands v return the two
// halves that pair lane l with lane l^16 (l^32) in every lane.
__device__ __forceinline__ float xor16_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float head_max(float v) { return xor32_pair_max(xor16_pair_max(v)); }
__device__ __forceinline__ float head_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
  const int l16 = lane & 15;
  const int q4 = lane >> 4;   // which 8-wide slice of a 32-long reduction step
  int err = 0;

  int T = seq_lens[b];
  if (T < 0 || T > max_pages * PAGE) {
    err = 1;
    T = min(max(T, 0), max_pages * PAGE);
  }
  const int L = split_len(max(T, 1), num_splits);
  const int lo = p * L;
  const int hi = min(lo + L, T);
  const int first_page = lo / PAGE;  // lo is a multiple of the page size
  const int n_st = hi > lo ? (hi - lo + ST - 1) / ST : 0;

  // this wave's 16 query rows: query token i, heads h0 .. h0 + 15, group g
  const int rows_total = s_q * heads;
  const int row0 = rb * ROWS_PER_WG + w * HEADS_PER_WAVE;
  const bool wave_active = row0 < rows_total;
  const int i = wave_active ? row0 / heads : 0;
  const int h0 = wave_active ? row0 % heads : 0;
  const int g = h0 / (heads / groups);
  const int hi_w = min(hi, T - s_q + i + 1);  // visible end for this query token
  // row of this lane's head (an idle wave uses row 0 and discards its results)
  const size_t my_row = ((size_t)b * s_q + i) * heads + h0 + l16;

  // Page-table window: lane j of every wave holds the entry of split page
  // wbase + j (64 pages, 4096 tokens), so a stage finds its page with one
  // v_readlane instead of a memory round trip inside the loop.
  int wbase = 0;
  int pwin;
  auto load_window = [&](int base) {
    const int j = first_page + base + fresh_lane();
    pwin = j < max_pages ? block_table[(size_t)b * max_pages + j] : -1;
  };
  load_window(0);

  // q~ as the B operand of QK: lane holds q~[head l16][32 kk + 8 q4 .. +8]
  bf16x8 qb[R / 32];
  bf16x8 qrb[DR / 32];
  {
    const bf16x8* qt = reinterpret_cast<const bf16x8*>(q_tilde + my_row * R) + q4;
#pragma unroll
    for (int kk = 0; kk < R / 32; ++kk) qb[kk] = qt[4 * kk];
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_rope + my_row * DR) + q4;
#pragma unroll
    for (int kk = 0; kk < DR / 32; ++kk) qrb[kk] = qr[4 * kk];
  }
  const float aq = USE_ALPHA ? alpha_q[my_row] : 1.f;
  // query operands and page window in registers before any page load is
  // issued (the page loads are not visible to the compiler's own waits)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS uint8_t*)smem));

  // validity of the pages of the stages in flight, bit s mod 4 (uniform)
  uint32_t vmask = 0;

  // The 6 loads of this wave for stage s (tokens lo + 32 s ..) into buffer
  // s mod 4: 4 content rows, a quarter of the RoPE block on lanes 0-31, and an
  // eighth of alpha^k on lanes 0 .. G-1 (lane 0 always takes part, so every
  // wave issues all 6 and the vmcnt bookkeeping holds).  plan() looks the page
  // up and builds the descriptors; load(k) issues load k.  Inside the page
  // loop the loads are spread over the QK products, so the address units work
  // through them while the matrix cores run.
  struct StagePlan {
    i32x4 rs, ra;  // KV rows of the stage, alpha^k rows of the stage
    uint32_t buf;  // LDS address of the stage buffer
  };
  auto plan = [&](int s) {
    const int rel = s >> 1;  // page of the split
    if (rel < wbase || rel >= wbase + 64) {  // uniform; once per 64 pages
      wbase = rel & ~63;
      load_window(wbase);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    int pg = __builtin_amdgcn_readlane(pwin, rel - wbase);
    pg = (pg >= 0 && pg < num_pages) ? pg : -1;
    vmask = (vmask & ~(1u << (s & 3))) | ((pg >= 0 ? 1u : 0u) << (s & 3));
    const int tok0 = lo + s * ST;
    const int nv = pg >= 0 ? min(ST, T - tok0) : 0;   // valid rows of the stage
    const size_t row0 = (size_t)(pg >= 0 ? pg : 0) * PAGE + (s & 1) * ST;  // cache row
    StagePlan pl;
    pl.rs = buffer_rsrc(reinterpret_cast<const uint8_t*>(kv) + row0 * ROW_BYTES, nv * ROW_BYTES);
    pl.ra = buffer_rsrc(alpha_k + row0 * groups, nv * groups * 4);
    pl.buf = lds_base + (s & (NSTAGE - 1)) * STAGE_BYTES;
    asm volatile("" : "+s"(pl.buf));  // keep the per-load LDS addresses out of loop-invariant registers
    return pl;
  };
  auto load = [&](const StagePlan& pl, int k) {
    const int ln = fresh_lane();
    if (k < ST / 8) {
      // content token t = w + 8k at t * ROW_BYTES; the lane's chunk is lane ^ f(t)
      const int t = w + 8 * k;
      dma16(pl.buf + t * 1024, t * ROW_BYTES + ((ln ^ swz(t)) << 4), pl.rs);
    } else if (k == ST / 8) {
      // RoPE keys of tokens 4w .. 4w + 3: token 4 w + lane / 8, chunk (lane % 8) ^ f_R(token)
      if (ln < 32) {
        const int t = 4 * w + (ln >> 3);
        dma16(pl.buf + CONTENT_BYTES + w * 512, t * ROW_BYTES + R * 2 + (((ln & 7) ^ swz_rope(t)) << 4), pl.rs);
      }
    } else {
      // alpha^k of the stage: 32 * G floats, 16 G bytes per wave
      if (ln < groups)
        dma16(pl.buf + CONTENT_BYTES + ROPE_BYTES + 16 * groups * w, 16 * groups * w + ln * 16, pl.ra);
    }
  };
  constexpr int LOADS = ST / 8 + 2;
  auto issue = [&](int s) {
    const StagePlan pl = plan(s);
#pragma unroll
    for (int k = 0; k < LOADS; ++k) load(pl, k);
  };

  f32x4 acc[R / 16];
  float m_ref = -INFINITY;   // reference of the exponent for this lane's head (logit units)
  float m_seen = -INFINITY;  // largest logit of this head seen so far
  float l_run = 0.f;         // this lane's share of the softmax denominator
  const float c2 = scale * kLog2e;  // logits -> log2 units

  // restart flag: set by any wave whose logits outgrew the reference, read by
  // all after the next barrier
  volatile LDS_AS int* flag = (volatile LDS_AS int*)((LDS_AS uint8_t*)smem + FLAG_OFFSET);
  if (tid == 0) *flag = 0;

  bool again;
  do {
    again = false;
#pragma unroll
    for (int om = 0; om < R / 16; ++om) acc[om] = f32x4{};
    l_run = 0.f;
    static_assert(NSTAGE == 4, "the prologue issues three stages");
    if (n_st > 0) issue(0);
    if (n_st > 1) issue(1);
    if (n_st > 2) issue(2);

    for (int s = 0; s < n_st; ++s) {
      // stage s has landed (its successors may still be in flight) and every
      // wave is done with stage s - 1
      const int ahead = min(n_st - 1 - s, NSTAGE - 2);
      if (ahead >= 2) {
        asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      } else if (ahead == 1) {
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      // the loads of stage s + 3 go into the buffer of stage s - 1
      const bool ahead3 = s + NSTAGE - 1 < n_st;
      StagePlan pl{};
      if (ahead3) pl = plan(s + NSTAGE - 1);
      const uint32_t stage_off = (s & (NSTAGE - 1)) * STAGE_BYTES;
      const LDS_AS uint8_t* lds0 = (LDS_AS uint8_t*)smem;
      const LDS_AS float* st_alpha = (const LDS_AS float*)(lds0 + stage_off + CONTENT_BYTES + ROPE_BYTES);
      const int tok0 = lo + s * ST;
      const bool page_ok = (vmask >> (s & 3)) & 1u;
      if (!page_ok) err = 1;
      // rows r of this stage with r < lim are visible to this wave
      const int lim = page_ok ? hi_w - tok0 : 0;
      int overflow = 0;

      if (!wave_active && ahead3) {
#pragma unroll
        for (int k = 0; k < LOADS; ++k) load(pl, k);
      }
      if (wave_active) {
        // Per-lane LDS byte offsets inside the stage.  The XOR swizzle only
        // touches the low 4 bits of a chunk index, and a chunk index splits
        // into disjoint bit fields, so every read is (per-lane base) XOR
        // (constant) plus a compile-time offset above those bits (stage bases
        // are multiples of 1024 and commute with the XORs):
        //  QK row read, token 16 tt + l16, chunk 4 kk + q4:
        //    [l16*1024 + ((q4 ^ f(l16)) << 4)] ^ (64 (kk % 4)) + 256 (kk / 4) + 1024 * 16 tt
        //  RoPE row read, chunk 4 kk + q4 (kk < 2):
        //    [l16*128 + ((q4 ^ f_R(l16)) << 4)] ^ (64 kk) + 128 * 16 tt
        //  PV transposed read of latents 16 om .. +15, tokens 4 q4 + (0..3) and
        //  + 16: row t = 4 q4 + l16 / 4, chunk 2 om + c1 with c1 = (l16 % 4) / 2,
        //  byte 8 (l16 % 2) of the chunk:
        //    [t*1024 + 8 (l16 % 2) + ((c1 ^ f(t)) << 4)] ^ (32 (om % 8)) + 256 (om / 8) [+ 1024 * 16]
        uint32_t qk_b, rp_b, pv_b;
        {
          const int ln = fresh_lane();
          const int lt = ln & 15, lq = ln >> 4;
          const int t = 4 * lq + (lt >> 2);
          qk_b = lt * 1024 + ((lq ^ swz(lt)) << 4) + stage_off;
          rp_b = lt * 128 + ((lq ^ swz_rope(lt)) << 4) + stage_off + CONTENT_BYTES;
          pv_b = t * 1024 + 8 * (lt & 1) + ((((lt & 3) >> 1) ^ swz(t)) << 4) + stage_off;
        }
        // ---- QK for the 32 tokens (two 16-token tiles): content, alpha, RoPE ----
        f32x4 sc[2] = {f32x4{}, f32x4{}};
        {
          // steps n = (k4, kh, tt) in that order; kk = 4 kh + k4
          constexpr int NK = 4 * (R / 128) * 2;
          bf16x8 abuf[QK_AHEAD];
          const uint32_t base = opaque(qk_b);
          auto rd = [&](int n) {
            const int k4 = n >> 3, kh = (n >> 1) & 3, tt = n & 1;
            return lds_read16(lds0 + (base ^ (64u * k4)) + 256 * kh + 1024 * 16 * tt);
          };
#pragma unroll
          for (int n = 0; n < QK_AHEAD; ++n) abuf[n] = rd(n);
#pragma unroll
          for (int n = 0; n < NK; ++n) {
            const bf16x8 a = abuf[n % QK_AHEAD];
            if (n + QK_AHEAD < NK) abuf[n % QK_AHEAD] = rd(n + QK_AHEAD);
            const int k4 = n >> 3, kh = (n >> 1) & 3, tt = n & 1;
            sc[tt] = mfma(a, qb[4 * kh + k4], sc[tt]);
            if (n % 5 == 2 && n / 5 < LOADS && ahead3) load(pl, n / 5);
          }
        }
        if (USE_ALPHA) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int t = 16 * tt + 4 * q4;  // rows of the four registers
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[tt][j] *= aq * st_alpha[(t + j) * groups + g];
          }
        }
        {
          const uint32_t base = opaque(rp_b);
#pragma unroll
          for (int kk = 0; kk < DR / 32; ++kk) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const bf16x8 a = lds_read16(lds0 + (base ^ (64u * kk)) + 128 * 16 * tt);
              sc[tt] = mfma(a, qrb[kk], sc[tt]);
            }
          }
        }
        // ---- mask rows past the visible end (tail page, causal window, bad page)
        if (lim < ST) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (16 * tt + 4 * q4 + j >= lim) sc[tt][j] = -INFINITY;
        }
        // ---- probabilities against the fixed reference ----
        float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        mx = head_max(mx);
        m_seen = fmaxf(m_seen, mx);
        if (m_ref == -INFINITY) m_ref = mx;  // first visible tokens of the split
        if ((mx - m_ref) * c2 > kMaxExp2) overflow = 1;
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
        bf16x8 pb;  // P^T as the B operand: elements 0-3 tile 0, 4-7 tile 1
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const __bf16 pr = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sc[tt][j], c2, -mc)));
            pb[4 * tt + j] = pr;
            l_run += static_cast<float>(pr);
          }
        // ---- PV: O^T[512 x 16] += C^T[512 x 32 tok] . P^T ----
        {
          // products n = (o8, oh) in that order; om = 8 oh + o8
          constexpr int NP = 8 * (R / 128);
          bf16x8 abuf[PV_AHEAD];
          const uint32_t base = opaque(pv_b);
          auto rd = [&](int n) {
            const int o8 = n >> 2, oh = n & 3;
            const uint32_t a_off = (base ^ (32u * o8)) + 256 * oh;
            const bf16x4 lo4 = lds_read_tr(lds0 + a_off);
            const bf16x4 hi4 = lds_read_tr(lds0 + a_off + 16 * 1024);
            return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          };
#pragma unroll
          for (int n = 0; n < PV_AHEAD; ++n) abuf[n] = rd(n);
#pragma unroll
          for (int n = 0; n < NP; ++n) {
            const bf16x8 a = abuf[n % PV_AHEAD];
            if (n + PV_AHEAD < NP) abuf[n % PV_AHEAD] = rd(n + PV_AHEAD);
            acc[8 * (n & 3) + (n >> 2)] = mfma(a, pb, acc[8 * (n & 3) + (n >> 2)]);
          }
        }
      }
      // did any head outgrow its reference?
      if (__builtin_amdgcn_ballot_w64(overflow != 0)) *flag = 1;
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(*flag)) {
        again = true;
        break;
      }
    }
    if (again) {
      // restart the split with the largest logit seen as the reference; every
      // wave has read the flag before it is cleared
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) *flag = 0;
      m_ref = m_seen;
    }
  } while (again);

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // an empty split never waited for its loads
  // ---- epilogue: o_p = acc / l, lse_p = scale * m_ref + ln l ----
  if (wave_active) {
    const float l_tot = head_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const size_t row_e = ((size_t)b * s_q + i) * heads + h0 + (fresh_lane() & 15);
    float* out = o_part + (row_e * num_splits + p) * R;
#pragma unroll
    for (int om = 0; om < R / 16; ++om) {
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = acc[om][j] * inv;
      *reinterpret_cast<f32x4*>(out + 16 * om + 4 * q4) = v;
    }
    if (q4 == 0) {
      lse_part[row_e * num_splits + p] =
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
