// Matrix-core split-KV decode for gfx950 (MI355X): bf16 latent cache, r = 512,
// d_R = 64, heads per KV group a multiple of 32.
//
// What it computes (QK-Normed MLA summary, "Metodologia", decode-logit
// equation; the RoPE dot of the shared RoPE key from the MQA-absorbed path of
// the GQLA summary, section 2): for query row (b, i, h) and split p, over the
// visible tokens t of the split,
//   l_t = scale * ((q~ . c_t) alpha^q alpha^k_{t,g(h)} + q^R . k^R_t)
//   o_p = sum_t softmax(l)_t c_t,   lse_p = ln sum_t e^{l_t}
// The inverse-RMS factors are a row (alpha^q, one per head) by column
// (alpha^k, one per token) scaling of the content logits: their product tile is
// one float32 outer product on the matrix core, and it is applied in registers
// as one fused multiply-add per logit that also adds the RoPE dot.  Nothing
// extra is read or written for them beyond the 4 bytes per token and group of
// the scalar cache.
//
// Work decomposition
//   one workgroup (4 waves, one per SIMD) per (sequence b, split p, block of
//   128 query rows); wave w owns 32 query rows = 32 heads of one query token,
//   all in one KV group.  Every token of the split is read from HBM once and
//   shared by the 4 waves through LDS.  With 32 heads per wave every latent
//   row read from LDS feeds 32 heads, which keeps the LDS traffic of a stage
//   (272 KB per CU) below what the matrix cores need in time.  A wave keeps
//   q~ and q^R (144 VGPRs) for the whole kernel and its 32 x 512 latent
//   accumulator in the 256 AGPRs.
//
// Per 32-token stage (half a page):
//   HBM -> LDS   LDS-DMA loads of 16 B per lane (buffer_load ... lds) into a
//                ring of 4 stage buffers: while stage s is multiplied, stage
//                s - 1 is still read by PV and stages s + 1, s + 2 are on their
//                way.  The buffer descriptor of a stage ends at its last valid
//                token, so a partial page reads zeros beyond it; an invalid
//                page entry reads zeros throughout.  The loads are spread over
//                the QK products.
//   QK           the RoPE dot R^T = K^R . q^R^T and the factor tile F^T =
//                alpha^k alpha^q^T (v_mfma_f32_32x32x2f32) first, off the path
//                to the softmax, then S_c^T[32 tok x 32 heads] = C[32 x 512] . q~^T
//                (v_mfma_f32_32x32x16_bf16, A = latent rows from LDS, B = q~ in
//                registers); S = S_c F + R, one fused multiply-add per logit,
//                in the first softmax steps.
//   softmax      base 2 against a per-head reference fixed at the first
//                visible tokens of the split, so the accumulator is never
//                rescaled inside the loop.  QK-norm bounds the logits, so the
//                probabilities stay far below the 2^96 headroom allowed; should
//                a later logit exceed it, the workgroup restarts the split with
//                the larger reference (exact; never seen with normalised
//                logits).  A head's 32 tokens sit in lanes l and l ^ 32.
//   PV           O^T[512 x 32 heads] += C^T . P^T, the C^T operand read with
//                ds_read_b64_tr_b16 straight from the row-major stage in LDS;
//                the token order inside a 16-token step follows the register
//                layout of the S^T tile (both operands use the same
//                permutation of the reduction index, which leaves the sum
//                unchanged).  PV of stage s - 1 is issued together with the
//                softmax of stage s, so the vector ALU work of one stage runs
//                under the matrix products of the previous one.
// LDS layout of a stage (bytes): content [32][1024] with the 16-byte chunk c of
// token t stored at chunk position c ^ f(t) (f below), RoPE keys [32][128] with
// chunk c of token t at c ^ ((t >> 1) & 7), then alpha^k [G][32].  The
// swizzles spread the row reads of QK and the transposed reads of PV over the
// LDS banks.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
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
constexpr int kMaxGroups = 8;
constexpr int ALPHA_BYTES = ST * kMaxGroups * 4;  // 1024
constexpr int STAGE_BYTES = CONTENT_BYTES + ROPE_BYTES + ALPHA_BYTES;  // 37888
constexpr int FLAG_OFFSET = NSTAGE * STAGE_BYTES; // the workgroup's restart flag
constexpr int LDS_BYTES = FLAG_OFFSET + 16;       // 151568
// selected-token decode: the cache rows of a split's list entries, as a table
// in LDS after the flag (at most this many entries per split)
constexpr int kSelMaxPerSplit = 2048;
constexpr int SEL_TABLE_BYTES = 4 * kSelMaxPerSplit;
constexpr int WAVES = 4;
constexpr int HEADS_PER_WAVE = 32;
constexpr int ROWS_PER_WG = WAVES * HEADS_PER_WAVE;  // 128
constexpr int LOADS = ST / WAVES + 2;             // per wave and stage: 8 content, RoPE, alpha
constexpr int QK_AHEAD = 3;                      // LDS reads in flight ahead of the MFMAs
constexpr int PV_AHEAD = 3;
constexpr float kMaxExp2 = 96.0f;                 // headroom of p = 2^(y - ref), log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// content chunk position of chunk c of token t: c ^ f(t mod 16), f the
// linear map over GF(2)^4 with f(1) = 9, f(2) = 5, f(4) = 2, f(8) = 6.  Chosen
// by measuring, on gfx950, every invertible map for the two read patterns of
// this kernel (32 rows x one chunk for QK, 8 rows x 4 chunks of transposed
// 8-byte reads for PV); this one runs both near the best rate seen.
// f(integral_constant<int, I>) for I = B .. E - 1, in order, each I a
// compile-time constant: the products of a stage and the vector steps placed
// between them are straight-line code whatever the size of the loop body.
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

__device__ __forceinline__ int swz(int t) {
  return static_cast<int>((0x81d4a3f6e7b2c590ull >> (4 * (t & 15))) & 15);
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
// Every cache line is read exactly once, so the loads are marked
// non-temporal (nt): they do not displace the split partials this kernel
// writes, which the combine reads next.
// Issued through asm so that the compiler does not hold every LDS read until
// all DMA in flight has landed; completion is awaited explicitly (vmcnt)
// before the barrier that publishes a stage.  Wait states: one after the
// scalar write of M0 (s_nop 0); the first load through a descriptor also
// covers the five a vector memory instruction needs after a vector
// instruction (v_readfirstlane) wrote one of its SGPRs (s_nop 4).
template <bool FIRST_USE>
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  if (FIRST_USE) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
  } else {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
  }
}

// 4 bytes per lane from rsrc + voff to LDS (M0 + 4 * lane); wait states as above
__device__ __forceinline__ void dma4_first(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ bf16x8 lds_read16(const LDS_AS uint8_t* p) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(p);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<LDS_AS bf16x4*>(const_cast<LDS_AS uint8_t*>(p)));
}

// A per-lane value the compiler must take as new at this point: the empty
// volatile asm keeps the addresses derived from it inside the stage loop (one
// instruction each per stage) instead of being hoisted out of the loop and
// held in registers for the whole kernel, where they would not fit.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Outer product of two float32 vectors in the 32 x 32 tile layout: lane l
// gives a[l % 32] (row factor) and b[l % 32] (column factor); the second term
// of the K = 2 product pairs lanes 32..63 of a with lanes 32..63 of b, which
// must be 0 in b (a finite there).  Element (i, j) = a_i b_j, rounded once.
__device__ __forceinline__ f32x16 outer32(float a, float b) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, f32x16{}, 0, 0, 0);
}

// PV product into an accumulator tile kept in the AGPR file.  Issued through
// asm so that the compiler keeps the 256 accumulator registers of a wave there
// and the VGPRs free for the operands.  Hazards the compiler cannot see
// through asm: 2 wait states before the MFMA reads operands written by the
// vector ALU (s_nop 1), and wait_acc_results() before anything reads the
// accumulator back.
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+a"(acc) : "v"(a), "v"(b));
}
// wait states between an MFMA writing registers and a vector instruction
// reading them (covers the longest MFMA; 3 x 8)
__device__ __forceinline__ void wait_acc_results() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// max / sum over the two lanes l, l ^ 32 that hold one head.  With both
// operands v, v_permlane32_swap returns the two halves of the wave, which pair
// lane l with lane l ^ 32 in every lane.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// SPARSE: the selected-token variant.  Query token (b, i) attends to the cache
// tokens listed in sel[b][i][0 .. sel_len) (logical positions, -1 = unused
// entry); split p takes list entries p L .. p L + L - 1, L = sel_len / P
// rounded up to whole 32-entry stages.  A workgroup's rows are then one query
// token (heads a multiple of 128, checked by the host), so its waves share the
// list.  Stage rows are gathered by cache row instead of by page.
template <bool USE_ALPHA, bool SPARSE>
__global__ __launch_bounds__(64 * WAVES, 1) void decode_mfma_kernel(
    const uint16_t* __restrict__ q_tilde, const float* __restrict__ alpha_q,
    const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ kv,
    const float* __restrict__ alpha_k, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel, int sel_len,
    _Float16* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ err_flag, int batch, int s_q, int heads,
    int groups, int max_pages, int num_pages, int num_splits, int row_blocks, int n_work,
    int per_xcd, float scale) {
  // a static allocation: its LDS address (0) is known when the kernel is
  // compiled, so stage offsets fold into the read instructions
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES + (SPARSE ? SEL_TABLE_BYTES : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // The work item (sequence b, split p, row block rb) of this block.  Blocks
  // are dealt to the 8 XCDs round-robin (block 8 j + x is the j-th of XCD x)
  // and the CUs of an XCD take its blocks in order as they free up.
  //  - Equal lengths, or a batch over 64: XCD x takes the consecutive items
  //    x n/8 .. (x + 1) n/8 - 1, so that the row blocks and splits of one
  //    sequence share an L2.
  //  - Ragged lengths: the (sequence, split) pairs, longest sequence first,
  //    are dealt round-robin over the XCDs, the row blocks of a pair staying
  //    together (they read the same pages).  Each XCD then holds the same
  //    mix of lengths and takes its longest items first, which keeps the
  //    XCDs, and the CUs of each, within about one item of one another.
  const int wg = blockIdx.x;
  int b, p, rb;
  int tl = 0;  // length of sequence `lane` (batch <= 64)
  {
    bool ragged = false;
    int rank = 0;  // place of sequence `lane` in the order (longest first, ties by index)
    if (!SPARSE && batch <= 64) {
      tl = lane < batch ? seq_lens[lane] : 0;
      const int t0 = __builtin_amdgcn_readfirstlane(tl);
      ragged = __ballot(lane < batch && tl != t0) != 0;
      if (ragged) {
        for (int j = 0; j < batch; ++j) {
          const int tj = __builtin_amdgcn_readlane(tl, j);
          rank += (tj > tl || (tj == tl && j < lane)) ? 1 : 0;
        }
      }
    }
    if (ragged) {
      const int pos = wg >> 3;
      rb = pos % row_blocks;
      const int k = (pos / row_blocks) * 8 + (wg & 7);  // pair k of the order
      if (k >= batch * num_splits) return;
      const int o = k / num_splits;
      p = k - o * num_splits;
      // the ranks are a permutation of 0 .. batch - 1: exactly one lane has rank o
      b = static_cast<int>(__builtin_ctzll(__ballot(lane < batch && rank == o)));
    } else {
      if ((wg >> 3) >= per_xcd) return;
      const int work = (wg & 7) * per_xcd + (wg >> 3);
      if (work >= n_work) return;
      rb = work % row_blocks;
      p = (work / row_blocks) % num_splits;
      b = work / (row_blocks * num_splits);
    }
  }
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int l32 = lane & 31;  // head within the wave
  const int hh = lane >> 5;   // which 8-wide half of a 16-long reduction step
  int err = 0;
  bool restarted = false;

  int T = (!SPARSE && batch <= 64) ? __builtin_amdgcn_readlane(tl, b) : seq_lens[b];
  if (T < 0 || T > max_pages * PAGE) {
    err = 1;
    T = min(max(T, 0), max_pages * PAGE);
  }
  // split p: tokens lo .. hi - 1 of the sequence (list entries lo .. hi - 1 when SPARSE)
  const int L = SPARSE ? ST * cdiv(cdiv(max(sel_len, 1), num_splits), ST)
                       : split_len(max(T, 1), num_splits);
  const int lo = p * L;
  const int hi = min(lo + L, SPARSE ? sel_len : T);
  const int first_page = lo / PAGE;  // lo is a multiple of the page size
  const int n_st = hi > lo ? (hi - lo + ST - 1) / ST : 0;

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

  // The prologue's memory traffic overlaps: the first page of the split comes
  // in by a scalar load, its two stages are issued as soon as it is in, and
  // alpha^q, q~, q^R and the page-table window follow (vector loads; the
  // page loads go first so that the HBM round trip starts early).  One wait
  // for everything then precedes the first stage.  (The page loads are not
  // visible to the compiler's own waits, so every vector load the compiler
  // issued must be complete before the loop.)
  const int first_pg = (!SPARSE && first_page < max_pages && n_st > 0)
                           ? block_table[(size_t)b * max_pages + first_page] : -1;
  float aq;
  // q~ and q^R as the B operand of QK: lane holds q[head l32][16 kk + 8 hh .. +8]
  bf16x8 qb[R / 16];
  bf16x8 qrb[DR / 16];
  auto load_query = [&]() {
    aq = USE_ALPHA ? alpha_q[my_row] : 1.f;
    const bf16x8* qt = reinterpret_cast<const bf16x8*>(q_tilde + my_row * R) + hh;
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) qb[kk] = qt[2 * kk];
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_rope + my_row * DR) + hh;
#pragma unroll
    for (int kk = 0; kk < DR / 16; ++kk) qrb[kk] = qr[2 * kk];
  };
  // Page-table window: lane j of every wave holds the entry of split page
  // wbase + j (64 pages, 4096 tokens), so a stage finds its page with one
  // v_readlane instead of a memory round trip inside the loop.
  int wbase = 0;
  int pwin;
  auto load_window = [&](int base) {
    const int j = first_page + base + lane;
    pwin = j < max_pages ? block_table[(size_t)b * max_pages + j] : -1;
  };

  // ---- per-lane constants of the LDS traffic (stage offsets are added per
  // stage, or folded into the instructions' immediate offsets) ----
  // DMA: content token t = w + 4k goes to chunk lane ^ f(t), i.e. byte
  // (16 lane) ^ (16 f(t)) of its row
  const uint32_t lane16 = static_cast<uint32_t>(lane << 4);
  // RoPE keys of tokens 8w .. 8w + 7: token 8w + lane / 8, chunk (lane % 8) ^ f_R(token)
  const uint32_t dma_r = static_cast<uint32_t>(
      (8 * w + (lane >> 3)) * ROW_BYTES + R * 2 + (((lane & 7) ^ swz_rope(8 * w + (lane >> 3))) << 4));
  // alpha^k of the stage transposed to [G][32 tokens]: slot i = g * 32 + t
  // takes element (t, g) of the rows; wave w fills slots 8Gw .. 8Gw + 8G - 1
  const bool dma_a_lane = lane < 8 * groups;
  const uint32_t dma_a = static_cast<uint32_t>(
      (((8 * groups * w + lane) & 31) * groups + ((8 * groups * w + lane) >> 5)) * 4);
  // QK row read of token l32, chunk 2 kk + hh:
  //   [l32*1024 + ((hh ^ f(l32)) << 4)] ^ (32 (kk % 8)) + 256 (kk / 8)
  const uint32_t qk_lane = static_cast<uint32_t>(l32 * 1024 + ((hh ^ swz(l32)) << 4));
  // RoPE row read, chunk 2 kk + hh (kk < 4): [l32*128 + ((hh ^ f_R(l32)) << 4)] ^ (32 kk)
  const uint32_t rp_lane =
      static_cast<uint32_t>(l32 * 128 + ((hh ^ swz_rope(l32)) << 4) + CONTENT_BYTES);
  // PV transposed read of latents 32 om .. +31, tokens 16 ks + 4 hh + (0..3)
  // [+ 8]: within a 16-lane group G, row t = 4 hh + l16 / 4, chunk 4 om + 2 G +
  // (l16 % 4) / 2, byte 8 (l16 % 2):
  //   [t*1024 + 8 (l16 % 2) + ((c_lo ^ f(t)) << 4)] ^ (64 (om % 4)) + 256 (om / 4) + 16384 ks
  // with c_lo = 2 G + (l16 % 4) / 2; the + 8 rows use their own base.
  uint32_t pv_lane0, pv_lane1;
  {
    const int l16 = lane & 15, G16 = (lane >> 4) & 1;
    const int t = 4 * hh + (l16 >> 2);
    const int c_lo = 2 * G16 + ((l16 & 3) >> 1);
    pv_lane0 = static_cast<uint32_t>(t * 1024 + 8 * (l16 & 1) + ((c_lo ^ swz(t)) << 4));
    pv_lane1 = static_cast<uint32_t>((t + 8) * 1024 + 8 * (l16 & 1) + ((c_lo ^ swz(t + 8)) << 4));
  }
  const uint32_t ak_lane = static_cast<uint32_t>(CONTENT_BYTES + ROPE_BYTES + (g * ST + l32) * 4);

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS uint8_t*)smem));
  const LDS_AS uint8_t* lds0 = (LDS_AS uint8_t*)smem;
  // validity of the pages of the stages in the ring, bit s mod 4 (uniform)
  uint32_t vmask = 0;

  // The 10 loads of this wave for stage s (tokens lo + 32 s ..) into buffer
  // s mod 4: 8 content rows, a quarter of the RoPE block, and a quarter of
  // alpha^k on lanes 0 .. 8G-1 (lane 0 always takes part, so every wave
  // issues all 10 and the vmcnt bookkeeping holds).  The two stages of a page
  // share its plan: plan_page() looks the page up and builds descriptors that
  // end at its last valid token; load(k) issues load k of either half (the
  // second half starts 32 rows into the page).
  struct PagePlan {
    i32x4 rs, ra;  // KV rows of the page, alpha^k rows of the page
  };
  auto plan_page = [&](int s, auto FIRST) {  // s: the first stage of the page (even)
    const int rel = s >> 1;  // page of the split
    PagePlan pp;
    if (s >= n_st) {
      // no such page: its loads read nothing (size 0) and write zeros into a
      // buffer nobody reads, which keeps the load count of every stage the same
      pp.rs = buffer_rsrc(kv, 0);
      pp.ra = buffer_rsrc(alpha_k, 0);
      return pp;
    }
    int pg;
    if constexpr (decltype(FIRST)::value) {
      pg = first_pg;  // the split's first page, from its own scalar load
    } else {
      if (rel < wbase || rel >= wbase + 64) {  // uniform; once per 64 pages
        wbase = rel & ~63;
        load_window(wbase);
        // a wait the compiler sees, so that it adds none of its own at every
        // later use of the window (which would also wait for the page loads)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      }
      pg = __builtin_amdgcn_readlane(pwin, rel - wbase);
    }
    pg = (pg >= 0 && pg < num_pages) ? pg : -1;
    const uint32_t ok = pg >= 0 ? 3u : 0u;  // validity of both stages of the page
    vmask = (vmask & ~(3u << (s & 3))) | (ok << (s & 3));
    const int tok0 = lo + s * ST;
    const int nv = pg >= 0 ? min(PAGE, T - tok0) : 0;   // valid rows of the page
    const size_t row0s = (size_t)(pg >= 0 ? pg : 0) * PAGE;  // cache row
    pp.rs = buffer_rsrc(reinterpret_cast<const uint8_t*>(kv) + row0s * ROW_BYTES, nv * ROW_BYTES);
    // the alpha-free instantiation reads no alpha^k bytes: its loads are still
    // issued (every stage keeps the same load count) but read nothing
    pp.ra = buffer_rsrc(alpha_k + row0s * groups, USE_ALPHA ? nv * groups * 4 : 0);
    return pp;
  };
  struct StagePlan {
    i32x4 rs, ra;    // the page's descriptors (SPARSE: the whole cache's)
    uint32_t buf;    // LDS address of the stage buffer
    uint32_t half;   // which half of the page (0, 1)
    uint32_t l16;    // 16 * lane, taken as new for this stage (see opaque)
    // SPARSE: lane l holds the byte offset of the stage's entry l % 32 in the
    // cache (a zero-reading offset for an unused or invalid entry) and its
    // cache row (-1 for none); vm has bit l set for a valid entry l
    uint32_t off;
    int row;
    uint32_t vm;
  };
  auto stage_plan = [&](const PagePlan& pp, int s) {
    StagePlan pl;
    pl.rs = pp.rs;
    pl.ra = pp.ra;
    pl.buf = lds_base + (s & (NSTAGE - 1)) * STAGE_BYTES;
    asm volatile("" : "+s"(pl.buf));  // keep the per-load LDS addresses out of loop-invariant registers
    pl.half = static_cast<uint32_t>(s & 1);
    pl.l16 = opaque(lane16);
    return pl;
  };
  // SPARSE: descriptors over the whole cache (its size fits 32-bit offsets,
  // checked by the host) and the entries' cache rows in LDS
  const uint32_t kv_bytes = static_cast<uint32_t>(num_pages) * PAGE * ROW_BYTES;
  const uint32_t ak_bytes = static_cast<uint32_t>(num_pages) * PAGE * groups * 4;
  const LDS_AS int* sel_rows = (const LDS_AS int*)((LDS_AS uint8_t*)smem + LDS_BYTES);
  auto gather_plan = [&](int s) {
    StagePlan pl;
    pl.rs = buffer_rsrc(kv, kv_bytes);
    pl.ra = buffer_rsrc(alpha_k, USE_ALPHA ? ak_bytes : 0);
    pl.buf = lds_base + (s & (NSTAGE - 1)) * STAGE_BYTES;
    asm volatile("" : "+s"(pl.buf));
    pl.half = 0;
    pl.l16 = opaque(lane16);
    pl.row = s < n_st ? sel_rows[s * ST + (lane & 31)] : -1;
    pl.off = pl.row >= 0 ? static_cast<uint32_t>(pl.row) * ROW_BYTES : kv_bytes;
    pl.vm = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(pl.row >= 0));
    return pl;
  };
  auto load = [&](const StagePlan& pl, int k) {
    if constexpr (SPARSE) {
      if (k < ST / WAVES) {
        // content token t = w + 4k from its own cache row
        const int t = w + WAVES * k;
        const uint32_t voff = (pl.l16 ^ static_cast<uint32_t>(swz(t) << 4)) +
                              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pl.off), t));
        if (k == 0) {
          dma16<true>(pl.buf + t * 1024, voff, pl.rs);
        } else {
          dma16<false>(pl.buf + t * 1024, voff, pl.rs);
        }
      } else if (k == ST / WAVES) {
        // RoPE key of token 8w + lane / 8 from its row
        const int tr = 8 * w + (lane >> 3);
        const uint32_t row_off = static_cast<uint32_t>(__shfl(static_cast<int>(pl.off), tr));
        const uint32_t voff = row_off == kv_bytes ? kv_bytes
                              : row_off + static_cast<uint32_t>(R * 2 + (((lane & 7) ^ swz_rope(tr)) << 4));
        dma16<false>(pl.buf + CONTENT_BYTES + w * 1024, voff, pl.rs);
      } else {
        // alpha^k slot i = 8Gw + lane: token i % 32, group i / 32
        const int si = 8 * groups * w + lane;
        const int row = __shfl(pl.row, si & 31);
        const uint32_t voff = row >= 0 ? static_cast<uint32_t>((row * groups + (si >> 5)) * 4) : ak_bytes;
        if (dma_a_lane)
          dma4_first(pl.buf + CONTENT_BYTES + ROPE_BYTES + 32 * groups * w, voff, pl.ra);
      }
      return;
    }
    if (k < ST / WAVES) {
      // content token t = w + 4k at t * ROW_BYTES; the lane's chunk is lane ^ f(t)
      const int t = w + WAVES * k;
      const uint32_t voff = (pl.l16 ^ static_cast<uint32_t>(swz(t) << 4)) +
                            static_cast<uint32_t>(t * ROW_BYTES) + pl.half * (ST * ROW_BYTES);
      if (k == 0) {
        dma16<true>(pl.buf + t * 1024, voff, pl.rs);
      } else {
        dma16<false>(pl.buf + t * 1024, voff, pl.rs);
      }
    } else if (k == ST / WAVES) {
      dma16<false>(pl.buf + CONTENT_BYTES + w * 1024, opaque(dma_r) + pl.half * (ST * ROW_BYTES), pl.rs);
    } else {
      if (dma_a_lane)
        dma4_first(pl.buf + CONTENT_BYTES + ROPE_BYTES + 32 * groups * w,
                   opaque(dma_a) + pl.half * (ST * 4 * groups), pl.ra);
    }
  };

  // column operand of the alpha^k alpha^q product tile (see outer32), formed
  // where it is used (opaque keeps it there), so that no wait for alpha^q
  // precedes the first page loads
  auto aq_col = [&]() { return hh == 0 ? __uint_as_float(opaque(__float_as_uint(aq))) : 0.f; };

  f32x16 acc[R / 32];
  float m_ref = -INFINITY;   // reference of the exponent for this lane's head (logit units)
  float m_seen = -INFINITY;  // largest logit of this head seen so far
  float l_run = 0.f;         // this lane's share of the softmax denominator
  const float c2 = scale * kLog2e;  // logits -> log2 units
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  // restart flag: set by any wave whose logits outgrew the reference, read by
  // all after the next barrier
  volatile LDS_AS int* flag = (volatile LDS_AS int*)((LDS_AS uint8_t*)smem + FLAG_OFFSET);
  if (tid == 0) *flag = 0;

  // PV of "stage -1" reads buffer 3 with zero probabilities: clear that
  // buffer once so that it holds finite values (later it only ever holds
  // cache rows or zeros)
  {
    const f32x4 z = {};
    for (int e = tid; e < CONTENT_BYTES / 16; e += 64 * WAVES)
      *reinterpret_cast<LDS_AS f32x4*>((LDS_AS uint8_t*)smem + 3 * STAGE_BYTES + 16 * e) = z;
  }

  if constexpr (SPARSE) {
    // The cache row of every list entry of the split (-1: unused or invalid),
    // into LDS: the list entries first, then the query loads (their latency
    // overlaps the page-table lookups), then the lookups.  An entry that is
    // not -1 and lies outside the visible tokens 0 .. T - s_q + i, or whose
    // page entry is out of range, is reported.
    constexpr int PER = kSelMaxPerSplit / (64 * WAVES);
    const int n_e = hi > lo ? hi - lo : 0;
    const int vis = T - s_q + i + 1;
    const int32_t* srow = sel + ((size_t)b * s_q + i) * sel_len + lo;
    int tv[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 64 * WAVES * u;
      tv[u] = e < n_e ? srow[e] : -1;
    }
    load_query();
    LDS_AS int* rows_w = (LDS_AS int*)((LDS_AS uint8_t*)smem + LDS_BYTES);
    bool bad = false;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 64 * WAVES * u;
      if (e < n_st * ST) {
        const int t = tv[u];
        int row = -1;
        if (t != -1) {
          const int pg = (t >= 0 && t < vis) ? block_table[(size_t)b * max_pages + t / PAGE] : -1;
          if (pg >= 0 && pg < num_pages) row = pg * PAGE + t % PAGE;
          else bad = true;
        }
        rows_w[e] = row;
      }
    }
    if (__builtin_amdgcn_ballot_w64(bad)) err = 1;
    __syncthreads();
  }
  // masks of valid entries of stages s and s + 1 at iteration s (SPARSE)
  uint32_t vm_cur = 0, vm_next = 0;

  bool again;
  do {
    again = false;
#pragma unroll
    for (int om = 0; om < R / 32; ++om) acc[om] = f32x16{};
    l_run = 0.f;
    PagePlan page;
    if constexpr (!SPARSE) page = plan_page(0, std::true_type{});
    {
      const StagePlan p0 = SPARSE ? gather_plan(0) : stage_plan(page, 0);
      vm_cur = p0.vm;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) load(p0, k);
    }
    if (!SPARSE && !restarted) {  // the first pass: the query side and the page window
      load_query();
      load_window(0);
    }
    // stage 0 has landed, and so has every vector load of the prologue; the
    // loads of stage 1 go out now (fewer bytes ahead of the first stage, when
    // every CU asks for its first pages at once), the loop waits for them
    // at the end of its first iteration
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    {
      const StagePlan p1 = SPARSE ? gather_plan(1) : stage_plan(page, 1);
      vm_next = p1.vm;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) load(p1, k);
    }
    __syncthreads();
    // probabilities of the previous stage / of this one, swapped every stage
    bf16x8 pA[2] = {}, pB[2];

    // PV of stage sp with the probabilities pb: O^T[512 x 32] += C^T[512 x 32
    // tok] . P^T over two 16-token steps, products n = (ks, om) in that
    // order, operands read PV_AHEAD products ahead; fill(n) runs after the
    // n-th product (vector work that needs no result of this PV)
    auto pv_stage = [&](int sp, const bf16x8 (&pb)[2], auto&& fill) {
      const uint32_t off_s = (sp & (NSTAGE - 1)) * STAGE_BYTES;
      uint32_t xb0[4], xb1[4];
      const uint32_t b0 = opaque(pv_lane0), b1 = opaque(pv_lane1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xb0[j] = (b0 ^ (64u * j)) + off_s;
        xb1[j] = (b1 ^ (64u * j)) + off_s;
      }
      constexpr int NP = 2 * (R / 32);
      bf16x8 pbuf[PV_AHEAD];
      auto rdp = [&](int n) {
        const int ks = n / (R / 32), om = n % (R / 32);
        const uint32_t off = 256 * (om >> 2) + 16384 * ks;
        const bf16x4 lo4 = lds_read_tr(lds0 + xb0[om & 3] + off);
        const bf16x4 hi4 = lds_read_tr(lds0 + xb1[om & 3] + off);
        return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      };
#pragma unroll
      for (int n = 0; n < PV_AHEAD; ++n) pbuf[n] = rdp(n);
      __builtin_amdgcn_sched_barrier(0);
      Unroll<0, NP>::run([&](auto N) {
        constexpr int n = decltype(N)::value;
        const bf16x8 a = pbuf[n % PV_AHEAD];
        if constexpr (n + PV_AHEAD < NP) pbuf[n % PV_AHEAD] = rdp(n + PV_AHEAD);
        mfma_acc(acc[n % (R / 32)], a, pb[n / (R / 32)]);
        fill(N);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // iteration s: QK and softmax of stage s (s < n_st) and PV of stage s - 1;
    // it ends with the one barrier of the iteration, after which stage s + 1
    // is in LDS, every wave is done with stage s - 1, and the restart flag
    // of stage s is visible
    // one iteration; HALF = s mod 2 (the stages of a page alternate), pprev the
    // probabilities of stage s - 1, pnew those of stage s.  Returns whether the
    // split must restart.
    auto iteration = [&](auto HALF, int s, bf16x8 (&pprev)[2], bf16x8 (&pnew)[2]) -> bool {
      const bool has_qk = s < n_st;
      // the loads of stage s + 2 go into the buffer of stage s - 2; an even
      // stage s + 2 starts a page and takes its plan, an odd one reuses it
      if constexpr (!SPARSE && decltype(HALF)::value == 0) page = plan_page(s + 2, std::false_type{});
      const StagePlan pl = SPARSE ? gather_plan(s + 2) : stage_plan(page, s + 2);
      const uint32_t stage_off = (s & (NSTAGE - 1)) * STAGE_BYTES;
      const int tok0 = lo + s * ST;
      const bool page_ok = SPARSE || ((vmask >> (s & 3)) & 1u);
      if (!SPARSE && has_qk && !page_ok) err = 1;
      // rows r of this stage with r < lim are visible to this wave; past the
      // last stage none (the softmax steps then only produce zeros).  SPARSE:
      // the valid entries of the stage instead (none past the last stage).
      const int lim = SPARSE ? (has_qk ? ST : 0) : (has_qk && page_ok) ? hi_w - tok0 : 0;
      const uint32_t vm_s = has_qk ? vm_cur : 0u;
      vm_cur = vm_next;
      vm_next = pl.vm;
      int overflow = 0;

      if (!wave_active) {
#pragma unroll
        for (int k = 0; k < LOADS; ++k) load(pl, k);
      } else {
        // ---- QK: S_c^T[32 tok x 32 heads] over the 512 latents (with the
        // RoPE dot first when there are no factors).  The latent rows are read
        // QK_AHEAD products ahead; the scheduling fences keep every read and
        // product at its place in that order.
        // past the last stage the tiles keep whatever they hold: every row
        // is masked to -inf before it is used
        f32x16 sc, fac;
        bf16x8 rope_a[DR / 16];
        if (has_qk) {
          const uint32_t rp_l = opaque(rp_lane);
          constexpr int NK = R / 16;
          bf16x8 abuf[QK_AHEAD];
          // each read forms its own address right before it (one xor-add
          // from the lane base, which is taken as new for every read), so no
          // address is held in a register across the chain
          uint32_t qx[8];
          const uint32_t qk_l = opaque(qk_lane);
#pragma unroll
          for (int j = 0; j < 8; ++j) qx[j] = (qk_l ^ (32u * j)) + stage_off;
          auto rd = [&](int n) { return lds_read16(lds0 + qx[n & 7] + 256 * (n >> 3)); };
#pragma unroll
          for (int n = 0; n < QK_AHEAD; ++n) abuf[n] = rd(n);
          if (!USE_ALPHA) {
#pragma unroll
            for (int kk = 0; kk < DR / 16; ++kk)
              rope_a[kk] = lds_read16(lds0 + ((rp_l ^ (32u * kk)) + stage_off));
          }
          __builtin_amdgcn_sched_barrier(0);
          if (!USE_ALPHA) {
            sc = mfma(rope_a[0], qrb[0], f32x16{});
#pragma unroll
            for (int kk = 1; kk < DR / 16; ++kk) sc = mfma(rope_a[kk], qrb[kk], sc);
            __builtin_amdgcn_sched_barrier(0);
          }
          float ak_row = 0.f;
          Unroll<0, NK>::run([&](auto N) {
            constexpr int n = decltype(N)::value;
            const bf16x8 a = abuf[n % QK_AHEAD];
            if constexpr (n + QK_AHEAD < NK) abuf[n % QK_AHEAD] = rd(n + QK_AHEAD);
            if constexpr (USE_ALPHA && n == 0) {
              sc = mfma(a, qb[n], f32x16{});
            } else {
              sc = mfma(a, qb[n], sc);
            }
            if constexpr (n % 3 == 1 && n / 3 < LOADS) load(pl, n / 3);
            if constexpr (USE_ALPHA) {
              // near the chain's end, in the registers its last reads free:
              // alpha^k of token l % 32 and two RoPE rows, then F^T =
              // alpha^k alpha^q as one float32 outer product (outer32),
              // independent of the chain
              if constexpr (n == NK - QK_AHEAD - 2)
                ak_row = *reinterpret_cast<const LDS_AS float*>(lds0 + opaque(ak_lane) + stage_off);
              if constexpr (n >= NK - 2) {
                constexpr int kk = n - (NK - 2);
                rope_a[kk] = lds_read16(lds0 + ((rp_l ^ (32u * kk)) + stage_off));
              }
              if constexpr (n == NK - 2) fac = outer32(ak_row, aq_col());
            }
            __builtin_amdgcn_sched_barrier(0);
          });
        } else {
#pragma unroll
          for (int k = 0; k < LOADS; ++k) load(pl, k);
        }
        // ---- softmax of this stage between the products of the previous
        // stage's PV.  With the factors: S = S_c F, then the RoPE products
        // accumulate onto it on the matrix core (S = S_c F + K^R q^R^T).
        // Rows past the visible end (tail page, causal window, bad page) are
        // then set to -inf.  S^T tile layout: lane holds head l32 and tokens
        // r % 4 + 8 (r / 4) + 4 hh for its 16 registers r.
        float mx = -INFINITY, mc = 0.f;
        auto softmax_step = [&](auto N) {
          constexpr int n = decltype(N)::value;
          constexpr int M = USE_ALPHA ? 3 : 0;  // steps taken by the factors and RoPE
          if constexpr (USE_ALPHA && n == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] *= fac[r];
            const uint32_t rp_l2 = opaque(rp_lane);
            rope_a[2] = lds_read16(lds0 + ((rp_l2 ^ 64u) + stage_off));
            rope_a[3] = lds_read16(lds0 + ((rp_l2 ^ 96u) + stage_off));
          } else if constexpr (USE_ALPHA && n == 1) {
            sc = mfma(rope_a[0], qrb[0], sc);
            sc = mfma(rope_a[1], qrb[1], sc);
          } else if constexpr (USE_ALPHA && n == 2) {
            sc = mfma(rope_a[2], qrb[2], sc);
            sc = mfma(rope_a[3], qrb[3], sc);
          } else if constexpr (n == M) {
            if constexpr (SPARSE) {
              if (vm_s != 0xffffffffu) {
                // register r holds token (r % 4) + 8 (r / 4) + 4 hh
                const uint32_t vl = vm_s >> (4 * hh);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  if (!((vl >> ((r & 3) + 8 * (r >> 2))) & 1u)) sc[r] = -INFINITY;
              }
            }
            if (__builtin_expect(lim < ST, 0)) {
              // register r holds token (r % 4) + 8 (r / 4) + 4 hh: compare the
              // constant part against lim - 4 hh (no per-register lane values)
              const int lim_l = lim - 4 * hh;
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if ((r & 3) + 8 * (r >> 2) >= lim_l) sc[r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
          } else if constexpr (n == M + 1) {
            mx = pair_max(mx);
            m_seen = fmaxf(m_seen, mx);
            if (m_ref == -INFINITY) m_ref = mx;  // first visible tokens of the split
            if ((mx - m_ref) * c2 > kMaxExp2) overflow = 1;
            mc = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
          } else if constexpr (n >= M + 2 && n < M + 2 + 8) {
            // P^T as the B operand of the two 16-token steps: registers 8 ks .. 8 ks + 7
            constexpr int r = 2 * (n - (M + 2));
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -mc));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[r + 1], c2, -mc));
            const bf16x2 pr = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
            pnew[r >> 3][r & 7] = pr[0];
            pnew[r >> 3][(r & 7) + 1] = pr[1];
            // the denominator is the sum of the same rounded values
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
          }
        };
        pv_stage(s - 1, pprev, softmax_step);
      }
      // did any head outgrow its reference?
      if (__builtin_amdgcn_ballot_w64(overflow != 0)) *flag = 1;
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");  // stage s + 1 has landed
      __syncthreads();
      return __builtin_amdgcn_readfirstlane(*flag) != 0;
    };
    for (int s = 0; s <= n_st; s += 2) {
      if (iteration(std::integral_constant<int, 0>{}, s, pA, pB)) {
        again = true;
        break;
      }
      if (s + 1 > n_st) break;
      if (iteration(std::integral_constant<int, 1>{}, s + 1, pB, pA)) {
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
      restarted = true;
    }
  } while (again);

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // an empty split never waited for its loads
  // ---- epilogue: o_p = acc / l, lse_p = scale * m_ref + ln l ----
  wait_acc_results();
  if (wave_active) {
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int ln = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    const size_t row_e = ((size_t)b * s_q + i) * heads + h0 + (ln & 31);
    // accumulator tile om: lane holds head l32 and latents 32 om + r % 4 +
    // 8 (r / 4) + 4 hh.  The two lanes of a head (l, l ^ 32) trade halves so
    // that each stores 8 consecutive latents as one 16-byte write: lane hh
    // takes latents 32 om + 16 j + 8 hh + 0..7 (registers 8 j .. 8 j + 7 of
    // both lanes, 4 from each).
    _Float16* out = o_part + (row_e * num_splits + p) * R + 8 * (ln >> 5);
    float mabs = 0.f;
#pragma unroll
    for (int om = 0; om < R / 32; ++om) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t h[4];  // latent pairs +0,1 / +2,3 of q = 2 j, then of q = 2 j + 1
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = acc[om][8 * j + 2 * k], x1 = acc[om][8 * j + 2 * k + 1];
          mabs = fmaxf(mabs, fmaxf(fabsf(x0), fabsf(x1)));
          h[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0 * inv, x1 * inv}, f16x2));
        }
        // lanes < 32 keep their q = 2 j pairs and take their partner's;
        // lanes >= 32 take their partner's q = 2 j + 1 pairs and keep their own
        const auto r0 = __builtin_amdgcn_permlane32_swap(h[0], h[2], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(h[1], h[3], false, false);
        const u32x4 v = {r0[0], r1[0], r0[1], r1[1]};
        *reinterpret_cast<u32x4*>(out + 32 * om + 16 * j) = v;
      }
    }
    // a partial beyond the half range was stored as +-inf (|x / l| >= 65520)
    if (mabs * inv >= 65520.f && err_flag) atomicOr(err_flag, QKN_FLAG_PARTIAL_RANGE);
    if ((ln >> 5) == 0) {
      lse_part[row_e * num_splits + p] =
          l_tot > 0.f ? m_ref * scale + log2f(l_tot) * kLn2 : -INFINITY;
    }
  }
  if (err && err_flag && lane == 0) atomicOr(err_flag, QKN_FLAG_INDEX);
  if (restarted && err_flag && tid == 0) atomicOr(err_flag, QKN_FLAG_RESTART);
}

template <bool USE_ALPHA, bool SPARSE>
hipError_t launch_typed(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s) {
  const int row_blocks = cdiv(d.s_q * d.heads, ROWS_PER_WG);
  const int n_work = d.batch * a.num_splits * row_blocks;
  const int per_xcd = cdiv(n_work, 8);
  // enough blocks for either dealing of the work items (the kernel takes the
  // longest-first one for a ragged batch of up to 64 sequences)
  const int per_xcd_ragged =
      (!SPARSE && d.batch <= 64) ? cdiv(d.batch * a.num_splits, 8) * row_blocks : 0;
  dim3 grid(8 * std::max(per_xcd, per_xcd_ragged));
  hipLaunchKernelGGL((decode_mfma_kernel<USE_ALPHA, SPARSE>), grid, dim3(64 * WAVES), 0, s,
                     static_cast<const uint16_t*>(a.q_tilde), a.alpha_q,
                     static_cast<const uint16_t*>(a.q_rope), static_cast<const uint16_t*>(a.kv),
                     a.alpha_k, a.block_table, a.seq_lens, a.sel, a.sel_len,
                     static_cast<_Float16*>(a.o_part),
                     a.lse_part, a.err_flag, d.batch, d.s_q,
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
  return a.use_alpha ? launch_typed<true, false>(d, a, s) : launch_typed<false, false>(d, a, s);
}

int sparse_decode_check(const qkn_mla_dims& d, int sel_len, int num_splits) {
  if (!mfma_decode_supported(d) || d.heads % ROWS_PER_WG != 0) return -2;
  if ((uint64_t)d.num_pages * PAGE * ROW_BYTES + ROW_BYTES >= (1ull << 32)) return -2;
  if (sel_len < 0) return -1;
  const int L = ST * cdiv(cdiv(std::max(sel_len, 1), num_splits), ST);
  return L <= kSelMaxPerSplit ? 0 : -2;
}

hipError_t launch_decode_sparse(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s) {
  return a.use_alpha ? launch_typed<true, true>(d, a, s) : launch_typed<false, true>(d, a, s);
}

}  // namespace qkn
