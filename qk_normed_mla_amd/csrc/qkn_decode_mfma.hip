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
//   in one KV group.  Every 64-token page of the split is read from HBM once
//   and shared by the 8 waves through LDS.  A wave keeps its 16 x 512 latent
//   accumulator (128 registers) and its q~ (64 registers) in registers, so two
//   waves fit on a SIMD and one wave's softmax overlaps the other's MFMAs.
//
// Per page (one pipeline stage):
//   HBM -> LDS   73 LDS-DMA loads of 16 B per lane (buffer_load ... lds), issued
//                two pages ahead into a double buffer.  The buffer descriptor of
//                a page ends at the last valid token, so a partial page reads
//                zeros beyond it; an invalid page entry reads zeros throughout.
//   QK           S^T[16 tok x 16 heads] = C[16 x 512] . q~^T  (v_mfma_f32_16x16x32_bf16,
//                A = latent rows from LDS, B = q~ held in registers for the whole
//                kernel), then S *= alpha^q alpha^k, then += K^R . q^R^T.
//   softmax      online, base 2, once per page, with the running maximum raised
//                only when a row's maximum grows by more than 8 (in log2
//                units): the probabilities stay <= 2^8 and the rescale factor
//                of the running sums is 1 almost always.  A head's tokens sit
//                in lanes l, l^16, l^32, l^48.
//   PV           O^T[512 x 16 heads] += C^T . P^T over 32-token steps, the C^T
//                operand read with ds_read_b64_tr_b16 straight from the
//                row-major page in LDS; the token order inside a step follows
//                the register layout of two S^T tiles (both operands use the
//                same permutation of the reduction index, which leaves the sum
//                unchanged).
// LDS layout of a staged page (bytes): content [64][1024] with the 16-byte
// chunk c of token t stored at chunk position c ^ f(t) (f below), RoPE keys
// [64][128] with chunk c of token t at c ^ ((t >> 1) & 7), then alpha^k [64][G].
// The swizzles make both the row reads of QK and the transposed reads of PV
// free of bank conflicts.
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
constexpr int PAGE = QKN_MLA_PAGE_SIZE;   // 64 tokens per page = per stage
constexpr int ROW_BYTES = (R + DR) * 2;   // 1152
constexpr int CONTENT_BYTES = PAGE * R * 2;       // 65536
constexpr int ROPE_BYTES = PAGE * DR * 2;         // 8192
constexpr int ALPHA_BYTES = PAGE * 16 * 4;        // room for G <= 16
constexpr int STAGE_BYTES = CONTENT_BYTES + ROPE_BYTES + ALPHA_BYTES;  // 77824
constexpr int LDS_BYTES = 2 * STAGE_BYTES;        // 155648
constexpr int WAVES = 8;
constexpr int HEADS_PER_WAVE = 16;
constexpr int ROWS_PER_WG = WAVES * HEADS_PER_WAVE;  // 128
constexpr int kMaxGroups = 16;
constexpr float kRescaleThreshold = 8.0f;         // log2 units
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

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the four lanes l, l^16, l^32, l^48 that hold one head
__device__ __forceinline__ float head_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float head_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
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
  const int first_page = lo / PAGE;
  const int n_st = hi > lo ? (hi - lo + PAGE - 1) / PAGE : 0;

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
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query operands are in registers

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS uint8_t*)smem));
  const int alpha_bytes_per_wave = PAGE * groups * 4 / WAVES;  // 32 G

  // page index of stage s (-1 when the entry is out of range)
  auto page_of = [&](int s) -> int {
    int pg = block_table[(size_t)b * max_pages + first_page + s];
    return (pg >= 0 && pg < num_pages) ? pg : -1;
  };

  // DMA source offsets inside a page.  Content token t = w + 8k starts at
  // t * ROW_BYTES; the per-lane chunk depends on t only through t mod 16 (w or
  // w + 8) in the swizzle.
  const uint32_t dma_content0 = (lane ^ swz(w)) << 4;
  const uint32_t dma_content1 = (lane ^ swz(w + 8)) << 4;
  // RoPE rows of tokens 8w .. 8w + 7: token 8 w + lane / 8, chunk (lane % 8) ^ f_R(token)
  const uint32_t dma_rope = (8 * w + (lane >> 3)) * ROW_BYTES + R * 2 +
                            (((lane & 7) ^ ((4 * w + (lane >> 4)) & 7)) << 4);
  const uint32_t dma_alpha = w * (PAGE * groups * 4 / WAVES) + lane * 16;

  // issue the 10 loads of this wave for stage s into buffer (s & 1):
  // 8 content rows, 1 RoPE block, 1 slice of alpha^k
  auto issue = [&](int s) {
    const int pg = page_of(s);
    const int tok0 = lo + s * PAGE;
    const int nv = pg >= 0 ? min(PAGE, T - tok0) : 0;   // valid rows of the page
    const uint8_t* page_ptr = reinterpret_cast<const uint8_t*>(kv) +
                              (size_t)(pg >= 0 ? pg : 0) * PAGE * ROW_BYTES;
    const i32x4 rs = buffer_rsrc(page_ptr, nv * ROW_BYTES);
    const uint32_t buf = lds_base + (s & 1) * STAGE_BYTES;
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // content: token t = w + 8k, lane -> chunk lane ^ f(t)
      const int t = w + 8 * k;
      dma16(buf + t * 1024, ((k & 1) ? dma_content1 : dma_content0) + t * ROW_BYTES, rs);
    }
    // RoPE keys of tokens 8w .. 8w + 7
    dma16(buf + CONTENT_BYTES + w * 1024, dma_rope, rs);
    {  // alpha^k of the page: 64 * G floats, an eighth per wave
      const float* ap = alpha_k + (size_t)(pg >= 0 ? pg : 0) * PAGE * groups;
      const i32x4 ra = buffer_rsrc(ap, nv * groups * 4);
      if (lane * 16 < alpha_bytes_per_wave)
        dma16(buf + CONTENT_BYTES + ROPE_BYTES + w * alpha_bytes_per_wave, dma_alpha, ra);
    }
  };

  // Per-lane LDS byte offsets inside a staged page.  The XOR swizzle only
  // touches the low bits of a chunk index, and a chunk index splits into
  // disjoint bit fields, so every read is  (per-lane base) XOR (compile-time
  // constant)  plus a compile-time offset above those bits:
  //   QK row read, token 32 tb + 16 tt + l16, chunk 4 kk + q4:
  //     [l16 * 1024 + ((q4 ^ f(l16)) << 4)] ^ (64 (kk % 4)) + 256 (kk / 4) + 1024 (32 tb + 16 tt)
  //   RoPE row read, chunk 4 kk + q4 (kk < 2):
  //     [l16 * 128 + ((q4 ^ f_R(l16)) << 4)] ^ (64 kk) + 128 (32 tb + 16 tt)
  //   PV transposed read of latents 16 om .. +15, tokens 32 tb + 4 q4 + (0..3)
  //   and + 16: row t = 4 q4 + l16 / 4, chunk 2 om + c1 with c1 = (l16 % 4) / 2,
  //   byte (l16 % 2) * 8 of the chunk:
  //     [t * 1024 + (l16 % 2) * 8 + ((c1 ^ f(t)) << 4)] ^ (32 (om % 8)) + 256 (om / 8) + 1024 (32 tb [+ 16])
  // A stage base is a multiple of 1024 and so commutes with the XORs.
  const uint32_t qk_base = l16 * 1024 + ((q4 ^ swz(l16)) << 4);
  const uint32_t rp_base = l16 * 128 + ((q4 ^ swz_rope(l16)) << 4);
  uint32_t pv_base;
  {
    const int t = 4 * q4 + (l16 >> 2);
    pv_base = t * 1024 + (l16 & 1) * 8 + (((((l16 & 3) >> 1)) ^ swz(t)) << 4);
  }

  f32x4 acc[R / 16];
#pragma unroll
  for (int om = 0; om < R / 16; ++om) acc[om] = f32x4{};
  float m_run = -INFINITY;  // running max of the unscaled logits of this lane's head
  float l_run = 0.f;        // this lane's share of the softmax denominator
  const float c2 = scale * kLog2e;  // logits -> log2 units

  if (n_st > 0) issue(0);
  if (n_st > 1) issue(1);

  for (int s = 0; s < n_st; ++s) {
    if (s + 1 < n_st) {
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");  // the next page's 10 loads may fly
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    const uint32_t stage_off = (s & 1) * STAGE_BYTES;
    const LDS_AS uint8_t* lds0 = (LDS_AS uint8_t*)smem;
    const LDS_AS float* st_alpha = (const LDS_AS float*)(lds0 + stage_off + CONTENT_BYTES + ROPE_BYTES);
    const uint32_t qk_b = qk_base + stage_off;
    const uint32_t rp_b = rp_base + stage_off + CONTENT_BYTES;
    const uint32_t pv_b = pv_base + stage_off;
    const int tok0 = lo + s * PAGE;
    const bool page_ok = page_of(s) >= 0;
    if (!page_ok) err = 1;
    // rows r of this page with r < lim are visible to this wave
    const int lim = page_ok ? hi_w - tok0 : 0;

    if (wave_active) {
      // ---- QK for the 64 tokens of the page: four 16-token tiles ----
      f32x4 sc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
      for (int kk = 0; kk < R / 32; ++kk) {
        const uint32_t a_off = (qk_b ^ (64u * (kk & 3))) + 256 * (kk >> 2);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const bf16x8 a = lds_read16(lds0 + a_off + 1024 * 16 * tt);
          sc[tt] = mfma(a, qb[kk], sc[tt]);
        }
      }
      if (USE_ALPHA) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int t = 16 * tt + 4 * q4;  // rows of the four registers
#pragma unroll
          for (int j = 0; j < 4; ++j) sc[tt][j] *= aq * st_alpha[(t + j) * groups + g];
        }
      }
#pragma unroll
      for (int kk = 0; kk < DR / 32; ++kk) {
        const uint32_t a_off = rp_b ^ (64u * kk);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const bf16x8 a = lds_read16(lds0 + a_off + 128 * 16 * tt);
          sc[tt] = mfma(a, qrb[kk], sc[tt]);
        }
      }
      // ---- mask rows past the visible end (tail page, causal window, bad page)
      if (lim < PAGE) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (16 * tt + 4 * q4 + j >= lim) sc[tt][j] = -INFINITY;
      }
      // ---- online softmax over the page; the running sums are rescaled by a
      // per-head factor (1 unless the maximum grew by more than the threshold)
      float mx = sc[0][0];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[tt][j]);
      mx = head_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const bool grow = (m_new - m_run) * c2 > kRescaleThreshold;  // false when both -inf
      float f = 1.f;
      if (grow) {
        f = (m_new == -INFINITY) ? 1.f : exp2f((m_run - m_new) * c2);
        m_run = m_new;
      }
#pragma unroll
      for (int om = 0; om < R / 16; ++om)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[om][j] *= f;
      l_run *= f;
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c2;
      bf16x8 pb[2];  // P^T of tokens 32 tb .. +31: elements 0-3 tile 2 tb, 4-7 tile 2 tb + 1
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const __bf16 pr = static_cast<__bf16>(exp2f(fmaf(sc[tt][j], c2, -mc)));
          pb[tt >> 1][4 * (tt & 1) + j] = pr;
          l_run += static_cast<float>(pr);
        }
      // ---- PV: O^T[512 x 16] += C^T[512 x 64 tok] . P^T, two 32-token steps ----
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int om = 0; om < R / 16; ++om) {
          const uint32_t a_off = (pv_b ^ (32u * (om & 7))) + 256 * (om >> 3) + 1024 * 32 * tb;
          const bf16x4 lo4 = lds_read_tr(lds0 + a_off);
          const bf16x4 hi4 = lds_read_tr(lds0 + a_off + 16 * 1024);
          const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[om] = mfma(a, pb[tb], acc[om]);
        }
      }
    }
    __syncthreads();
    if (s + 2 < n_st) issue(s + 2);
  }

  // ---- epilogue: o_p = acc / l, lse_p = scale * m + ln l ----
  if (wave_active) {
    const float l_tot = head_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* out = o_part + (my_row * num_splits + p) * R;
#pragma unroll
    for (int om = 0; om < R / 16; ++om) {
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = acc[om][j] * inv;
      *reinterpret_cast<f32x4*>(out + om * 16 + q4 * 4) = v;
    }
    if (q4 == 0) {
      lse_part[my_row * num_splits + p] =
          l_tot > 0.f ? m_run * scale + log2f(l_tot) * kLn2 : -INFINITY;
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
