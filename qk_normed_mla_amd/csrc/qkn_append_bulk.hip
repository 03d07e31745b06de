// alpha^k of many new tokens at once (a prompt's worth, or a whole history):
// for every token and KV group, alpha^k_{t,g} = 1/RMS(c_t W^K_g) with c_t the
// latent as stored (QK-Normed MLA summary, "Metodologia" items 2-3).  For a few
// tokens per call the append kernel forms each key in one block; for thousands
// the keys K = C W^K_g are a matrix product, done here on the matrix cores.
//
// One block of 8 waves per 256 tokens and KV group; wave w owns tokens
// 32 w .. 32 w + 31 of the block (the A rows) and all d / 32 column tiles of
// their keys (v_mfma_f32_32x32x16_bf16).  A is the stored latent itself: the
// bf16 words of c_t are exact operands.  W^K_g passes through LDS in chunks of
// up to 8192 values (16-byte loads), each value split into three bf16 words
// w = hi + mid + lo (24 significant bits: the split is exact up to the last
// rounding, |e| <= 2^-24 |w|); a step takes c.hi + c.mid + c.lo, so every
// product is exact and the key is a float32 sum, as accurate as the append
// kernel's own.  W is read with ds_read_b64_tr_b16 (one column over four rows
// per lane), which sets the order of the reduction index within a step; the
// latent operand is loaded in the same order.  The next chunk of W and of the
// latents is in flight while the current one is multiplied.  Then each token's
// sum of squares is added over its columns in a fixed order through LDS, and
// the token's alpha^k goes to its cache slot (tokens whose slot is invalid are
// skipped: the store kernel flags them).
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

#define LDS_AS __attribute__((address_space(3)))
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int WAVES = 8;
constexpr int TOK = 32 * WAVES;    // tokens per block
constexpr int WCHUNK = 8192;       // W^K_g values per staged chunk
constexpr int W_PAD = 16;          // bf16 of padding per staged row
constexpr int KC_MAX = 128;        // W^K_g rows per chunk (at most 8 steps of latents in registers)
constexpr int chunk_rows(int d) { return WCHUNK / d < KC_MAX ? WCHUNK / d : KC_MAX; }

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

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(const_cast<__bf16*>(p)));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// NT = d / 32 column tiles; KC = min(8192 / d, 128) rows of W^K_g per chunk
template <int NT>
__global__ __launch_bounds__(64 * WAVES) void append_alpha_mfma(
    const float* __restrict__ c_new, const int32_t* __restrict__ seq_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_table,
    const float* __restrict__ w_k, float* __restrict__ alpha_k, int n_tokens, int batch,
    int max_pages, int num_pages, int rank, int groups, float eps) {
  constexpr int D = NT * 32;
  constexpr int KC = chunk_rows(D);
  constexpr int PER = KC * D / 4 / (64 * WAVES);  // float4 of a chunk per thread
  constexpr int SPC = KC / 16;  // steps per chunk
  constexpr int WROW = D + W_PAD;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __bf16* W0 = reinterpret_cast<__bf16*>(smem);
  __bf16* W1 = W0 + KC * WROW;
  __bf16* W2 = W1 + KC * WROW;
  float* red = reinterpret_cast<float*>(smem + 3 * KC * WROW * 2);  // [WAVES][32][32]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int l16 = lane & 15, G = (lane >> 4) & 1;
  const int g = blockIdx.y;
  const int t = blockIdx.x * TOK + 32 * wave + l32;  // token of this lane's A row
  const bool tok_ok = t < n_tokens;
  const float* crow = c_new + (size_t)(tok_ok ? t : 0) * rank;
  const float* wg = w_k + (size_t)g * rank * D;

  // the next chunk: W^K_g rows k0 .. k0 + KC - 1, and this lane's latents of
  // its SPC steps, in the order of the transposed read (4 hh + 0..3, 8 + 4 hh + 0..3)
  float4 wv[PER];
  float4 av[SPC][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * 64 * WAVES;
      wv[u] = *reinterpret_cast<const float4*>(wg + (size_t)(k0 + e / (D / 4)) * D + 4 * (e % (D / 4)));
    }
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
      const float* ap = crow + k0 + 16 * st + 4 * hh;
      av[st][0] = tok_ok ? *reinterpret_cast<const float4*>(ap) : make_float4(0.f, 0.f, 0.f, 0.f);
      av[st][1] = tok_ok ? *reinterpret_cast<const float4*>(ap + 8) : make_float4(0.f, 0.f, 0.f, 0.f);
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
      const int e = tid + u * 64 * WAVES;
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
      const f32x8 x = {av[st][0].x, av[st][0].y, av[st][0].z, av[st][0].w,
                       av[st][1].x, av[st][1].y, av[st][1].z, av[st][1].w};
      a[st] = __builtin_convertvector(x, bf16x8);  // the stored words of c_t
    }
    if (k0 + KC < rank) load(k0 + KC);  // in flight during this chunk's products
    __syncthreads();
#pragma unroll
    for (int st = 0; st < SPC; ++st) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int off = tr_off + 16 * st * WROW + 32 * ct;
        const bf16x8 b0 = __builtin_shufflevector(lds_read_tr(W0 + off), lds_read_tr(W0 + off + 8 * WROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b1 = __builtin_shufflevector(lds_read_tr(W1 + off), lds_read_tr(W1 + off + 8 * WROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b2 = __builtin_shufflevector(lds_read_tr(W2 + off), lds_read_tr(W2 + off + 8 * WROW),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        acc[ct] = mfma(a[st], b0, acc[ct]);
        acc[ct] = mfma(a[st], b1, acc[ct]);
        acc[ct] = mfma(a[st], b2, acc[ct]);
      }
    }
  }

  // sum of squares per token: lane holds tokens m = r % 4 + 8 (r / 4) + 4 hh
  // (r < 16) of the wave, column 32 ct + l32; columns of a tile in lane order
  float* rw = red + wave * 32 * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float q = 0.f;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) q = fmaf(acc[ct][r], acc[ct][r], q);
    rw[((r & 3) + 8 * (r >> 2) + 4 * hh) * 32 + l32] = q;
  }
  __syncthreads();
  if (hh == 0 && tok_ok) {
    float ss = 0.f;
    for (int x = 0; x < 32; ++x) ss += rw[l32 * 32 + x];
    const int b = seq_idx[t], p = pos[t];
    if (b >= 0 && b < batch && p >= 0 && p < max_pages * QKN_MLA_PAGE_SIZE) {
      const int page = block_table[(size_t)b * max_pages + p / QKN_MLA_PAGE_SIZE];
      if (page >= 0 && page < num_pages) {
        const size_t slot = (size_t)page * QKN_MLA_PAGE_SIZE + p % QKN_MLA_PAGE_SIZE;
        alpha_k[slot * groups + g] = 1.0f / sqrtf(ss / (float)D + eps);
      }
    }
  }
}

template <int NT>
hipError_t launch_nt(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                     const int32_t* seq_idx, const int32_t* pos, const int32_t* block_table,
                     const float* w_k, float* alpha_k, hipStream_t s) {
  constexpr int D = NT * 32;
  constexpr int KC = chunk_rows(D);
  const size_t lds = (size_t)3 * KC * (D + W_PAD) * 2 + WAVES * 32 * 32 * 4;
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&append_alpha_mfma<NT>),
                                          (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_alpha_mfma<NT>, dim3(cdiv(n_tokens, TOK), d.groups), dim3(64 * WAVES),
                     lds, s, c_new, seq_idx, pos, block_table, w_k, alpha_k, n_tokens, d.batch,
                     d.max_pages_per_seq, d.num_pages, d.rank, d.groups, d.eps);
  return hipGetLastError();
}

}  // namespace

bool append_bulk_applies(const qkn_mla_dims& d) {
  const int dv = d.head_dim;
  return d.cache_dtype == QKN_BF16 && (dv == 32 || dv == 64 || dv == 128 || dv == 256) &&
         d.rank % chunk_rows(dv) == 0;
}

hipError_t launch_append_alpha_bulk(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                                    const int32_t* seq_idx, const int32_t* pos,
                                    const int32_t* block_table, const float* w_k, float* alpha_k,
                                    hipStream_t s) {
  switch (d.head_dim) {
    case 32: return launch_nt<1>(d, n_tokens, c_new, seq_idx, pos, block_table, w_k, alpha_k, s);
    case 64: return launch_nt<2>(d, n_tokens, c_new, seq_idx, pos, block_table, w_k, alpha_k, s);
    case 128: return launch_nt<4>(d, n_tokens, c_new, seq_idx, pos, block_table, w_k, alpha_k, s);
    case 256: return launch_nt<8>(d, n_tokens, c_new, seq_idx, pos, block_table, w_k, alpha_k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qkn
