// Internal declarations shared by the HIP translation units of libqknmla.so.
// Not part of the public interface (include/qkn_mla.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qkn_mla.h"

namespace qkn {

// ----------------------------------------------------------------------------
// bfloat16 storage words
// ----------------------------------------------------------------------------

// float -> bfloat16 word, round to nearest even (gfx950 has a native convert).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t w) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(w) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(uint16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// ----------------------------------------------------------------------------
// RoPE on the RMS-normed RoPE block (NeoX halves): the angle pos * omega_j,
// omega_j = theta^(-2 j / d_R), is formed and reduced in double precision (at
// positions of 2^18 a float angle would already be off by ~1e-2 rad).  The
// cosine and sine of the reduced angle |r| <= pi are taken in double when the
// result is stored in float32 (PRECISE), else in float (sincosf on r rounded
// to float: ~3e-7 absolute, far below the bf16 step of the stored key or
// query, at a small fraction of the double routine's cost).  omega_j is w^j with w = theta^(-2/d_R),
// raised by repeated squaring (at most 8 double products for j < 256; the
// relative error stays ~1e-14), and the reduction subtracts k * 2 pi with 2 pi
// in two double parts, which leaves the reduced angle good to ~1e-15 rad.
// ----------------------------------------------------------------------------
__device__ __forceinline__ double rope_omega(int j, int rope_dim, float theta) {
  const double w = exp2(-2.0 / (double)rope_dim * log2((double)theta));
  double omega = 1.0, b = w;
  for (int e = j; e != 0; e >>= 1) {
    if (e & 1) omega *= b;
    b *= b;
  }
  return omega;
}

template <bool PRECISE>
__device__ __forceinline__ void rope_cos_sin_at(int pos, double omega, float* c, float* s) {
  const double ang = (double)pos * omega;
  const double k = rint(ang * 0.15915494309189533577);          // ang / (2 pi)
  const double r = fma(-k, 2.44929359829470635445e-16, fma(-k, 6.28318530717958623200, ang));
  if constexpr (PRECISE) {
    double sd, cd;
    sincos(r, &sd, &cd);  // |r| <= pi: the short path
    *c = static_cast<float>(cd);
    *s = static_cast<float>(sd);
  } else {
    sincosf(static_cast<float>(r), s, c);
  }
}

template <bool PRECISE>
__device__ __forceinline__ void rope_cos_sin(int pos, int j, int rope_dim, float theta,
                                             float* c, float* s) {
  rope_cos_sin_at<PRECISE>(pos, rope_omega(j, rope_dim, theta), c, s);
}

// ----------------------------------------------------------------------------
// wave-level reductions (64 lanes), all in registers: DPP lane permutations
// within rows of 16 (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror), then v_permlane16_swap and v_permlane32_swap across rows.  Each
// step combines a lane with one partner by a commutative operation, so every
// lane ends with the same bits.
// ----------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_partner<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, dpp_partner<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = op(v, dpp_partner<0x141>(v));  // row_half_mirror: the other quad of 8
  v = op(v, dpp_partner<0x140>(v));  // row_mirror: the other half of 16
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));  // rows 2k and 2k + 1
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));  // the two halves
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Raises the dynamic LDS limit of kernel `fn` to `bytes` on the current device,
// once per (kernel, device).  Safe to call from several host threads at once.
hipError_t set_lds_limit_once(const void* fn, int bytes);

// Tokens per split-KV partition: ceil(T / P) rounded up to whole 64-token pages.
__host__ __device__ __forceinline__ int split_len(int T, int P) {
  return QKN_MLA_PAGE_SIZE * cdiv(cdiv(T, P), QKN_MLA_PAGE_SIZE);
}

// ----------------------------------------------------------------------------
// launchers (defined in the kernel translation units)
// ----------------------------------------------------------------------------
hipError_t launch_absorb_query(const qkn_mla_dims& d, const float* q, const float* q_rope,
                               const int32_t* q_pos, const float* w_k, const float* gamma_q,
                               const float* gamma_k, const float* gamma_qr, void* q_tilde,
                               float* alpha_q, void* q_rope_normed, hipStream_t s);

hipError_t launch_append(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                         const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                         const int32_t* block_table, const float* w_k, const float* gamma_kr,
                         void* kv_cache, float* alpha_k_cache, int32_t* err_flag, hipStream_t s);

// From this many tokens in one call the append takes the bulk route.
constexpr int kBulkMinTokens = 4096;

// Element type of the split-KV partials for a cache of element type CacheT:
// half for a bf16 cache (stored as uint16_t words), float32 for a float32 one.
template <typename CacheT>
struct PartialDtype {
  using type = float;
};
template <>
struct PartialDtype<uint16_t> {
  using type = _Float16;
};
template <typename CacheT>
using PartialOf = typename PartialDtype<CacheT>::type;

struct DecodeArgs {
  const void* q_tilde;
  const float* alpha_q;
  const void* q_rope;
  const void* kv;
  const float* alpha_k;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o_part;  // partial dtype: half for a bf16 cache, float32 for a float32 cache
  float* lse_part;
  int32_t* err_flag;
  int num_splits;
  bool use_alpha;
  const int32_t* sel = nullptr;  // selected-token decode: [B, s_q, sel_len] positions
  int sel_len = 0;
};

hipError_t launch_decode_generic(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s);
bool mfma_decode_supported(const qkn_mla_dims& d);
hipError_t launch_decode_mfma(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s);
// Selected-token decode on the matrix cores: 0 when it takes these dims, list
// length and split count, -1 for a bad argument, -2 for unsupported dims
// (heads not a multiple of 128, a cache of 4 GiB or more, or more than 2048
// list entries per split).
int sparse_decode_check(const qkn_mla_dims& d, int sel_len, int num_splits);

// Chunked prefill on the explicit path (bf16 cache, r = 512, d = 128, d_R = 64,
// a multiple of 32 heads per group).
bool prefill_supported(const qkn_mla_dims& d);
hipError_t launch_prefill_query(const qkn_mla_dims& d, const float* q, const float* q_rope,
                                const int32_t* q_pos, const float* gamma_q, const float* gamma_qr,
                                void* q_hat, void* q_rope_normed, hipStream_t s);
hipError_t launch_prefill_expand(const qkn_mla_dims& d, const void* kv, const float* alpha_k,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const float* w_k, const float* w_v, const float* gamma_k,
                                 void* k_hat, void* v, int32_t* err_flag, hipStream_t s);
hipError_t launch_prefill_attend(const qkn_mla_dims& d, const void* q_hat, const void* q_rope_normed,
                                 const void* k_hat, const void* v, const void* kv,
                                 const int32_t* block_table, const int32_t* seq_lens, float* o,
                                 float* lse, int32_t* err_flag, hipStream_t s);
hipError_t launch_decode_sparse(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s);

// The GQA path (bf16 cache, d = 128, d_R = 64, r a multiple of 16, a multiple
// of 32 heads per group): a paged cache of gqa_row_words(d) 16-bit words per
// token.  With num_splits > 1 the attend writes half partials [rows, P, d]
// and lse partials [rows, P] and merges them into o, lse.
bool gqa_supported(const qkn_mla_dims& d);
int gqa_row_words(const qkn_mla_dims& d);
hipError_t launch_gqa_append(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                             const float* k_rope_new, const int32_t* seq_idx, const int32_t* pos,
                             const int32_t* block_table, const float* w_k, const float* w_v,
                             const float* gamma_k, const float* gamma_kr, void* kvg,
                             int32_t* err_flag, hipStream_t s);
hipError_t launch_gqa_attend(const qkn_mla_dims& d, const void* q_hat, const void* q_rope_normed,
                             const void* kvg, const int32_t* block_table, const int32_t* seq_lens,
                             int num_splits, void* o_part, float* lse_part, float* o, float* lse,
                             int32_t* err_flag, hipStream_t s);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_combine(const qkn_mla_dims& d, int num_splits, const void* o_part,
                          const float* lse_part, float* o_lat, float* lse, hipStream_t s);
// The same merge for n_rows rows of row_len (a multiple of 8) entries, the
// partials half (half_parts) or float32.
hipError_t launch_combine_rows(int n_rows, int num_splits, int row_len, bool half_parts,
                               const void* o_part, const float* lse_part, float* o, float* lse,
                               hipStream_t s);
bool append_bulk_applies(const qkn_mla_dims& d);
hipError_t launch_append_alpha_bulk(const qkn_mla_dims& d, int32_t n_tokens, const float* c_new,
                                    const int32_t* seq_idx, const int32_t* pos,
                                    const int32_t* block_table, const float* w_k, float* alpha_k,
                                    hipStream_t s);
bool project_mfma_applies(const qkn_mla_dims& d);
// Device address of the library's static scratch array on the current device
// (QKN_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned).
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_combine_project(const qkn_mla_dims& d, int num_splits, const void* o_part,
                                  const float* lse_part, const float* w_v, float* o_lat,
                                  float* lse, float* o, uint32_t flags, hipStream_t s);

}  // namespace qkn
