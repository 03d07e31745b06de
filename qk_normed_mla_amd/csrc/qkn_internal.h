// Internal declarations shared by the HIP translation units of libqknmla.so.
// Not part of the public interface (include/qkn_mla.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// RoPE on the RMS-normed RoPE block (NeoX halves).  The angle pos * freq is
// formed and reduced in double precision: at positions of 2^18 a float angle
// would already be off by ~1e-2 rad.
// ----------------------------------------------------------------------------
__device__ __forceinline__ void rope_cos_sin(int pos, int j, int rope_dim, float theta,
                                             float* c, float* s) {
  double inv_freq = pow((double)theta, -2.0 * (double)j / (double)rope_dim);
  double ang = (double)pos * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// ----------------------------------------------------------------------------
// wave-level reductions (64 lanes)
// ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

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

struct DecodeArgs {
  const void* q_tilde;
  const float* alpha_q;
  const void* q_rope;
  const void* kv;
  const float* alpha_k;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* o_part;
  float* lse_part;
  int32_t* err_flag;
  int num_splits;
  bool use_alpha;
};

hipError_t launch_decode_generic(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s);
bool mfma_decode_supported(const qkn_mla_dims& d);
hipError_t launch_decode_mfma(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s);

hipError_t launch_combine(const qkn_mla_dims& d, int num_splits, const float* o_part,
                          const float* lse_part, float* o_lat, float* lse, hipStream_t s);

}  // namespace qkn
