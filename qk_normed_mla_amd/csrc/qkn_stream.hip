// qkn_mla_stream_read: a plain read-only stream over device memory, the
// achievable HBM read rate that the cache-reading kernels are set against
// besides the published peak.  Every 16-byte word is read once with
// non-temporal loads (as the decode reads the cache), four independent loads
// in flight per thread and iteration, consecutive lanes on consecutive words;
// the XOR of everything read goes into *sink, so no load can be dropped.
#include <algorithm>

#include "qkn_internal.h"

namespace qkn {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int STREAM_THREADS = 256;
// three blocks per CU: the fastest of a sweep over 256 .. 1536 blocks and 4,
// 8 or 16 loads in flight (2 GiB: 7.29 TB/s here against 5.97 at 2048 blocks)
constexpr int STREAM_BLOCKS = 768;

__global__ __launch_bounds__(STREAM_THREADS) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                     size_t n, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * STREAM_THREADS;
  size_t i = (size_t)blockIdx.x * STREAM_THREADS + threadIdx.x;
  u32x4 a = {0u, 0u, 0u, 0u}, b = a, c = a, d = a;
  for (; i + 3 * stride < n; i += 4 * stride) {
    a ^= __builtin_nontemporal_load(p + i);
    b ^= __builtin_nontemporal_load(p + i + stride);
    c ^= __builtin_nontemporal_load(p + i + 2 * stride);
    d ^= __builtin_nontemporal_load(p + i + 3 * stride);
  }
  for (; i < n; i += stride) a ^= __builtin_nontemporal_load(p + i);
  a ^= b ^ c ^ d;
  uint32_t v = a.x ^ a.y ^ a.z ^ a.w;
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v ^= __shfl_xor(v, k, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, v);
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>(STREAM_BLOCKS, (n + STREAM_THREADS - 1) / STREAM_THREADS);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(STREAM_THREADS), 0, s,
                     static_cast<const u32x4*>(src), n, sink);
  return hipGetLastError();
}

}  // namespace qkn
