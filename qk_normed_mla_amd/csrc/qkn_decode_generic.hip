// Generic split-KV decode on the vector ALUs, float32 arithmetic throughout
// (the partials are stored in the partial dtype: half for a bf16 cache).
// It serves the float32 cache and any size the matrix-core kernel does not
// take (few heads, other ranks); it is also a second, independent GPU
// implementation the matrix-core kernel is tested against.
//
// Per query row (b, i, h) and split p, over the visible tokens of the split
// (QK-Normed MLA summary, "Metodologia", decode-logit equation):
//   l_t = scale * ((q~ . c_t) alpha^q alpha^k_{t,g(h)} + q^R . k^R_t)
// followed by an online softmax and the latent-space accumulation sum_t p_t c_t.
//
// Block: 256 threads = (b, i, split, 8 heads).  Tokens are staged 16 at a time
// in LDS as float; two threads share each (head, token) dot product.
#include <math.h>

#include "qkn_internal.h"

namespace qkn {
namespace {

constexpr int HB = 8;    // heads per block
constexpr int TC = 16;   // tokens per staged chunk
constexpr int kMaxAccPerThread = 4;  // rank <= 1024 = 4 * 256 threads

template <typename CacheT>
__global__ __launch_bounds__(256) void decode_generic(
    const CacheT* __restrict__ q_tilde, const float* __restrict__ alpha_q,
    const CacheT* __restrict__ q_rope, const CacheT* __restrict__ kv,
    const float* __restrict__ alpha_k, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, PartialOf<CacheT>* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ err_flag, int s_q, int heads,
    int groups, int rank, int rope_dim, int max_pages, int num_pages, int num_splits,
    float scale, int use_alpha) {
  extern __shared__ float smem[];
  float* qs = smem;                          // [HB][rank]     q~ of the block's heads
  float* qrs = qs + HB * rank;               // [HB][rope_dim] normed RoPE queries
  float* cs = qrs + HB * rope_dim;           // [TC][rank]     staged latents
  float* krs = cs + TC * rank;               // [TC][rope_dim] staged RoPE keys
  __shared__ float aqs[HB];                  // alpha^q per head
  __shared__ float aks[TC][HB];              // alpha^k of each token for each head's group
  __shared__ float lg[HB][TC];               // logits, then probabilities
  __shared__ float fac[HB];                  // rescale factor of the running sums
  __shared__ int slot[TC];                   // cache row of each staged token + 1, 0 = none

  const int tid = threadIdx.x;
  const int h0 = blockIdx.x * HB;
  const int p = blockIdx.y;
  const int bi = blockIdx.z;            // b * s_q + i
  const int b = bi / s_q, i = bi % s_q;
  const int nh = min(HB, heads - h0);
  const int hpg = heads / groups;
  const int row_stride = rank + rope_dim;

  int T = seq_lens[b];
  if (T > max_pages * QKN_MLA_PAGE_SIZE || T < 0) {
    if (err_flag && tid == 0 && p == 0 && blockIdx.x == 0 && i == 0) atomicOr(err_flag, QKN_FLAG_INDEX);
    T = min(max(T, 0), max_pages * QKN_MLA_PAGE_SIZE);
  }
  const int n_vis = T - s_q + i + 1;  // tokens this query may see
  const int L = split_len(max(T, 1), num_splits);
  const int lo = p * L;
  const int hi = min(min((p + 1) * L, T), n_vis);

  for (int e = tid; e < HB * rank; e += 256) {
    int h = e / rank, m = e % rank;
    qs[e] = h < nh ? Elem<CacheT>::load(q_tilde, ((size_t)bi * heads + h0 + h) * rank + m) : 0.f;
  }
  for (int e = tid; e < HB * rope_dim; e += 256) {
    int h = e / rope_dim, j = e % rope_dim;
    qrs[e] = h < nh ? Elem<CacheT>::load(q_rope, ((size_t)bi * heads + h0 + h) * rope_dim + j) : 0.f;
  }
  if (tid < HB) aqs[tid] = (tid < nh && use_alpha) ? alpha_q[(size_t)bi * heads + h0 + tid] : 1.f;

  float m_run = -INFINITY, l_run = 0.f;  // running max / sum, kept by threads tid < HB
  float acc[HB][kMaxAccPerThread];
#pragma unroll
  for (int h = 0; h < HB; ++h)
#pragma unroll
    for (int k = 0; k < kMaxAccPerThread; ++k) acc[h][k] = 0.f;

  for (int t0 = lo; t0 < hi; t0 += TC) {
    __syncthreads();  // previous chunk fully consumed
    if (tid < TC) {
      int t = t0 + tid, sr = 0;
      if (t < hi) {
        int page = block_table[(size_t)b * max_pages + t / QKN_MLA_PAGE_SIZE];
        if (page >= 0 && page < num_pages)
          sr = page * QKN_MLA_PAGE_SIZE + t % QKN_MLA_PAGE_SIZE + 1;
        else if (err_flag)
          atomicOr(err_flag, QKN_FLAG_INDEX);
      }
      slot[tid] = sr;
    }
    __syncthreads();
    for (int e = tid; e < TC * row_stride; e += 256) {
      int t = e / row_stride, m = e % row_stride;
      int sr = slot[t] - 1;
      float v = sr >= 0 ? Elem<CacheT>::load(kv, (size_t)sr * row_stride + m) : 0.f;
      if (m < rank) cs[t * rank + m] = v;
      else krs[t * rope_dim + (m - rank)] = v;
    }
    for (int e = tid; e < TC * HB; e += 256) {
      int t = e / HB, h = e % HB;
      int sr = slot[t] - 1;
      int g = min(h0 + h, heads - 1) / hpg;
      aks[t][h] = (sr >= 0 && use_alpha) ? alpha_k[(size_t)sr * groups + g] : 1.f;
    }
    __syncthreads();
    {  // logits: threads 2k and 2k+1 split the dot products of pair k = (head, token)
      const int pair = tid >> 1, half = tid & 1;
      const int h = pair / TC, t = pair % TC;
      const int mh = rank / 2, jh = rope_dim / 2;
      float dc = 0.f, dr = 0.f;
      for (int m = half * mh; m < (half + 1) * mh; ++m) dc = fmaf(qs[h * rank + m], cs[t * rank + m], dc);
      for (int j = half * jh; j < (half + 1) * jh; ++j)
        dr = fmaf(qrs[h * rope_dim + j], krs[t * rope_dim + j], dr);
      dc += __shfl_xor(dc, 1, 64);
      dr += __shfl_xor(dr, 1, 64);
      if (half == 0) {
        float l = -INFINITY;
        if (h < nh && slot[t] > 0) l = scale * (dc * aqs[h] * aks[t][h] + dr);
        lg[h][t] = l;
      }
    }
    __syncthreads();
    if (tid < HB) {  // online softmax, one thread per head
      const int h = tid;
      float mx = m_run;
      for (int t = 0; t < TC; ++t) mx = fmaxf(mx, lg[h][t]);
      float f = 1.f, sum = 0.f;
      if (mx != -INFINITY) {
        f = (m_run == -INFINITY) ? 0.f : expf(m_run - mx);
        for (int t = 0; t < TC; ++t) {
          float pt = lg[h][t] == -INFINITY ? 0.f : expf(lg[h][t] - mx);
          lg[h][t] = pt;
          sum += pt;
        }
        m_run = mx;
      } else {
        for (int t = 0; t < TC; ++t) lg[h][t] = 0.f;
      }
      l_run = l_run * f + sum;
      fac[h] = f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxAccPerThread; ++k) {
      const int m = tid + 256 * k;
      if (m >= rank) break;
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        float a = acc[h][k] * fac[h];
        for (int t = 0; t < TC; ++t) a = fmaf(lg[h][t], cs[t * rank + m], a);
        acc[h][k] = a;
      }
    }
  }
  __syncthreads();
  if (tid < HB) {  // publish 1/l and lse of each head
    fac[tid] = l_run > 0.f ? 1.f / l_run : 0.f;
    if (tid < nh) {
      size_t row = (size_t)bi * heads + h0 + tid;
      lse_part[row * num_splits + p] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
    }
  }
  __syncthreads();
  bool out_of_range = false;  // a half partial rounded to +-inf
#pragma unroll
  for (int k = 0; k < kMaxAccPerThread; ++k) {
    const int m = tid + 256 * k;
    if (m >= rank) break;
    for (int h = 0; h < nh; ++h) {
      size_t row = (size_t)bi * heads + h0 + h;
      const auto v = static_cast<PartialOf<CacheT>>(acc[h][k] * fac[h]);
      if constexpr (sizeof(v) == 2) out_of_range |= __builtin_isinf(static_cast<float>(v));
      o_part[(row * num_splits + p) * rank + m] = v;
    }
  }
  if (out_of_range && err_flag) atomicOr(err_flag, QKN_FLAG_PARTIAL_RANGE);
}

template <typename CacheT>
hipError_t launch_typed(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s) {
  const size_t shmem = (size_t)(HB + TC) * (d.rank + d.rope_dim) * sizeof(float);
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&decode_generic<CacheT>),
                                          128 * 1024);
  if (e != hipSuccess) return e;
  dim3 grid(cdiv(d.heads, HB), a.num_splits, d.batch * d.s_q);
  hipLaunchKernelGGL(decode_generic<CacheT>, grid, dim3(256), shmem, s,
                     static_cast<const CacheT*>(a.q_tilde), a.alpha_q,
                     static_cast<const CacheT*>(a.q_rope), static_cast<const CacheT*>(a.kv),
                     a.alpha_k, a.block_table, a.seq_lens,
                     static_cast<PartialOf<CacheT>*>(a.o_part), a.lse_part, a.err_flag,
                     d.s_q, d.heads, d.groups, d.rank, d.rope_dim, d.max_pages_per_seq,
                     d.num_pages, a.num_splits, d.softmax_scale, a.use_alpha ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_generic(const qkn_mla_dims& d, const DecodeArgs& a, hipStream_t s) {
  if (d.cache_dtype == QKN_BF16) return launch_typed<uint16_t>(d, a, s);
  return launch_typed<float>(d, a, s);
}

}  // namespace qkn
