// Log-sum-exp merge of split-K partial results.
//
// Each split s of a query row holds O_s = softmax over its own keys times V
// (normalised) and lse_s = log2 of its softmax denominator (plus its running max).
// Because softmax over the union of the splits' keys reweights each split by its
// share of the total denominator, out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M)
// with M = max_s lse_s is exactly the attention output over all keys
// (softmax of the llms.blog GQA/MQA page, "Multi-Query Attention" > "Mathematical
// Formulation", evaluated piecewise). Splits past the sequence end were never
// written and are not read; empty splits carry lse = -inf and weigh nothing.

#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <typename TT> __device__ __forceinline__ void put(TT* dst, float v);
template <> __device__ __forceinline__ void put<float>(float* dst, float v) { *dst = v; }
template <> __device__ __forceinline__ void put<__bf16>(__bf16* dst, float v) { *dst = (__bf16)v; }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// One wave per output row (b, t, h); 4 rows per 256-thread workgroup.
template <typename TT, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p, int total_rows) {
  constexpr int PER_LANE = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int b = row / (p.q_len * p.H);
  int L = p.seq_lens[b];
  L = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  int ns = (L + p.chunk - 1) / p.chunk;
  ns = ns > p.max_splits ? p.max_splits : ns;

  const float* lse = p.ws_lse + (size_t)row * p.max_splits;
  const float* po = p.ws_o + (size_t)row * p.max_splits * D;

  float M = kNegInf;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, lse[s]);
  M = wave_max(M);
  const float Mu = (M == kNegInf) ? 0.f : M;

  float acc[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(lse[s] - Mu);
    wsum += w;
    const float* src = po + (size_t)s * D + lane * PER_LANE;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) acc[i] = fmaf(w, src[i], acc[i]);
  }
  const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
  TT* dst = static_cast<TT*>(p.out) + (size_t)row * D + lane * PER_LANE;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) put<TT>(dst + i, acc[i] * inv);
}

template <typename TT, int D>
hipError_t go(const DecodeParams& p, hipStream_t stream) {
  const int total = p.B * p.q_len * p.H;
  hipLaunchKernelGGL((merge_kernel<TT, D>), dim3((total + 3) / 4), dim3(256), 0, stream, p, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeParams& p, int dtype, int d_h, hipStream_t stream) {
  if (dtype == 0) return d_h == 64 ? go<float, 64>(p, stream) : go<float, 128>(p, stream);
  return d_h == 64 ? go<__bf16, 64>(p, stream) : go<__bf16, 128>(p, stream);
}

}  // namespace gqa
