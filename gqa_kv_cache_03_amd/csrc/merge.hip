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
//
// One 256-thread workgroup per output row (b, t, h). A split's D partial values are
// read by D/4 lanes with 16-byte loads; the workgroup walks 4 * (256 / D) splits per
// round, several rounds in flight per lane, and reduces across waves through LDS.

#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;

typedef __attribute__((ext_vector_type(4))) float f32x4;

template <typename TT> __device__ __forceinline__ void put4(TT* dst, f32x4 v);
template <> __device__ __forceinline__ void put4<float>(float* dst, f32x4 v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}
template <> __device__ __forceinline__ void put4<__bf16>(__bf16* dst, f32x4 v) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (__bf16)v[i];
  *reinterpret_cast<bf16x4*>(dst) = o;
}

template <typename TT, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams p) {
  constexpr int LPS = D / 4;                 // lanes per split row
  constexpr int SPR = kThreads / LPS;        // splits per round (whole workgroup)
  constexpr int U = 4;                       // rounds in flight per lane
  __shared__ float red_m[kThreads / 64];
  __shared__ f32x4 red_o[SPR][LPS];
  __shared__ float red_w[SPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = blockIdx.x;
  const int b = row / (p.q_len * p.H);
  int L = p.seq_lens[b];
  L = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  int ns = (L + p.chunk - 1) / p.chunk;
  ns = ns > p.max_splits ? p.max_splits : ns;

  const float* lse = p.ws_lse + (size_t)row * p.max_splits;
  const float* po = p.ws_o + (size_t)row * p.max_splits * D;

  // M = max over the row's splits
  float M = kNegInf;
  for (int s = tid; s < ns; s += kThreads) M = fmaxf(M, lse[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const float Mu = (M == kNegInf) ? 0.f : M;

  // this thread: split slot sl = tid / LPS of every round, columns 4 * (tid % LPS)
  const int sl = tid / LPS;
  const int c = (tid % LPS) * 4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += SPR * U) {
    f32x4 v[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SPR + sl;
      if (s < ns) {
        w[u] = __builtin_amdgcn_exp2f(lse[s] - Mu);
        v[u] = *reinterpret_cast<const f32x4*>(po + (size_t)s * D + c);
      } else {
        w[u] = 0.f;
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc += w[u] * v[u];
      wsum += w[u];
    }
  }
  red_o[sl][tid % LPS] = acc;
  if (tid % LPS == 0) red_w[sl] = wsum;
  __syncthreads();
  if (tid < LPS) {
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    float wt = 0.f;
#pragma unroll
    for (int k = 0; k < SPR; ++k) {
      tot += red_o[k][tid];
      wt += red_w[k];
    }
    const float inv = (wt > 0.f) ? 1.f / wt : 0.f;
    put4<TT>(static_cast<TT*>(p.out) + (size_t)row * D + tid * 4, tot * inv);
  }
}

template <typename TT, int D>
hipError_t go(const DecodeParams& p, hipStream_t stream) {
  const int total = p.B * p.q_len * p.H;
  hipLaunchKernelGGL((merge_kernel<TT, D>), dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeParams& p, int dtype, int d_h, hipStream_t stream) {
  if (dtype == 0) return d_h == 64 ? go<float, 64>(p, stream) : go<float, 128>(p, stream);
  return d_h == 64 ? go<__bf16, 64>(p, stream) : go<__bf16, 128>(p, stream);
}

}  // namespace gqa
