// The projections around the latent attention of a GQLA layer's absorbed (MQA)
// execution (the thelatestinai page for 2604.07766, GQLA abstract).
//
// A group of query heads shares one pair of up-projections W_UK[g], W_UV[g]
// (d_h x d_c): its keys and values are W_UK[g] c_j and W_UV[g] c_j for the joint
// latent c_j of token j. Folding W_UK[g] into the query gives the same logits
// against the latent itself, q . (W_UK c_j) = (W_UK^T q) . c_j, and W_UV[g] can be
// applied after the weighted sum over tokens. So the step is
//   1. q_lat[h] = W_UK[g(h)]^T q[h]            (absorb_q_kernel, here)
//   2. u[h] = softmax(scale q_lat[h] . c_j) c   (the matrix-core decode kernel, with
//      the latent as a single KV head that is both K and V)
//   3. out[h] = W_UV[g(h)] u[h]                 (up_proj_kernel, here)
// Steps 1 and 3 are small (rows x d_h x d_c multiply-adds per step, with rows =
// B * q_len * H); step 2 streams the latent cache and dominates.

#include "gqa_internal.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kThreads = 256;
constexpr int kHeadChunk = 16;  // query heads of one group handled per workgroup
constexpr int kAbsorbCols = 64; // latent columns per absorb workgroup
constexpr int kUpCols = 16;     // output columns per up-projection workgroup

// Workgroup (row set, column chunk): rows = up to 16 heads of group g for token
// (b, t); each of the 256 lanes owns one latent column c and four of the heads.
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(LatentProjParams p) {
  __shared__ float qs[kHeadChunk][128 + 1];
  const int hpg = p.H / p.G;
  const int n_hc = (hpg + kHeadChunk - 1) / kHeadChunk;
  int x = blockIdx.x;
  const int hc = x % n_hc;
  x /= n_hc;
  const int g = x % p.G;
  const int bt = x / p.G;                       // b * q_len + t
  const int h0 = g * hpg + hc * kHeadChunk;
  const int nh = min(kHeadChunk, hpg - hc * kHeadChunk);
  const __bf16* q = static_cast<const __bf16*>(p.q);
  for (int e = threadIdx.x; e < nh * p.d_h; e += kThreads) {
    const int k = e / p.d_h, i = e - k * p.d_h;
    qs[k][i] = (float)q[((size_t)bt * p.H + h0 + k) * p.d_h + i];
  }
  __syncthreads();
  const int c = blockIdx.y * kAbsorbCols + (threadIdx.x % kAbsorbCols);
  const int kq = threadIdx.x / kAbsorbCols;    // heads kq, kq + 4, kq + 8, kq + 12
  const __bf16* w = static_cast<const __bf16*>(p.w_uk) + (size_t)g * p.d_h * p.d_c + c;
  float acc[kHeadChunk / 4] = {};
  for (int i = 0; i < p.d_h; ++i) {
    const float wv = (float)w[(size_t)i * p.d_c];
#pragma unroll
    for (int j = 0; j < kHeadChunk / 4; ++j) acc[j] = __builtin_fmaf(qs[kq + 4 * j][i], wv, acc[j]);
  }
  __bf16* dst = static_cast<__bf16*>(p.q_lat);
#pragma unroll
  for (int j = 0; j < kHeadChunk / 4; ++j) {
    const int k = kq + 4 * j;
    if (k < nh) dst[((size_t)bt * p.H + h0 + k) * p.d_c + c] = (__bf16)acc[j];
  }
}

// Workgroup (row set, output chunk): lane (k, i) of 16 x 16 computes output column
// i of head k as a dot product over the d_c latent columns, 8 at a time.
__global__ __launch_bounds__(kThreads) void up_proj_kernel(LatentProjParams p) {
  const int hpg = p.H / p.G;
  const int n_hc = (hpg + kHeadChunk - 1) / kHeadChunk;
  int x = blockIdx.x;
  const int hc = x % n_hc;
  x /= n_hc;
  const int g = x % p.G;
  const int bt = x / p.G;
  const int k = threadIdx.x / kUpCols;
  const int i = blockIdx.y * kUpCols + (threadIdx.x % kUpCols);
  if (hc * kHeadChunk + k >= hpg) return;
  const size_t row = (size_t)bt * p.H + g * hpg + hc * kHeadChunk + k;
  const float* u = p.u + row * p.d_c;
  const __bf16* w = static_cast<const __bf16*>(p.w_uv) + ((size_t)g * p.d_h + i) * p.d_c;
  float acc0 = 0.f, acc1 = 0.f;
  for (int c = 0; c < p.d_c; c += 8) {
    const bf16x8 wv = *reinterpret_cast<const bf16x8*>(w + c);
    const f32x4 u0 = *reinterpret_cast<const f32x4*>(u + c);
    const f32x4 u1 = *reinterpret_cast<const f32x4*>(u + c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc0 = __builtin_fmaf(u0[e], (float)wv[e], acc0);
      acc1 = __builtin_fmaf(u1[e], (float)wv[4 + e], acc1);
    }
  }
  static_cast<__bf16*>(p.out)[row * p.d_h + i] = (__bf16)(acc0 + acc1);
}

}  // namespace

hipError_t launch_latent_absorb_q(const LatentProjParams& p, hipStream_t stream) {
  const int n_hc = (p.H / p.G + kHeadChunk - 1) / kHeadChunk;
  const dim3 grid(p.B * p.q_len * p.G * n_hc, p.d_c / kAbsorbCols);
  hipLaunchKernelGGL(absorb_q_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_latent_up_proj(const LatentProjParams& p, hipStream_t stream) {
  const int n_hc = (p.H / p.G + kHeadChunk - 1) / kHeadChunk;
  const dim3 grid(p.B * p.q_len * p.G * n_hc, p.d_h / kUpCols);
  hipLaunchKernelGGL(up_proj_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
