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
//      the latent as a single KV head that is both K and V, and its merge)
//   3. out[h] = W_UV[g(h)] u[h]                 (at the end of that merge, one row per
//      workgroup, from the merged u in LDS)
// Steps 1 and 3 are small (rows x d_h x d_c multiply-adds per step, with rows =
// B * q_len * H); step 2 streams the latent cache and dominates.

#include "gqa_internal.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kThreads = 256;   // four independent waves per workgroup
constexpr int kMaxDc = 512;     // the latent width d_c

// The query fold runs on the matrix cores, one 16 x 16 output tile per wave
// (v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of A and column l % 16 of B,
// each at the eight reduction indices 8 (l / 16) .. + 7 of every 32-wide step, and
// receives D rows 4 (l / 16) .. + 3 of column l % 16). A tile's 16 rows are 16
// consecutive rows of one group: row r of group g is head g H/G + r % (H/G) of token
// r / (H/G), so every row of a tile uses the same W[g]. All of a wave's loads are
// independent and issued together.
__device__ __forceinline__ size_t group_row(const LatentProjParams& p, int g, int r) {
  const int hpg = p.H / p.G;
  return (size_t)(r / hpg) * p.H + g * hpg + r % hpg;   // row of [B q_len H]
}

// q_lat[row, c0 .. c0 + 15] = sum_i q[row, i] W_UK[g][i, c]
template <int D_H>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(LatentProjParams p) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int R_g = p.B * p.q_len * (p.H / p.G);           // rows per group
  const int n_rt = (R_g + 15) / 16;
  const int tile = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  constexpr int NCT = kMaxDc / 16;                        // column tiles
  if (tile >= p.G * n_rt * NCT) return;
  const int ct = tile % NCT;
  const int rt = (tile / NCT) % n_rt;
  const int g = tile / (NCT * n_rt);
  const int r = rt * 16 + l16;                            // this lane's A row
  const int c = ct * 16 + l16;                            // this lane's B column
  const __bf16* q = static_cast<const __bf16*>(p.q);
  const __bf16* w = static_cast<const __bf16*>(p.w_uk) + (size_t)g * D_H * kMaxDc + c;
  constexpr int KS = D_H / 32;                            // reduction steps
  bf16x8 a[KS], b[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    a[ks] = r < R_g ? *reinterpret_cast<const bf16x8*>(q + group_row(p, g, r) * D_H + ks * 32 + g4 * 8) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) b[ks][e] = w[(size_t)(ks * 32 + g4 * 8 + e) * kMaxDc];
  }
  f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b[ks], d, 0, 0, 0);
  __bf16* dst = static_cast<__bf16*>(p.q_lat);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = rt * 16 + g4 * 4 + j;
    if (rr < R_g) dst[group_row(p, g, rr) * kMaxDc + c] = (__bf16)d[j];
  }
}

}  // namespace

// d_c must be 512 and d_h 64 or 128 (checked by the planner).
static int tile_blocks(const LatentProjParams& p, int col_tiles) {
  const int R_g = p.B * p.q_len * (p.H / p.G);
  const long long tiles = (long long)p.G * ((R_g + 15) / 16) * col_tiles;
  return (int)((tiles + kThreads / 64 - 1) / (kThreads / 64));
}

hipError_t launch_latent_absorb_q(const LatentProjParams& p, hipStream_t stream) {
  if (p.d_c != kMaxDc || (p.d_h != 64 && p.d_h != 128)) return hipErrorInvalidValue;
  const dim3 grid(tile_blocks(p, kMaxDc / 16));
  if (p.d_h == 64)
    hipLaunchKernelGGL(absorb_q_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(absorb_q_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
