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
// Split-K grid: one 256-thread workgroup per output row (b, t, h). A split's D
// partial values are read by D/4 lanes with 16-byte loads; the workgroup walks
// 4 * (256 / D) splits per round, several rounds in flight per lane, and reduces
// across waves through LDS.
//
// Persistent schedule: the decode kernel's workgroups share one flat sequence of
// key tiles (segment (b, g, rb) = the n_b tiles of sequence b for row block rb of KV
// group g, segments in (b, g, rb) order). Workgroup w owns tiles [lo(w), hi(w)), lo(w) = floor(w W / nwg).
// A segment inside one workgroup was written straight to the output; a segment cut
// by workgroup boundaries left one partial per workgroup it touches: in the
// workgroup's slot 0 if the segment holds the workgroup's first tile, else in
// slot 1 (it is then that workgroup's last segment). The merge recomputes the same
// ownership from the prefix sums the decode kernel published. One wave per (segment,
// packed row), four rows per workgroup, when segments hold few partials; else (and
// with a call-time head map, whose rows are found with a workgroup-wide ballot, or
// 512-wide rows) one workgroup per (segment, row).

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
hipError_t go(const DecodeParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int total = p.B * p.q_len * p.H;
  launch_timed(merge_kernel<TT, D>, dim3(total), stream, start, stop, p);
  return hipGetLastError();
}

constexpr int kPersistSlots = 2;

__device__ __forceinline__ int tile_lo(int w, int W, int nwg) {
  return (int)(((long long)w * W) / nwg);
}

// Workgroup owning flat tile f: the largest w with lo(w) <= f.
__device__ __forceinline__ int tile_owner(int f, int W, int nwg) {
  return (int)((((long long)f + 1) * nwg - 1) / W);
}

// GQLA absorbed execution, after the merge of a row's weighted latent u (512 values
// in sm_u): out[row, i] = sum_c W_UV[gq][i, c] u[c], gq the row's query group. A wave
// takes eight outputs at a time: lane l works on output i0 + l / 8 and reads 16-byte
// chunks (l % 8) + 8 s, s = 0..7, of that output's 1 KiB weight row, so every load
// instruction covers eight whole 128-byte lines (one thread per output instead made
// each load touch 64 lines). Each lane keeps the 64 values of u its chunks meet in
// registers; the eight lanes of an output add their fp32 dot products by lane swaps.
__device__ __forceinline__ void project_up(const DecodeParams& p, const float* sm_u, size_t orow, int h) {
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 7;    // chunk within each 128-byte line
  const int oi = lane >> 3;    // output within the wave's eight
  const int dh = p.proj_dh;    // 64 or 128
  const int gq = h / (p.H / p.proj_groups);
  const __bf16* w = static_cast<const __bf16*>(p.w_uv) + (size_t)gq * dh * 512;
  f32x4 u[8][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u[s][0] = *reinterpret_cast<const f32x4*>(sm_u + (sub + 8 * s) * 8);
    u[s][1] = *reinterpret_cast<const f32x4*>(sm_u + (sub + 8 * s) * 8 + 4);
  }
  // eight loads in flight per pass; issuing every pass's loads at once (208 instead
  // of 126 registers) measured no faster
  for (int i0 = wave * 8; i0 < dh; i0 += kThreads / 8) {
    const __bf16* wrow = w + (size_t)(i0 + oi) * 512 + sub * 8;
    bf16x8 wv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) wv[s] = *reinterpret_cast<const bf16x8*>(wrow + s * 64);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = __builtin_fmaf((float)wv[s][e], u[s][0][e], a[e]);
        a[e] = __builtin_fmaf((float)wv[s][4 + e], u[s][1][e], a[e]);
      }
    float acc = (a[0] + a[1]) + (a[2] + a[3]);
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (sub == 0) static_cast<__bf16*>(p.proj_out)[orow * dh + i0 + oi] = (__bf16)acc;
  }
}

// With a call-time head -> KV head map, the packed tile of KV group g holds the rows
// r = t * n_g + k (token t, k-th head of the group in ascending order) below
// cap = n_row_blocks * row_block. A group larger than the planned bound leaves its rows
// r >= cap uncomputed, and a head whose map entry lies outside [0, G) belongs to no
// group: the decode kernel never writes those (token, head) rows of `out`. This routine
// writes NaN into exactly those rows, so that `out` is always fully overwritten and a
// bad map shows up in the result. One workgroup per (sequence, token): bt = b * q_len + t.
// The persistent merge kernels run it in extra workgroups after their own; the split-K
// path launches it as a kernel of its own.
__device__ __forceinline__ void fill_unmapped_rows(const DecodeParams& p, int d_h, int bt) {
  __shared__ int grp[kThreads];
  __shared__ unsigned char dropped[kThreads];
  const int tid = threadIdx.x;
  const int t = bt % p.q_len;
  if (tid < p.H) grp[tid] = p.head_group[tid];
  __syncthreads();
  if (tid < p.H) {
    const int g = grp[tid];
    bool drop = g < 0 || g >= p.G;
    if (!drop) {
      int k = 0, n_g = 0;
      for (int h = 0; h < p.H; ++h) {
        if (grp[h] == g) {
          k += h < tid;
          ++n_g;
        }
      }
      drop = t * n_g + k >= p.n_row_blocks * p.row_block;
    }
    dropped[tid] = drop ? 1 : 0;
  }
  __syncthreads();
  // the rows to fill, d_h / 4 lanes per head
  const int lph = d_h / 4;
  for (int i = tid; i < p.H * lph; i += kThreads) {
    const int h = i / lph;
    if (!dropped[h]) continue;
    const size_t off = ((size_t)bt * p.H + h) * d_h + (i % lph) * 4;
    put4<__bf16>(static_cast<__bf16*>(p.out) + off, f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                          __builtin_nanf(""), __builtin_nanf("")});
  }
}

__global__ __launch_bounds__(kThreads) void fill_unmapped_rows_kernel(DecodeParams p, int d_h) {
  fill_unmapped_rows(p, d_h, blockIdx.x);
}

// One workgroup per (segment, row): D/4 lanes cover the row's D columns and the
// workgroup's 256 / (D/4) lane groups take the segment's partials in turn, several
// in flight per lane, each group keeping a running max; the groups then combine
// through LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_persistent_kernel(DecodeParams p) {
  constexpr int LPR = D / 4;               // lanes per row (4 columns each)
  constexpr int NGRP = kThreads / LPR;     // partial groups
  // partials in flight per lane: a 512-wide row leaves only two lane groups per
  // workgroup, so each takes more at once
  constexpr int U = D == 512 ? 16 : 4;
  __shared__ float sm_m[NGRP];
  __shared__ float sm_l[NGRP];
  __shared__ f32x4 sm_o[NGRP][LPR];
  __shared__ unsigned long long sm_heads[kThreads / 64];
  __shared__ __attribute__((aligned(16))) float sm_u[D == 512 ? D : 4];  // GQLA: the merged latent
  const bool proj = D == 512 && p.w_uv != nullptr;

  const int RB = p.row_block;                     // rows per segment
  const int GS = p.G * p.n_row_blocks;            // segments per sequence
  if constexpr (D <= 128) {
    const int merge_blocks = p.B * GS * RB;
    if ((int)blockIdx.x >= merge_blocks) {  // the head map's unmapped rows
      fill_unmapped_rows(p, D, blockIdx.x - merge_blocks);
      return;
    }
  }
  const int seg = blockIdx.x / RB;
  const int r_local = blockIdx.x - seg * RB;
  const int b = seg / GS;
  const int gs = seg - b * GS;
  const int g = gs / p.n_row_blocks;
  const int r = (gs - g * p.n_row_blocks) * RB + r_local;  // packed row of group g

  // (token, head) of packed row r, as the decode kernel maps it: token r / n_g of the
  // group's (r % n_g)-th head in ascending order (contiguous groups without a map)
  int n_g = p.hpg;
  if (p.head_group) {
    const bool in = (int)threadIdx.x < p.H && p.head_group[threadIdx.x] == g;
    const unsigned long long bits = __builtin_amdgcn_ballot_w64(in);
    if ((threadIdx.x & 63) == 0) sm_heads[threadIdx.x >> 6] = bits;
    __syncthreads();
    n_g = 0;
#pragma unroll
    for (int wv = 0; wv < kThreads / 64; ++wv) n_g += __builtin_popcountll(sm_heads[wv]);
  }
  if (r >= n_g * p.q_len) return;
  const int t = r / n_g;
  const int kh = r - t * n_g;  // the row's head is the group's kh-th
  int h = g * n_g + kh;
  if (p.head_group) {
    int seen = 0;
    for (int wv = 0; wv < kThreads / 64; ++wv) {
      unsigned long long bits = sm_heads[wv];
      while (bits) {
        if (seen == kh) h = wv * 64 + __builtin_ctzll(bits);
        ++seen;
        bits &= bits - 1;
      }
    }
  }
  const size_t orow = ((size_t)b * p.q_len + t) * p.H + h;
  const bool on = p.head_active == nullptr || p.head_active[orow] != 0;

  const int W = p.ws_prefix[p.B];
  const int pre = p.ws_prefix[b];
  const int n = (p.ws_prefix[b + 1] - pre) / GS;  // tiles per segment of b
  if (n <= 0 || W <= 0) return;
  const int s0 = pre + gs * n;
  const int wa = tile_owner(s0, W, p.nwg);
  const int wb = tile_owner(s0 + n - 1, W, p.nwg);
  const int tid = threadIdx.x;
  const int grp = tid / LPR;
  const int c = (tid % LPR) * 4;
  if (wa == wb) {  // written whole by one workgroup
    if constexpr (D == 512) {
      if (proj) {
        if (grp == 0)
          *reinterpret_cast<f32x4*>(sm_u + c) =
              *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.out) + orow * D + c);
        __syncthreads();
        project_up(p, sm_u, orow, h);
      }
    }
    return;
  }
  const int slot_a = tile_lo(wa, W, p.nwg) < s0 ? 1 : 0;

  float m = kNegInf, l = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // with at least as many tiles as workgroups every workgroup owns a tile, and the
  // per-partial emptiness test (two 64-bit divisions) can be skipped
  const bool all_owned = W >= p.nwg;
  for (int base = wa + grp; base <= wb; base += NGRP * U) {
    float lse[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = base + u * NGRP;
      lse[u] = kNegInf;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (w <= wb && (all_owned || tile_lo(w, W, p.nwg) < tile_lo(w + 1, W, p.nwg))) {  // else empty
        const size_t prow = ((size_t)w * kPersistSlots + (w == wa ? slot_a : 0)) * RB + r_local;
        lse[u] = p.ws_lse[prow];
        v[u] = *reinterpret_cast<const f32x4*>(p.ws_o + prow * D + c);
      }
    }
    float mu = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mu = fmaxf(mu, lse[u]);
    if (mu == kNegInf) continue;  // nothing visible yet
    const float sc = __builtin_amdgcn_exp2f(m - mu);  // 0 while m = -inf
    acc *= sc;
    l *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wt = __builtin_amdgcn_exp2f(lse[u] - mu);
      acc += wt * v[u];
      l += wt;
    }
    m = mu;
  }
  if (tid % LPR == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
  sm_o[grp][tid % LPR] = acc;
  __syncthreads();
  if (grp == 0) {
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < NGRP; ++k) M = fmaxf(M, sm_m[k]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
#pragma unroll
    for (int k = 0; k < NGRP; ++k) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[k] - Mu);
      tot += wt * sm_o[k][tid];
      lt += wt * sm_l[k];
    }
    const float inv = (lt > 0.f && on) ? 1.f / lt : 0.f;
    if (proj)
      *reinterpret_cast<f32x4*>(sm_u + c) = tot * inv;
    else if (p.out_f32)
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow * D + c) = tot * inv;
    else
      put4<__bf16>(static_cast<__bf16*>(p.out) + orow * D + c, tot * inv);
  }
  if constexpr (D == 512) {
    if (proj) {
      __syncthreads();
      project_up(p, sm_u, orow, h);
    }
  }
}

// The same merge with one wave per (segment, packed row) and four rows of a segment
// per workgroup, for contiguous head groups and D <= 128: the wave's 256 / D lane
// groups take the row's partials in turn and combine through lane swaps, with no LDS
// and no workgroup barrier.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_persistent_wave_kernel(DecodeParams p) {
  constexpr int LPR = D / 4;   // lanes per row group (4 columns each)
  constexpr int NG = 64 / LPR; // row groups per wave
  constexpr int U = 4;         // partials in flight per lane
  static_assert(NG >= 2 && NG * LPR == 64, "a wave holds whole row groups");

  const int RB = p.row_block;
  const int quads = (RB + 3) / 4;
  const int GS = p.G * p.n_row_blocks;
  const int merge_blocks = p.B * GS * quads;
  if ((int)blockIdx.x >= merge_blocks) {  // the head map's unmapped rows
    fill_unmapped_rows(p, D, blockIdx.x - merge_blocks);
    return;
  }
  const int seg = blockIdx.x / quads;
  const int r_local = (blockIdx.x - seg * quads) * 4 + (int)(threadIdx.x >> 6);
  if (r_local >= RB) return;  // the whole wave
  const int b = seg / GS;
  const int gs = seg - b * GS;
  const int g = gs / p.n_row_blocks;
  const int r = (gs - g * p.n_row_blocks) * RB + r_local;
  // (token, head) of packed row r as the decode kernel maps it: token r / n_g of the
  // group's (r % n_g)-th head in ascending order. With a head map the wave finds the
  // group's heads with one ballot per 64 heads.
  int n_g = p.hpg;
  unsigned long long gm[4] = {0ull, 0ull, 0ull, 0ull};
  if (p.head_group) {
    n_g = 0;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int hh = ch * 64 + (int)(threadIdx.x & 63);
      gm[ch] = __builtin_amdgcn_ballot_w64(hh < p.H && p.head_group[hh] == g);
      n_g += __builtin_popcountll(gm[ch]);
    }
  }
  if (r >= n_g * p.q_len) return;
  const int t = r / n_g;
  const int kh = r - t * n_g;
  int h = g * n_g + kh;
  if (p.head_group) {
    int before = 0;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int cnt = __builtin_popcountll(gm[ch]);
      if (kh >= before && kh < before + cnt) {
        unsigned long long bits = gm[ch];
        for (int i = before; i < kh; ++i) bits &= bits - 1;  // drop the lower set bits
        h = ch * 64 + __builtin_ctzll(bits);
      }
      before += cnt;
    }
  }
  const size_t orow = ((size_t)b * p.q_len + t) * p.H + h;
  const bool on = p.head_active == nullptr || p.head_active[orow] != 0;

  const int W = p.ws_prefix[p.B];
  const int pre = p.ws_prefix[b];
  const int n = (p.ws_prefix[b + 1] - pre) / GS;
  if (n <= 0 || W <= 0) return;
  const int s0 = pre + gs * n;
  const int wa = tile_owner(s0, W, p.nwg);
  const int wb = tile_owner(s0 + n - 1, W, p.nwg);
  if (wa == wb) return;

  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR;
  const int c = (lane % LPR) * 4;
  const int slot_a = tile_lo(wa, W, p.nwg) < s0 ? 1 : 0;
  const bool all_owned = W >= p.nwg;
  float m = kNegInf, l = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int base = wa + grp; base <= wb; base += NG * U) {
    float lse[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = base + u * NG;
      lse[u] = kNegInf;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (w <= wb && (all_owned || tile_lo(w, W, p.nwg) < tile_lo(w + 1, W, p.nwg))) {
        const size_t prow = ((size_t)w * kPersistSlots + (w == wa ? slot_a : 0)) * RB + r_local;
        lse[u] = p.ws_lse[prow];
        v[u] = *reinterpret_cast<const f32x4*>(p.ws_o + prow * D + c);
      }
    }
    float mu = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mu = fmaxf(mu, lse[u]);
    if (mu == kNegInf) continue;
    const float sc = __builtin_amdgcn_exp2f(m - mu);
    acc *= sc;
    l *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wt = __builtin_amdgcn_exp2f(lse[u] - mu);
      acc += wt * v[u];
      l += wt;
    }
    m = mu;
  }
  // combine the row groups: lanes LPR, 2 LPR, ... apart hold the same columns
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    f32x4 a2;
#pragma unroll
    for (int i = 0; i < 4; ++i) a2[i] = __shfl_xor(acc[i], off);
    const float M = fmaxf(m, m2);
    const float Mu = (M == kNegInf) ? 0.f : M;
    const float w1 = __builtin_amdgcn_exp2f(m - Mu);
    const float w2 = __builtin_amdgcn_exp2f(m2 - Mu);
    acc = acc * w1 + a2 * w2;
    l = l * w1 + l2 * w2;
    m = M;
  }
  if (grp != 0) return;
  const float inv = (l > 0.f && on) ? 1.f / l : 0.f;
  if (p.out_f32)
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow * D + c) = acc * inv;
  else
    put4<__bf16>(static_cast<__bf16*>(p.out) + orow * D + c, acc * inv);
}

template <int D>
hipError_t go_persistent(const DecodeParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  // with a head map, one more workgroup per (sequence, token) fills the unmapped rows
  if (p.head_group && (D > 128 || p.H > kThreads)) return hipErrorInvalidValue;
  const int fill_blocks = p.head_group ? p.B * p.q_len : 0;
  if constexpr (D <= 128) {
    // A wave takes 4 * (256 / D) partials per round, a workgroup four times as many:
    // the wave form wins while segments average up to two of its rounds of partials
    // (about nwg / segments each), the workgroup form beyond.
    const long long segments = (long long)p.B * p.G * p.n_row_blocks;
    if (p.nwg <= 2 * (4 * (256 / D)) * segments) {
      const dim3 grid(p.B * p.G * p.n_row_blocks * ((p.row_block + 3) / 4) + fill_blocks);
      launch_timed(merge_persistent_wave_kernel<D>, grid, stream, start, stop, p);
      return hipGetLastError();
    }
  }
  const dim3 grid(p.B * p.G * p.n_row_blocks * p.row_block + fill_blocks);
  launch_timed(merge_persistent_kernel<D>, grid, stream, start, stop, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_unmapped(const DecodeParams& p, int d_h, hipStream_t stream) {
  if (p.H > kThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_unmapped_rows_kernel, dim3(p.B * p.q_len), dim3(kThreads), 0, stream, p, d_h);
  return hipGetLastError();
}

hipError_t launch_merge_persistent(const DecodeParams& p, int d_h, hipStream_t stream, hipEvent_t start,
                                   hipEvent_t stop) {
  if (d_h == 512) return go_persistent<512>(p, stream, start, stop);
  return d_h == 64 ? go_persistent<64>(p, stream, start, stop) : go_persistent<128>(p, stream, start, stop);
}

hipError_t launch_merge(const DecodeParams& p, int dtype, int d_h, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop) {
  if (dtype == 0) return d_h == 64 ? go<float, 64>(p, stream, start, stop) : go<float, 128>(p, stream, start, stop);
  return d_h == 64 ? go<__bf16, 64>(p, stream, start, stop) : go<__bf16, 128>(p, stream, start, stop);
}

}  // namespace gqa
