// Split-K GQA decode on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// What is computed: for the H/G query heads of KV group g (the aiwiki GQA listing's
// repeat_interleave grouping; the llms.blog page, "Grouped-Query Attention" >
// "Mathematical Formulation": the group's K/V head is broadcast to its H/G query
// heads) and the q_len new tokens, softmax(scale * Q K^T + mask) V over the cached
// keys (llms.blog, "Multi-Query Attention" > "Mathematical Formulation").
//
// How: one workgroup owns one (sequence b, group g, context split s). The group's
// R = (H/G) * q_len query rows are packed into 16-row MFMA tiles and held in
// registers; K/V tiles of the split are streamed from HBM once (each group is read
// once, as the aiwiki note after the listing asks), staged through LDS, and every
// packed row consumes them -- the H/G-fold broadcast happens in registers, never in
// memory.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, A 16x32 / B 32x16 / C 16x16):
//   QK^T is computed transposed, S^T = K Q^T, with K as the A operand (rows = keys)
//   and Q^T as B (columns = query rows). The C layout then leaves lane l with the
//   scores of query row l%16 for keys 4*(l/16)+i -- exactly the B-operand layout PV
//   needs for P^T, so no cross-lane shuffle sits between the two products.
//   PV is O^T = V^T P^T: A = V^T read transposed out of LDS, B = P^T (bf16), C = O^T
//   with lane l holding output row l%16. Online-softmax rescales (per query row) are
//   therefore per-lane scalars.
// The workgroup's waves split the tile either by keys (each wave its own key slice,
// merged through LDS at the end) or by row tiles (all waves read the same keys).

#include "gqa_internal.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float wave_max_across_groups(float x) {
  // lanes l, l^16, l^32, l^48 hold the same query row
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_across_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// LDS swizzles (16-byte chunk index XOR a function of the row) so that
//  * the QK A-operand reads (16 consecutive key rows, one chunk each) and
//  * the transposed V reads (rows 4 apart, two adjacent chunks each)
// hit distinct banks.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
__device__ __forceinline__ int swz_v(int row) { return ((row >> 2) & 3) << 1; }

__device__ __forceinline__ uint16_t lds_u16(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const uint16_t*>(base + byte_off);
}

template <int D, int T, int NKW, int NRW, int RTW, bool PAGED>
struct MfmaKernel {
  static constexpr int KW = T / NKW;          // keys per wave per step
  static constexpr int KB = KW / 16;          // 16-key blocks per wave
  static constexpr int CC = D / 32;           // k-steps of QK^T
  static constexpr int CB = D / 16;           // 16-column output blocks
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TENSOR_BYTES = T * ROW_BYTES;
  static constexpr int STAGE_BYTES = 2 * TENSOR_BYTES;
  static constexpr int LOADS = T * CPR / kThreads;   // 16-B loads per thread per tensor
  static constexpr int ROWS_PAD = 16 * RTW * NRW;     // packed rows covered
  static constexpr int RED_BYTES = (NKW > 1) ? NKW * ROWS_PAD * (D + 2) * 4 : 0;
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > RED_BYTES) ? 2 * STAGE_BYTES : RED_BYTES;
  static_assert(KW % 16 == 0 && (KB == 1 || KB % 2 == 0), "wave key slice");
  static_assert((T * CPR) % kThreads == 0, "tile load split");
  static_assert(NKW * NRW == 4, "four waves per workgroup");
};

template <int D, int T, int NKW, int NRW, int RTW, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  using K_ = MfmaKernel<D, T, NKW, NRW, RTW, PAGED>;
  constexpr int KW = K_::KW, KB = K_::KB, CC = K_::CC, CB = K_::CB, CPR = K_::CPR;
  constexpr int LOADS = K_::LOADS;
  __shared__ __attribute__((aligned(16))) unsigned char smem[K_::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kw = wave % NKW;
  const int rw = wave / NKW;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int split = blockIdx.x;
  const int grp = blockIdx.y;
  const int b = blockIdx.z;

  int L = p.seq_lens[b];
  L = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  const int start = split * p.chunk;
  if (start >= L) return;  // beyond this sequence: nothing to do (merge skips it)
  const int end = min(start + p.chunk, L);
  const int n_tiles = (end - start + T - 1) / T;

  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
  const unsigned char* __restrict__ kg = static_cast<const unsigned char*>(p.k);
  const unsigned char* __restrict__ vg = static_cast<const unsigned char*>(p.v);

  // ---- packed query rows of this group, as B operands of S^T = K Q^T ----
  bf16x8 qf[RTW][CC];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int r = (rw * RTW + rt) * 16 + l16;
    if (r < p.R) {
      const int t = r / p.hpg;
      const int h = grp * p.hpg + (r - t * p.hpg);
      const __bf16* qrow = qg + ((size_t)(b * p.q_len + t) * p.H + h) * D;
#pragma unroll
      for (int cc = 0; cc < CC; ++cc)
        qf[rt][cc] = *reinterpret_cast<const bf16x8*>(qrow + cc * 32 + g4 * 8);
    } else {
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) qf[rt][cc] = bf16x8{};
    }
  }

  // ---- K/V addressing ----
  size_t seq_base = 0;  // contiguous: start of (b, g) rows
  if constexpr (!PAGED) seq_base = ((size_t)b * p.G + grp) * (size_t)p.capacity * K_::ROW_BYTES;
  const int32_t* trow = PAGED ? p.table + (size_t)b * p.max_blocks : nullptr;
  const int pmask = (1 << p.page_shift) - 1;

  auto row_offset = [&](int j) -> size_t {
    if constexpr (PAGED) {
      int page = trow[j >> p.page_shift];
      page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
      return (((size_t)page * p.G + grp) * (size_t)(pmask + 1) + (j & pmask)) * K_::ROW_BYTES;
    } else {
      return seq_base + (size_t)j * K_::ROW_BYTES;
    }
  };

  u32x4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int tile) {
    const int t0 = start + tile * T;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int qi = n * kThreads + tid;
      const int row = qi / CPR, ch = qi % CPR;
      const int j = t0 + row;
      if (j < end) {
        const size_t off = row_offset(j) + ch * 16;
        kreg[n] = *reinterpret_cast<const u32x4*>(kg + off);
        vreg[n] = *reinterpret_cast<const u32x4*>(vg + off);
      } else {
        kreg[n] = u32x4{0, 0, 0, 0};
        vreg[n] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* ks = smem + stage * K_::STAGE_BYTES;
    unsigned char* vs = ks + K_::TENSOR_BYTES;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int qi = n * kThreads + tid;
      const int row = qi / CPR, ch = qi % CPR;
      *reinterpret_cast<u32x4*>(ks + row * K_::ROW_BYTES + ((ch ^ swz_k<CPR>(row)) << 4)) = kreg[n];
      *reinterpret_cast<u32x4*>(vs + row * K_::ROW_BYTES + ((ch ^ swz_v(row)) << 4)) = vreg[n];
    }
  };

  // ---- online-softmax state (per lane: query row l16 of each row tile) ----
  float m_run[RTW], l_run[RTW];
  f32x4 o[RTW][CB];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[rt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // last visible key of each of this lane's query rows
  int lim[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    int r = (rw * RTW + rt) * 16 + l16;
    r = r < p.R ? r : p.R - 1;
    lim[rt] = p.causal ? (L - p.q_len + r / p.hpg) : (L - 1);
  }
  const int lim_min = p.causal ? (L - p.q_len) : (L - 1);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    if (it + 1 < n_tiles) load_tile(it + 1);  // in flight while this tile is consumed

    const unsigned char* ks = smem + (it & 1) * K_::STAGE_BYTES;
    const unsigned char* vs = ks + K_::TENSOR_BYTES;
    const int tile0 = start + it * T;

    // S^T = K Q^T for this wave's KW keys and RTW row tiles
    f32x4 s[RTW][KB];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[rt][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = kw * KW + kb * 16 + l16;
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        const int ch = cc * 4 + g4;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(ks + row * K_::ROW_BYTES + ((ch ^ swz_k<CPR>(row)) << 4));
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
          s[rt][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][cc], s[rt][kb], 0, 0, 0);
      }
    }

    // online softmax (base 2) and P^T in bf16
    const bool need_mask = (tile0 + T - 1) > lim_min;
    float pr[RTW][KB][4];
    __bf16 pb16[RTW][KB][4];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[rt][kb][i] * p.qk_scale_log2;
          if (need_mask) {
            const int j = tile0 + kw * KW + kb * 16 + g4 * 4 + i;
            x = (j <= lim[rt]) ? x : kNegInf;
          }
          pr[rt][kb][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = wave_max_across_groups(mx);
      const float m_new = fmaxf(m_run[rt], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
      // P is rounded to bf16 for the PV product; the denominator sums the same
      // rounded weights so that the normalised weights sum to one.
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 e = (__bf16)__builtin_amdgcn_exp2f(pr[rt][kb][i] - m_use);
          pb16[rt][kb][i] = e;
          sum += (float)e;
        }
      l_run[rt] = l_run[rt] * alpha + sum;
      m_run[rt] = m_new;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) o[rt][cb] *= alpha;
    }

    // O^T += V^T P^T
    if constexpr (KB == 1) {
      bf16x4 pb[RTW];
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[rt][i] = pb16[rt][0][i];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c = cb * 16 + l16;
        uint32_t w[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int r0 = kw * KW + g4 * 4 + 2 * e2;
          const int r1 = r0 + 1;
          const uint32_t lo = lds_u16(vs, r0 * K_::ROW_BYTES + ((((c >> 3) ^ swz_v(r0)) << 4) | ((c & 7) << 1)));
          const uint32_t hi = lds_u16(vs, r1 * K_::ROW_BYTES + ((((c >> 3) ^ swz_v(r1)) << 4) | ((c & 7) << 1)));
          w[e2] = lo | (hi << 16);
        }
        const bf16x4 a = __builtin_bit_cast(bf16x4, u32x2{w[0], w[1]});
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
          o[rt][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[rt], o[rt][cb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kp = 0; kp < KB / 2; ++kp) {
        bf16x8 pb[RTW];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[rt][i] = pb16[rt][2 * kp][i];
            pb[rt][4 + i] = pb16[rt][2 * kp + 1][i];
          }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int c = cb * 16 + l16;
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            // k-slots 8*g4 + {2e2, 2e2+1}: keys of block 2kp (slots 0-3) then 2kp+1 (4-7)
            const int blk = 2 * kp + (e2 >> 1);
            const int r0 = kw * KW + blk * 16 + g4 * 4 + 2 * (e2 & 1);
            const int r1 = r0 + 1;
            const uint32_t lo = lds_u16(vs, r0 * K_::ROW_BYTES + ((((c >> 3) ^ swz_v(r0)) << 4) | ((c & 7) << 1)));
            const uint32_t hi = lds_u16(vs, r1 * K_::ROW_BYTES + ((((c >> 3) ^ swz_v(r1)) << 4) | ((c & 7) << 1)));
            w[e2] = lo | (hi << 16);
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt)
            o[rt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], o[rt][cb], 0, 0, 0);
        }
      }
    }

    if (it + 1 < n_tiles) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: per-row totals, cross-wave merge, normalise, write ----
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) l_run[rt] = wave_sum_across_groups(l_run[rt]);

  const size_t rows_per_b = (size_t)p.q_len * p.H;
  auto write_row4 = [&](int r, int c, f32x4 val, float m, float l) {
    // r < R: query row of this group; c multiple of 4
    const int t = r / p.hpg;
    const int h = grp * p.hpg + (r - t * p.hpg);
    const size_t orow = (size_t)b * rows_per_b + (size_t)t * p.H + h;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    val *= inv;
    if (p.max_splits == 1) {
      __bf16* op = static_cast<__bf16*>(p.out) + orow * D + c;
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)val[i];
      *reinterpret_cast<bf16x4*>(op) = ov;
    } else {
      const size_t ws_row = orow * p.max_splits + split;
      *reinterpret_cast<f32x4*>(p.ws_o + ws_row * D + c) = val;
      if (c == 0) p.ws_lse[ws_row] = (l > 0.f) ? m + __log2f(l) : kNegInf;
    }
  };

  if constexpr (NKW == 1) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int r = (rw * RTW + rt) * 16 + l16;
      if (r < p.R) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) write_row4(r, cb * 16 + g4 * 4, o[rt][cb], m_run[rt], l_run[rt]);
      }
    }
  } else {
    // Waves with the same row tiles but different key slices hold partial
    // (max, sum, unnormalised O) for the same rows: merge them through LDS.
    float* red_o = reinterpret_cast<float*>(smem);                         // [NKW][ROWS_PAD][D]
    float* red_m = red_o + NKW * K_::ROWS_PAD * D;                         // [NKW][ROWS_PAD]
    float* red_l = red_m + NKW * K_::ROWS_PAD;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int rl = (rw * RTW + rt) * 16 + l16;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<f32x4*>(red_o + ((size_t)kw * K_::ROWS_PAD + rl) * D + cb * 16 + g4 * 4) = o[rt][cb];
      if (g4 == 0) {
        red_m[kw * K_::ROWS_PAD + rl] = m_run[rt];
        red_l[kw * K_::ROWS_PAD + rl] = l_run[rt];
      }
    }
    __syncthreads();
    constexpr int ITEMS = K_::ROWS_PAD * D / 4;
    for (int item = tid; item < ITEMS; item += kThreads) {
      const int rl = item / (D / 4);
      const int c = (item % (D / 4)) * 4;
      if (rl >= p.R) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NKW; ++w) M = fmaxf(M, red_m[w * K_::ROWS_PAD + rl]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < NKW; ++w) {
        const float f = __builtin_amdgcn_exp2f(red_m[w * K_::ROWS_PAD + rl] - Mu);
        l += f * red_l[w * K_::ROWS_PAD + rl];
        acc += f * *reinterpret_cast<const f32x4*>(red_o + ((size_t)w * K_::ROWS_PAD + rl) * D + c);
      }
      write_row4(rl, c, acc, M, l);
    }
  }
}

template <int D, int T, int NKW, int NRW, int RTW>
hipError_t launch_variant(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream) {
  if (paged)
    hipLaunchKernelGGL((decode_mfma_kernel<D, T, NKW, NRW, RTW, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, T, NKW, NRW, RTW, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_for_rows(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream) {
  if (p.R <= 16) return launch_variant<D, 64, 4, 1, 1>(p, paged, grid, stream);
  if (p.R <= 32) return launch_variant<D, 64, 4, 1, 2>(p, paged, grid, stream);
  if (p.R <= 64) return launch_variant<D, 64, 2, 2, 2>(p, paged, grid, stream);
  if (p.R <= 128) return launch_variant<D, 64, 1, 4, 2>(p, paged, grid, stream);
  return launch_variant<D, 32, 1, 4, 4>(p, paged, grid, stream);
}

}  // namespace

MfmaVariant mfma_variant_for_rows(int R, int d_h) {
  auto mk = [&](int rows, int tile, int lds) { return MfmaVariant{rows, tile, lds}; };
  if (d_h == 64) {
    if (R <= 16) return mk(16, 64, MfmaKernel<64, 64, 4, 1, 1, false>::LDS_BYTES);
    if (R <= 32) return mk(32, 64, MfmaKernel<64, 64, 4, 1, 2, false>::LDS_BYTES);
    if (R <= 64) return mk(64, 64, MfmaKernel<64, 64, 2, 2, 2, false>::LDS_BYTES);
    if (R <= 128) return mk(128, 64, MfmaKernel<64, 64, 1, 4, 2, false>::LDS_BYTES);
    return mk(256, 32, MfmaKernel<64, 32, 1, 4, 4, false>::LDS_BYTES);
  }
  if (R <= 16) return mk(16, 64, MfmaKernel<128, 64, 4, 1, 1, false>::LDS_BYTES);
  if (R <= 32) return mk(32, 64, MfmaKernel<128, 64, 4, 1, 2, false>::LDS_BYTES);
  if (R <= 64) return mk(64, 64, MfmaKernel<128, 64, 2, 2, 2, false>::LDS_BYTES);
  if (R <= 128) return mk(128, 64, MfmaKernel<128, 64, 1, 4, 2, false>::LDS_BYTES);
  return mk(256, 32, MfmaKernel<128, 32, 1, 4, 4, false>::LDS_BYTES);
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int d_h, bool paged, dim3 grid,
                              hipStream_t stream) {
  (void)dtype;  // bf16 only (checked by the planner)
  if (d_h == 64) return launch_for_rows<64>(p, paged, grid, stream);
  return launch_for_rows<128>(p, paged, grid, stream);
}

}  // namespace gqa
