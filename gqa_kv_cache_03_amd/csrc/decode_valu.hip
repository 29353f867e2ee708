// Split-K GQA decode on the vector ALUs: fp32 caches, and bf16 groups with too few
// packed query rows (R < 4) for a dense matrix-core contraction.
//
// Same method as the MFMA kernel (softmax(scale * Q K^T + mask) V per group, the
// group's K/V read once and broadcast in registers to its query rows; llms.blog GQA
// page, "Grouped-Query Attention" > "Mathematical Formulation"), with a different
// inner product: a row of d_h elements is spread over LPK lanes, 16 bytes each, so a
// group of LPK lanes reads one key row with one coalesced 16-byte load per lane.
// Dot products reduce across those lanes with xor-shuffles; every lane group keeps
// its own online-softmax state over a strided subset of the split's keys, and the
// groups are merged through LDS at the end.

#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

template <typename TT> struct Elem;
template <> struct Elem<float> {
  __device__ static void unpack(const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the lane out first: bit-casting a vector-element expression directly
      // reads element 0 on this compiler
      const uint32_t x = w[i];
      f[i] = __builtin_bit_cast(float, x);
    }
  }
};
template <> struct Elem<__bf16> {
  __device__ static void unpack(const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
};

template <typename TT> __device__ __forceinline__ void store_out(TT* dst, float v);
template <> __device__ __forceinline__ void store_out<float>(float* dst, float v) { *dst = v; }
template <> __device__ __forceinline__ void store_out<__bf16>(__bf16* dst, float v) { *dst = (__bf16)v; }

template <typename TT, int D, int RB>
struct ValuGeo {
  static constexpr int ES = sizeof(TT);
  static constexpr int E = 16 / ES;            // elements per lane per row
  static constexpr int LPK = D / E;            // lanes per key row
  static constexpr int NG = kThreads / LPK;    // key groups per workgroup
  static constexpr int LDS_BYTES = NG * RB * (D + 2) * 4;
  static_assert(LPK <= 64 && (64 % LPK) == 0, "row must fit in a wave");
};

template <typename TT, int D, int RB, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeParams p) {
  using Geo = ValuGeo<TT, D, RB>;
  constexpr int E = Geo::E, LPK = Geo::LPK, NG = Geo::NG;
  constexpr int ROW_BYTES = D * Geo::ES;
  __shared__ __attribute__((aligned(16))) float red[NG * RB * (D + 2)];

  const int tid = threadIdx.x;
  const int li = tid % LPK;      // lane within the key-row group
  const int kgp = tid / LPK;     // key group

  const int split = blockIdx.x;
  const int g = blockIdx.y / p.n_row_blocks;
  const int rb = blockIdx.y % p.n_row_blocks;
  const int b = blockIdx.z;

  int L = p.seq_lens[b];
  L = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  const int start = split * p.chunk;
  if (start >= L) return;
  const int end = min(start + p.chunk, L);

  const int r0 = rb * RB;
  const int nrows = min(RB, p.R - r0);

  float qv[RB][E];
  int lim[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int rr = r0 + (r < nrows ? r : nrows - 1);
    const int t = rr / p.hpg;
    const int h = g * p.hpg + (rr - t * p.hpg);
    const TT* qrow = static_cast<const TT*>(p.q) + ((size_t)(b * p.q_len + t) * p.H + h) * D;
    const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + li * E);
    Elem<TT>::unpack(w, qv[r]);
    lim[r] = p.causal ? (L - p.q_len + t) : (L - 1);
  }

  const unsigned char* kg = static_cast<const unsigned char*>(p.k);
  const unsigned char* vg = static_cast<const unsigned char*>(p.v);
  const int pmask = (1 << p.page_shift) - 1;
  auto row_offset = [&](int j) -> size_t {
    if constexpr (PAGED) {
      int page = p.table[(size_t)b * p.max_blocks + (j >> p.page_shift)];
      page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
      return (((size_t)page * p.G + g) * (size_t)(pmask + 1) + (j & pmask)) * ROW_BYTES;
    } else {
      return (((size_t)b * p.G + g) * (size_t)p.capacity + j) * ROW_BYTES;
    }
  };

  float m[RB], l[RB], o[RB][E];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[r][e] = 0.f;
  }

  constexpr int U = 2;  // keys per group per iteration (loads issued together)
  for (int j0 = start + kgp; j0 < end; j0 += NG * U) {
    u32x4 kw[U], vw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * NG;
      ok[u] = j < end;
      if (ok[u]) {
        const size_t off = row_offset(j) + li * 16;
        kw[u] = *reinterpret_cast<const u32x4*>(kg + off);
        vw[u] = *reinterpret_cast<const u32x4*>(vg + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      const int j = j0 + u * NG;
      float kf[E], vf[E];
      Elem<TT>::unpack(kw[u], kf);
      Elem<TT>::unpack(vw[u], vf);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(qv[r][e], kf[e], s);
#pragma unroll
        for (int off = LPK / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
        if (r >= nrows || j > lim[r]) continue;
        const float x = s * p.qk_scale_log2;
        const float m_new = fmaxf(m[r], x);
        const float alpha = __builtin_amdgcn_exp2f(m[r] - m_new);
        const float pe = __builtin_amdgcn_exp2f(x - m_new);
        l[r] = l[r] * alpha + pe;
#pragma unroll
        for (int e = 0; e < E; ++e) o[r][e] = fmaf(pe, vf[e], o[r][e] * alpha);
        m[r] = m_new;
      }
    }
  }

  // merge the NG key groups
  float* red_o = red;                        // [NG][RB][D]
  float* red_m = red + NG * RB * D;          // [NG][RB]
  float* red_l = red_m + NG * RB;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int e = 0; e < E; ++e) red_o[((size_t)kgp * RB + r) * D + li * E + e] = o[r][e];
    if (li == 0) {
      red_m[kgp * RB + r] = m[r];
      red_l[kgp * RB + r] = l[r];
    }
  }
  __syncthreads();
  const size_t rows_per_b = (size_t)p.q_len * p.H;
  for (int item = tid; item < RB * D; item += kThreads) {
    const int r = item / D, c = item % D;
    if (r >= nrows) continue;
    float M = kNegInf;
    for (int w = 0; w < NG; ++w) M = fmaxf(M, red_m[w * RB + r]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float acc = 0.f, lt = 0.f;
    for (int w = 0; w < NG; ++w) {
      const float f = __builtin_amdgcn_exp2f(red_m[w * RB + r] - Mu);
      lt += f * red_l[w * RB + r];
      acc += f * red_o[((size_t)w * RB + r) * D + c];
    }
    const int rr = r0 + r;
    const int t = rr / p.hpg;
    const int h = g * p.hpg + (rr - t * p.hpg);
    const size_t orow = (size_t)b * rows_per_b + (size_t)t * p.H + h;
    const float val = (lt > 0.f) ? acc / lt : 0.f;
    if (p.max_splits == 1) {
      store_out<TT>(static_cast<TT*>(p.out) + orow * D + c, val);
    } else {
      const size_t ws_row = orow * p.max_splits + split;
      p.ws_o[ws_row * D + c] = val;
      if (c == 0) p.ws_lse[ws_row] = (lt > 0.f) ? M + __log2f(lt) : kNegInf;
    }
  }
}

template <typename TT, int D, int RB>
hipError_t launch3(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream, hipEvent_t start,
                   hipEvent_t stop) {
  if (paged)
    launch_timed(decode_valu_kernel<TT, D, RB, true>, grid, stream, start, stop, p);
  else
    launch_timed(decode_valu_kernel<TT, D, RB, false>, grid, stream, start, stop, p);
  return hipGetLastError();
}

template <typename TT, int D>
hipError_t launch2(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream, hipEvent_t start,
                   hipEvent_t stop) {
  switch (p.row_block) {
    case 1: return launch3<TT, D, 1>(p, paged, grid, stream, start, stop);
    case 2: return launch3<TT, D, 2>(p, paged, grid, stream, start, stop);
    case 4: return launch3<TT, D, 4>(p, paged, grid, stream, start, stop);
    default: return launch3<TT, D, 8>(p, paged, grid, stream, start, stop);
  }
}

}  // namespace

int valu_tile_tokens(int dtype, int d_h) {
  // keys consumed by one workgroup pass (every key group takes U = 2 keys)
  const int lpk = d_h / (dtype == 0 ? 4 : 8);
  return 2 * (kThreads / lpk);
}

int valu_lds_bytes(int dtype, int d_h, int row_block) {
  const int lpk = d_h / (dtype == 0 ? 4 : 8);
  return (kThreads / lpk) * row_block * (d_h + 2) * 4;
}

hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int d_h, bool paged, dim3 grid,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (dtype == 0) {
    if (d_h == 64) return launch2<float, 64>(p, paged, grid, stream, start, stop);
    return launch2<float, 128>(p, paged, grid, stream, start, stop);
  }
  if (d_h == 64) return launch2<__bf16, 64>(p, paged, grid, stream, start, stop);
  return launch2<__bf16, 128>(p, paged, grid, stream, start, stop);
}

}  // namespace gqa
