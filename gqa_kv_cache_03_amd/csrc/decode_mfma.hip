// Split-K GQA decode on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// What is computed: for the H/G query heads of KV group g (the aiwiki GQA listing's
// repeat_interleave grouping; the llms.blog page, "Grouped-Query Attention" >
// "Mathematical Formulation": the group's K/V head is broadcast to its H/G query
// heads) and the q_len new tokens, softmax(scale * Q K^T + mask) V over the cached
// keys (llms.blog, "Multi-Query Attention" > "Mathematical Formulation").
//
// How: one workgroup owns one (sequence b, group g, context split s). The group's
// R = (H/G) * q_len query rows are packed into 16-row MFMA tiles held in registers.
// The split's K/V rows stream from HBM exactly once (the aiwiki note after the
// listing: the cache is read once, not copied per head) into a 4-stage LDS ring with
// direct global->LDS loads (nontemporal, 16 bytes per lane), so three tiles are in
// flight while the fourth is consumed; every packed row consumes each staged tile,
// i.e. the H/G-fold broadcast happens in registers, never in memory.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, A 16x32 / B 32x16 / C 16x16):
//   QK^T is computed transposed, S^T = K Q^T, with K as the A operand (rows = keys)
//   and Q^T as B (columns = query rows). The C layout leaves lane l with the scores
//   of query row l%16 for keys 4*(l/16)+i -- the B-operand layout PV needs for P^T,
//   so nothing is shuffled between the two products.
//   PV is O^T = V^T P^T: A = V^T read transposed out of LDS, B = P^T (bf16), C = O^T
//   with lane l holding output row l%16, so online-softmax rescales are per lane.
// The four waves split the work of a tile by keys (NKW), by row tiles (NRW) and by
// output columns (NCW); key slices are merged through LDS at the end.

#include "gqa_internal.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kTile = 32;     // keys per pipeline stage
constexpr int kStages = 4;    // LDS ring depth
constexpr int kNontemporal = 2;  // cache-policy bit for streaming loads
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

// Wait until at most N vector-memory operations of this wave are outstanding and all
// of its LDS operations are done, then synchronise the workgroup. The direct-to-LDS
// loads are tracked by the vector-memory counter, so after this every wave's loads of
// the awaited tile have landed in LDS.
template <int N>
__device__ __forceinline__ void wait_tile_and_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4);  // vmcnt(N) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits for this wave's LDS operations only: vector-memory
// loads in flight (the register prefetch ring) are not awaited.
__device__ __forceinline__ void lds_sync() {
  constexpr int imm = 15 | (3 << 14) | (7 << 4);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS swizzles (16-byte chunk index XOR a function of the row) so that the QK
// A-operand reads (16 consecutive key rows, one chunk each) and the transposed V
// reads (rows 4 apart, two adjacent chunks each) hit distinct banks.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
__device__ __forceinline__ int swz_v(int row) { return ((row >> 2) & 3) << 1; }

// One 16-byte direct global->LDS load per lane (nontemporal): lane i of the wave
// writes LDS bytes [lds_wave_base + 16 i, +16). Device-only: the host pass of this
// translation unit must not see the builtin (it would drop the kernel stubs).
__device__ __forceinline__ void load16_to_lds(const unsigned char* src, unsigned char* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)lds_wave_base, 16, 0, kNontemporal);
#else
  (void)src;
  (void)lds_wave_base;
#endif
}

// The block table is read-only for the whole kernel: reading it through the constant
// address space makes the (wave-uniform) reads scalar loads, which the direct-to-LDS
// loads in flight cannot delay (a vector load would have to wait for all of them).
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* base, int idx) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(4))) int32_t*)base)[idx];
#else
  return base[idx];
#endif
}

__device__ __forceinline__ uint32_t lds_u16(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const uint16_t*>(base + byte_off);
}

// Staging of K/V tiles on their way from HBM to the matrix cores.
//  kDmaRing: direct global->LDS loads into a 4-stage LDS ring (no registers used;
//            bytes in flight are bounded by the ring, i.e. by LDS capacity).
//  kRegRing: nontemporal 16-byte loads into a ring of register sets P tiles deep,
//            copied into a 2-stage LDS buffer one step ahead of use; the register
//            file is ~3x larger than LDS, so far more bytes can be in flight.
enum Staging { kDmaRing = 0, kRegRing = 1 };

template <int D, int NKW, int NRW, int NCW, int RTW, int T_, int MODE, int P_>
struct MfmaCfg {
  static constexpr int T = T_;                // keys per pipeline stage
  static constexpr int NS = MODE == kDmaRing ? kStages : 2;   // LDS stages
  static constexpr int P = P_;                // register sets (kRegRing)
  static constexpr int KW = T / NKW;          // keys per wave per stage
  static constexpr int KB = KW / 16;          // 16-key blocks per wave
  static constexpr int CC = D / 32;           // k-steps of QK^T
  static constexpr int CB = D / 16;           // 16-column output blocks
  static constexpr int CBW = CB / NCW;        // output blocks per wave
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TENSOR_BYTES = T * ROW_BYTES;
  static constexpr int STAGE_BYTES = 2 * TENSOR_BYTES;
  static constexpr int LOADS = T * CPR / kThreads;  // 16-B loads per thread per tensor
  static constexpr int LD = 2 * LOADS;              // per thread per stage (K and V)
  static constexpr int ROWS_PAD = 16 * RTW * NRW;
  static constexpr int RED_BYTES = (NKW > 1) ? NKW * ROWS_PAD * (D + 2) * 4 : 0;
  static constexpr int RING_BYTES = NS * STAGE_BYTES;
  static constexpr int LDS_BYTES = RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;
  static constexpr int NGRP = T / 16;               // 16-row groups per stage (paged)
  static_assert(NKW * NRW * NCW == 4, "four waves per workgroup");
  static_assert(KW % 16 == 0 && (KB == 1 || KB % 2 == 0), "wave key slice");
  static_assert(LOADS >= 1 && (T * CPR) % kThreads == 0, "stage load split");
  static_assert(CB % NCW == 0, "column split");
  static_assert(MODE == kDmaRing || P >= 2, "register ring depth");
};

template <int D, int NKW, int NRW, int NCW, int RTW, int T_, int MODE, int P_, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  using C = MfmaCfg<D, NKW, NRW, NCW, RTW, T_, MODE, P_>;
  constexpr int T = C::T, NS = C::NS, KW = C::KW, KB = C::KB, CC = C::CC, CBW = C::CBW;
  constexpr int CPR = C::CPR, LOADS = C::LOADS, LD = C::LD, ROW_BYTES = C::ROW_BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cw = wave % NCW;
  const int kw = (wave / NCW) % NKW;
  const int rw = wave / (NCW * NKW);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int split = blockIdx.x;
  const int grp = blockIdx.y;
  const int b = blockIdx.z;

  int L = p.seq_lens[b];
  L = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  const int start = split * p.chunk;
  if (start >= L) return;  // beyond this sequence: nothing to do (the merge skips it)
  const int end = min(start + p.chunk, L);
  const int n_tiles = (end - start + T - 1) / T;

  const unsigned char* __restrict__ kg = static_cast<const unsigned char*>(p.k);
  const unsigned char* __restrict__ vg = static_cast<const unsigned char*>(p.v);

  // ---- direct global -> LDS staging of one tile (K and V) ----
  const size_t seq_base = PAGED ? 0 : ((size_t)b * p.G + grp) * (size_t)p.capacity * ROW_BYTES;
  const int32_t* trow = PAGED ? p.table + (size_t)b * p.max_blocks : nullptr;
  const int pshift = p.page_shift;
  const int pmask = (1 << pshift) - 1;

  // pool page of each 16-row group of a tile (paged caches; scalar loads)
  auto tile_pages = [&](int tile, int* pg) {
#pragma unroll
    for (int gi = 0; gi < C::NGRP; ++gi) {
      const int j = min(start + tile * T + gi * 16, end - 1);
      int page = load_uniform_i32(trow, j >> pshift);
      pg[gi] = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
    }
  };

  auto issue_tile = [&](int tile, const int* pg) {
    unsigned char* st = smem + (tile % NS) * C::STAGE_BYTES;
    const int t0 = start + tile * T;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int qi = n * kThreads + tid;
      const int row = qi / CPR, pch = qi % CPR;
      // rows past the split end re-read its last row: finite data, masked later
      const int j = min(t0 + row, end - 1);
      size_t rb;
      if constexpr (PAGED) {
        const int page = pg[row >> 4];
        rb = (((size_t)page * p.G + grp) * (size_t)(pmask + 1) + (j & pmask)) * ROW_BYTES;
      } else {
        rb = seq_base + (size_t)j * ROW_BYTES;
      }
      const int lds_off = n * kThreads * 16 + wave * 1024;  // this wave's 64 x 16 B slots
      load16_to_lds(kg + rb + ((pch ^ swz_k<CPR>(row)) << 4), st + lds_off);
      load16_to_lds(vg + rb + ((pch ^ swz_v(row)) << 4), st + C::TENSOR_BYTES + lds_off);
    }
  };

  // ---- online-softmax state (per lane: query row l16 of each row tile) ----
  float m_run[RTW], l_run[RTW];
  f32x4 o[RTW][CBW];
  int lim[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) o[rt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int r = (rw * RTW + rt) * 16 + l16;
    r = r < p.R ? r : p.R - 1;
    lim[rt] = p.causal ? (L - p.q_len + r / p.hpg) : (L - 1);  // last visible key
  }
  const int lim_min = p.causal ? (L - p.q_len) : (L - 1);

  // ---- packed query rows of this group, as B operands of S^T = K Q^T ----
  bf16x8 qf[RTW][CC];
  auto load_q = [&]() {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int r = (rw * RTW + rt) * 16 + l16;
      if (r < p.R) {
        const int t = r / p.hpg;
        const int h = grp * p.hpg + (r - t * p.hpg);
        const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((size_t)(b * p.q_len + t) * p.H + h) * D;
#pragma unroll
        for (int cc = 0; cc < CC; ++cc)
          qf[rt][cc] = *reinterpret_cast<const bf16x8*>(qrow + cc * 32 + g4 * 8);
      } else {
#pragma unroll
        for (int cc = 0; cc < CC; ++cc) qf[rt][cc] = bf16x8{};
      }
    }
  };

  // ---- consume one staged tile: S^T = K Q^T, online softmax, O^T += V^T P^T ----
  auto consume = [&](const unsigned char* ks, const unsigned char* vs, const int tile0) {
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
            *reinterpret_cast<const bf16x8*>(ks + row * ROW_BYTES + ((ch ^ swz_k<CPR>(row)) << 4));
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
          s[rt][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][cc], s[rt][kb], 0, 0, 0);
      }
    }

    // online softmax (base 2); P is rounded to bf16 for the PV product and the
    // denominator sums the same rounded weights
    const bool need_mask = (tile0 + T - 1) > lim_min;
    __bf16 pb16[RTW][KB][4];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float x[KB][4];
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = s[rt][kb][i] * p.qk_scale_log2;
          if (need_mask) {
            const int j = tile0 + kw * KW + kb * 16 + g4 * 4 + i;
            v = (j <= lim[rt]) ? v : kNegInf;
          }
          x[kb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = wave_max_across_groups(mx);
      const float m_new = fmaxf(m_run[rt], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 e = (__bf16)__builtin_amdgcn_exp2f(x[kb][i] - m_use);
          pb16[rt][kb][i] = e;
          sum += (float)e;
        }
      l_run[rt] = l_run[rt] * alpha + sum;
      m_run[rt] = m_new;
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) o[rt][cb] *= alpha;
    }

    // O^T += V^T P^T over this wave's output columns
    if constexpr (KB == 1) {
      bf16x4 pb[RTW];
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[rt][i] = pb16[rt][0][i];
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) {
        const int c = (cw * CBW + cb) * 16 + l16;
        uint32_t w[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int r0 = kw * KW + g4 * 4 + 2 * e2;
          const int r1 = r0 + 1;
          const uint32_t lo = lds_u16(vs, r0 * ROW_BYTES + ((((c >> 3) ^ swz_v(r0)) << 4) | ((c & 7) << 1)));
          const uint32_t hi = lds_u16(vs, r1 * ROW_BYTES + ((((c >> 3) ^ swz_v(r1)) << 4) | ((c & 7) << 1)));
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
        // k-slots 8*g4 + e: keys of block 2kp (e < 4) then of block 2kp+1 (e >= 4)
        bf16x8 pb[RTW];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[rt][i] = pb16[rt][2 * kp][i];
            pb[rt][4 + i] = pb16[rt][2 * kp + 1][i];
          }
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) {
          const int c = (cw * CBW + cb) * 16 + l16;
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int blk = 2 * kp + (e2 >> 1);
            const int r0 = kw * KW + blk * 16 + g4 * 4 + 2 * (e2 & 1);
            const int r1 = r0 + 1;
            const uint32_t lo = lds_u16(vs, r0 * ROW_BYTES + ((((c >> 3) ^ swz_v(r0)) << 4) | ((c & 7) << 1)));
            const uint32_t hi = lds_u16(vs, r1 * ROW_BYTES + ((((c >> 3) ^ swz_v(r1)) << 4) | ((c & 7) << 1)));
            w[e2] = lo | (hi << 16);
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt)
            o[rt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], o[rt][cb], 0, 0, 0);
        }
      }
    }
  };

  if constexpr (MODE == kDmaRing) {
    // prologue: tiles 0 .. NS-2 in flight
    {
      int pg[C::NGRP] = {};
#pragma unroll
      for (int tl = 0; tl < NS - 1; ++tl) {
        if (tl < n_tiles) {
          if constexpr (PAGED) tile_pages(tl, pg);
          issue_tile(tl, pg);
        }
      }
    }
    // The query rows are loaded after the prologue's tiles are in flight; one full
    // wait then covers both, so no wait for these registers is left in the loop.
    asm volatile("" ::: "memory");
    load_q();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((7 << 4));  // vmcnt(0) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");

    for (int it = 0; it < n_tiles; ++it) {
      int pg[C::NGRP] = {};
      const bool more = it + NS - 1 < n_tiles;
      if constexpr (PAGED) {
        if (more) tile_pages(it + NS - 1, pg);
      }
      // tiles issued after this one: min(NS - 2, n_tiles - 1 - it)
      const int after = n_tiles - 1 - it;
      if (after >= 2) wait_tile_and_sync<2 * LD>();
      else if (after == 1) wait_tile_and_sync<LD>();
      else wait_tile_and_sync<0>();
      // the stage refilled next was consumed in the previous step by every wave
      if (more) issue_tile(it + NS - 1, pg);
      const unsigned char* ks = smem + (it % NS) * C::STAGE_BYTES;
      consume(ks, ks + C::TENSOR_BYTES, start + it * T);
    }
  } else {
    // Register ring: tile t lives in register set t % P from its load until it is
    // copied into LDS stage t % 2 one step before it is consumed. The compiler places
    // the vector-memory waits for these registers; the workgroup barriers below wait
    // only for LDS, so the other P - 1 tiles stay in flight across them.
    constexpr int P = C::P;
    u32x4 pre[P][LOADS][2];
    auto load_set = [&](int tile, u32x4 (&dst)[LOADS][2]) {
      int pg[C::NGRP] = {};
      if constexpr (PAGED) tile_pages(tile, pg);
      const int t0 = start + tile * T;
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int qi = n * kThreads + tid;
        const int row = qi / CPR, pch = qi % CPR;
        const int j = min(t0 + row, end - 1);  // past the end: re-read the last row (masked)
        size_t rb;
        if constexpr (PAGED) {
          rb = (((size_t)pg[row >> 4] * p.G + grp) * (size_t)(pmask + 1) + (j & pmask)) * ROW_BYTES;
        } else {
          rb = seq_base + (size_t)j * ROW_BYTES;
        }
        dst[n][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kg + rb + ((pch ^ swz_k<CPR>(row)) << 4)));
        dst[n][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + rb + ((pch ^ swz_v(row)) << 4)));
      }
    };
    auto store_set = [&](int stage, const u32x4 (&src)[LOADS][2]) {
      unsigned char* st = smem + stage * C::STAGE_BYTES;
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int off = (n * kThreads + tid) * 16;
        *reinterpret_cast<u32x4*>(st + off) = src[n][0];
        *reinterpret_cast<u32x4*>(st + C::TENSOR_BYTES + off) = src[n][1];
      }
    };

    // One pipeline step: copy tile t + 1 from its register set into LDS, refill the
    // set with tile t + 1 + P, consume tile t. Which of the first two happen is decided
    // by the caller so that the steady-state loop below issues them unconditionally:
    // its register-set schedule is then the same on every iteration and the compiler's
    // vector-memory waits stay exact (they only wait for the set being copied).
    auto step = [&](int t, u32x4 (&set_next)[LOADS][2], bool copy_next, bool refill) {
      if (copy_next) {
        store_set((t + 1) & 1, set_next);
        if (refill) load_set(t + 1 + P, set_next);
      }
      const unsigned char* ks = smem + (t & 1) * C::STAGE_BYTES;
      consume(ks, ks + C::TENSOR_BYTES, start + t * T);
      lds_sync();
    };

    load_q();  // oldest loads: every later wait covers them
    if (n_tiles > P) {
#pragma unroll
      for (int k = 0; k < P; ++k) load_set(k, pre[k]);
      store_set(0, pre[0]);
      load_set(P, pre[0]);
      lds_sync();
      int it = 0;
      for (; it + 2 * P < n_tiles; it += P) {
#pragma unroll
        for (int k = 0; k < P; ++k) step(it + k, pre[(k + 1) % P], true, true);
      }
      // drain: at most 2P steps remain
#pragma unroll
      for (int k = 0; k < 2 * P; ++k) {
        const int t = it + k;
        if (t < n_tiles) step(t, pre[(k + 1) % P], t + 1 < n_tiles, t + 1 + P < n_tiles);
      }
    } else {
      // short split (at most P tiles): load everything, then consume tile by tile
#pragma unroll
      for (int k = 0; k < P; ++k)
        if (k < n_tiles) load_set(k, pre[k]);
#pragma unroll
      for (int k = 0; k < P; ++k) {
        if (k < n_tiles) {
          store_set(k & 1, pre[k]);
          lds_sync();
          const unsigned char* ks = smem + (k & 1) * C::STAGE_BYTES;
          consume(ks, ks + C::TENSOR_BYTES, start + k * T);
          lds_sync();
        }
      }
    }
  }

  // ---- epilogue: per-row totals, cross-wave merge, normalise, write ----
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) l_run[rt] = wave_sum_across_groups(l_run[rt]);

  const size_t rows_per_b = (size_t)p.q_len * p.H;
  auto write_row4 = [&](int r, int c, f32x4 val, float m, float l) {
    // r < R: packed row of this group; c: first of 4 output columns
    const int t = r / p.hpg;
    const int h = grp * p.hpg + (r - t * p.hpg);
    const size_t orow = (size_t)b * rows_per_b + (size_t)t * p.H + h;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    val *= inv;
    if (p.max_splits == 1) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)val[i];
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + orow * D + c) = ov;
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
        for (int cb = 0; cb < CBW; ++cb)
          write_row4(r, (cw * CBW + cb) * 16 + g4 * 4, o[rt][cb], m_run[rt], l_run[rt]);
      }
    }
  } else {
    // Waves with the same rows but different key slices hold partial (max, sum,
    // unnormalised O) for the same rows: merge them through LDS.
    __syncthreads();  // every wave is done with the ring (all its loads were awaited)
    float* red_o = reinterpret_cast<float*>(smem);            // [NKW][ROWS_PAD][D]
    float* red_m = red_o + NKW * C::ROWS_PAD * D;             // [NKW][ROWS_PAD]
    float* red_l = red_m + NKW * C::ROWS_PAD;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int rl = (rw * RTW + rt) * 16 + l16;
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
        *reinterpret_cast<f32x4*>(red_o + ((size_t)kw * C::ROWS_PAD + rl) * D + (cw * CBW + cb) * 16 + g4 * 4) =
            o[rt][cb];
      if (g4 == 0 && cw == 0) {
        red_m[kw * C::ROWS_PAD + rl] = m_run[rt];
        red_l[kw * C::ROWS_PAD + rl] = l_run[rt];
      }
    }
    __syncthreads();
    constexpr int ITEMS = C::ROWS_PAD * D / 4;
    for (int item = tid; item < ITEMS; item += kThreads) {
      const int rl = item / (D / 4);
      const int c = (item % (D / 4)) * 4;
      if (rl >= p.R) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NKW; ++w) M = fmaxf(M, red_m[w * C::ROWS_PAD + rl]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < NKW; ++w) {
        const float f = __builtin_amdgcn_exp2f(red_m[w * C::ROWS_PAD + rl] - Mu);
        l += f * red_l[w * C::ROWS_PAD + rl];
        acc += f * *reinterpret_cast<const f32x4*>(red_o + ((size_t)w * C::ROWS_PAD + rl) * D + c);
      }
      write_row4(rl, c, acc, M, l);
    }
  }
}

template <int D, int NKW, int NRW, int NCW, int RTW, int T, int MODE, int P>
hipError_t launch_variant(const DecodeParams& p, bool paged, dim3 grid, hipStream_t stream) {
  if (paged)
    hipLaunchKernelGGL((decode_mfma_kernel<D, NKW, NRW, NCW, RTW, T, MODE, P, true>), grid, dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, NKW, NRW, NCW, RTW, T, MODE, P, false>), grid, dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

// Wave layouts by packed row count R: X(max R, key slices, row slices, column
// slices, row tiles per wave, keys per stage, register sets).
#define GQA_REG_VARIANTS(X)          \
  X(16, 4, 1, 1, 1, 64, 3)           \
  X(32, 4, 1, 1, 2, 64, 2)           \
  X(64, 2, 2, 1, 2, 32, 6)           \
  X(128, 1, 4, 1, 2, 32, 4)          \
  X(256, 1, 4, 1, 4, 32, 2)
#define GQA_DMA_VARIANTS(X)          \
  X(16, 2, 1, 2, 1, kTile, 0)        \
  X(32, 2, 1, 2, 2, kTile, 0)        \
  X(64, 2, 2, 1, 2, kTile, 0)        \
  X(128, 1, 4, 1, 2, kTile, 0)       \
  X(256, 1, 4, 1, 4, kTile, 0)

template <int D>
hipError_t launch_for_rows(const DecodeParams& p, int staging, bool paged, dim3 grid, hipStream_t stream) {
  if (staging == kRegRing) {
#define X(ROWS, NKW, NRW, NCW, RTW, T, P) \
    if (p.R <= ROWS) return launch_variant<D, NKW, NRW, NCW, RTW, T, kRegRing, P>(p, paged, grid, stream);
    GQA_REG_VARIANTS(X)
#undef X
  } else {
#define X(ROWS, NKW, NRW, NCW, RTW, T, P) \
    if (p.R <= ROWS) return launch_variant<D, NKW, NRW, NCW, RTW, T, kDmaRing, P>(p, paged, grid, stream);
    GQA_DMA_VARIANTS(X)
#undef X
  }
  return hipErrorInvalidValue;
}

template <int D>
MfmaVariant variant_for(int R, int staging) {
  if (staging == kRegRing) {
#define X(ROWS, NKW, NRW, NCW, RTW, T, P) \
    if (R <= ROWS) return MfmaVariant{ROWS, T, MfmaCfg<D, NKW, NRW, NCW, RTW, T, kRegRing, P>::LDS_BYTES};
    GQA_REG_VARIANTS(X)
#undef X
  } else {
#define X(ROWS, NKW, NRW, NCW, RTW, T, P) \
    if (R <= ROWS) return MfmaVariant{ROWS, T, MfmaCfg<D, NKW, NRW, NCW, RTW, T, kDmaRing, P>::LDS_BYTES};
    GQA_DMA_VARIANTS(X)
#undef X
  }
  return MfmaVariant{0, kTile, 0};
}

}  // namespace

MfmaVariant mfma_variant_for_rows(int R, int d_h, int staging) {
  return d_h == 64 ? variant_for<64>(R, staging) : variant_for<128>(R, staging);
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int d_h, bool paged, dim3 grid,
                              hipStream_t stream) {
  (void)dtype;  // bf16 only (checked by the planner)
  if (d_h == 64) return launch_for_rows<64>(p, p.staging, paged, grid, stream);
  return launch_for_rows<128>(p, p.staging, paged, grid, stream);
}

}  // namespace gqa
