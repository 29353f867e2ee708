// Device helpers shared by the matrix-core decode kernels: vector types, wave-level
// reductions over the lanes that share a query row of an MFMA result, the ring's
// waits, the LDS swizzles of staged K/V rows, direct global->LDS loads and the LDS
// operand reads that feed the matrix cores.
#pragma once

#include "gqa_internal.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kTile = 32;        // keys per pipeline stage
[[maybe_unused]] constexpr int kNontemporal = 2;  // cache-policy bit for streaming loads
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (factor 2^8)
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// Lanes l, l^16, l^32 and l^48 hold the same query row of an MFMA result. On gfx950
// v_permlane32_swap(x, x) leaves {x[l], x[l^32]} in each lane and
// v_permlane16_swap(x, x) leaves {x[l], x[l^16]} (checked with an in-bounds probe),
// so two VALU swaps reduce across the four lanes without a trip through LDS.
__device__ __forceinline__ float wave_max_across_groups(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
#else
  return x;
#endif
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_sum_across_groups(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
#else
  return x;
#endif
}

// Wait until at most N vector-memory operations of this wave are outstanding and all
// of its LDS operations are done, then synchronise the workgroup. The direct-to-LDS
// loads are tracked by the vector-memory counter (in issue order), so after this
// every wave's loads of the awaited tile have landed in LDS.
template <int N>
__device__ __forceinline__ void wait_vm_and_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4);  // vmcnt(N) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for the oldest staged tile when `after` later tiles (at most K) may stay in
// flight, each LD loads per wave.
template <int LD, int K>
__device__ __forceinline__ void wait_tiles(int after) {
  if constexpr (K == 0) {
    wait_vm_and_sync<0>();
  } else {
    if (after >= K) wait_vm_and_sync<K * LD>();
    else wait_tiles<LD, K - 1>(after);
  }
}

// LDS swizzles (16-byte chunk index XOR a function of the row) so that the QK
// A-operand reads (16 consecutive key rows, one chunk each) and the transposed V
// reads (16 consecutive key rows, the same two chunks each) spread over the banks.
// When one staged tile serves as both K and V (the latent cache, SHARED), a single
// swizzle must suit both reads: rotating the row's low four bits left by one maps 16
// consecutive rows onto all 16 chunk positions (the K reads) and any 8 aligned rows
// onto 8 distinct chunk pairs (the transposed reads).
__device__ __forceinline__ int swz_rot4(int row) { return ((row << 1) & 14) | ((row >> 3) & 1); }
template <int CPR, bool SHARED>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (SHARED) return swz_rot4(row);
  else return row & (CPR - 1);
}
template <int CPR, bool SHARED>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (SHARED) return swz_rot4(row);
  else return (row << 1) & (CPR - 2);
}

// One 16-byte direct global->LDS load per lane (nontemporal unless POLICY says
// otherwise): lane i of the wave writes LDS bytes [lds_wave_base + 16 i, +16).
// Device-only: the host pass of this translation unit must not see the builtin (it
// would drop the kernel stubs).
template <int POLICY = kNontemporal>
__device__ __forceinline__ void load16_to_lds(const unsigned char* src, unsigned char* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)lds_wave_base, 16, 0, POLICY);
#else
  (void)src;
  (void)lds_wave_base;
#endif
}

// Transposed 64-bit LDS reads (ds_read_b64_tr_b16). Within each 16-lane group, lane
// i receives as element e the 16-bit element i % 4 of the 8 bytes addressed by lane
// 4e + i / 4 of the group (measured on gfx950 with an in-bounds probe).
//
// They are issued from asm blocks that also wait for their own results, so every
// output register holds its data when the block ends. Issued through the builtin
// instead, the compiler cannot rule out that the read aliases a direct-to-LDS load
// still in flight and drains all of them (vmcnt(0)) before it, which leaves only the
// tile being consumed in flight. The ring's own wait and barrier already order these
// reads after the loads of the tile they read.
//
// One column block: rows r (address a) and r + 16 (a + HI) of the same columns.
template <int HI>
__device__ __forceinline__ void lds_read_tr16_x2(unsigned a, bf16x4& lo, bf16x4& hi) {
  static_assert(HI > 0 && HI < 65536, "LDS offset field");
#if defined(__HIP_DEVICE_COMPILE__)
  u32x2 x, y;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y)
      : "v"(a), "i"(HI)
      : "memory");
  lo = __builtin_bit_cast(bf16x4, x);
  hi = __builtin_bit_cast(bf16x4, y);
#else
  (void)a;
  lo = hi = bf16x4{};
#endif
}

// Two column blocks at addresses a and b.
template <int HI>
__device__ __forceinline__ void lds_read_tr16_x4(unsigned a, unsigned b, bf16x4& lo0, bf16x4& hi0,
                                                 bf16x4& lo1, bf16x4& hi1) {
  static_assert(HI > 0 && HI < 65536, "LDS offset field");
#if defined(__HIP_DEVICE_COMPILE__)
  u32x2 x0, y0, x1, y1;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(y0), "=&v"(x1), "=&v"(y1)
      : "v"(a), "v"(b), "i"(HI)
      : "memory");
  lo0 = __builtin_bit_cast(bf16x4, x0);
  hi0 = __builtin_bit_cast(bf16x4, y0);
  lo1 = __builtin_bit_cast(bf16x4, x1);
  hi1 = __builtin_bit_cast(bf16x4, y1);
#else
  (void)a;
  (void)b;
  lo0 = hi0 = lo1 = hi1 = bf16x4{};
#endif
}

// Four column blocks at addresses a[0..3]: all eight reads, then one wait.
template <int HI>
__device__ __forceinline__ void lds_read_tr16_x8(const unsigned (&a)[4], u32x2 (&v)[4][2]) {
  static_assert(HI > 0 && HI < 65536, "LDS offset field");
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[2][0]), "=&v"(v[2][1]),
        "=&v"(v[3][0]), "=&v"(v[3][1])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(HI)
      : "memory");
#else
  (void)a;
  for (auto& x : v) x[0] = x[1] = u32x2{};
#endif
}

// Plain 16-byte LDS reads of rows r (address a[i]) and r + 16 (a[i] + HI) for N
// addresses, N = 2 or 4, all issued before one wait, for the same reason as the
// transposed reads.
template <int N, int HI>
__device__ __forceinline__ void lds_read_b128_rows(const unsigned (&a)[N], u32x4 (&v)[N][2]) {
  static_assert(N == 2 || N == 4, "two or four addresses");
  static_assert(HI > 0 && HI < 65536, "LDS offset field");
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %5\n\t"
        "ds_read_b128 %3, %5 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1])
        : "v"(a[0]), "v"(a[1]), "i"(HI)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:%12\n\t"
        "ds_read_b128 %2, %9\n\t"
        "ds_read_b128 %3, %9 offset:%12\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %10 offset:%12\n\t"
        "ds_read_b128 %6, %11\n\t"
        "ds_read_b128 %7, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[2][0]), "=&v"(v[2][1]),
          "=&v"(v[3][0]), "=&v"(v[3][1])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(HI)
        : "memory");
  }
#else
  (void)a;
  for (auto& x : v) x[0] = x[1] = u32x4{};
#endif
}

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const unsigned char* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return (unsigned)(uintptr_t)(LDS_AS const unsigned char*)p;
#else
  return (unsigned)(uintptr_t)p;
#endif
}

// Read-only int32 data through the constant address space: wave-uniform reads become
// scalar loads, which the direct-to-LDS loads in flight cannot delay (a vector load
// would have to wait for all of them: the vector-memory counter is in order).
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* base, int idx) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(4))) int32_t*)base)[idx];
#else
  return base[idx];
#endif
}

__device__ __forceinline__ int clamp_len(int L, int capacity) {
  return L < 1 ? 1 : (L > capacity ? capacity : L);
}

// The persistent schedule's view for workgroup w. The (sequence, group, row block)
// segments, cut into tiles of T keys, lie end to end: sequence b contributes GS =
// G * n_row_blocks consecutive segments of n_b = ceil(L_b / T) tiles each. Workgroup w
// of nwg takes the tiles [lo, lo + count) with lo = floor(w W / nwg). Every wave scans
// seq_lens (a few hundred bytes) on its own, with cross-lane operations only (no LDS,
// no barrier), to find the total W and the sequence b holding tile lo (pre: the tiles
// before b's segments, L: its clamped length); `publish` (one wave of one workgroup)
// also writes the per-sequence prefix sums ws_prefix[0..B] for the merge kernel. All
// results are wave-uniform.
struct ScheduleStart {
  int lo, count;  // this workgroup's tile range
  int b, pre, L;  // the sequence holding tile lo (b = -1: none)
  int W;          // tiles in all
};

__device__ __forceinline__ ScheduleStart schedule_start(const DecodeParams& p, int T, int w, bool publish) {
  const int lane = threadIdx.x & 63;
  const int L0 = lane < p.B ? clamp_len(p.seq_lens[lane], p.capacity) : 0;
  int total = wave_sum_i32(L0 > 0 ? (L0 + T - 1) / T : 0);
  for (int b0 = 64; b0 < p.B; b0 += 64) {
    const int bb = b0 + lane;
    total += wave_sum_i32(bb < p.B ? (clamp_len(p.seq_lens[bb], p.capacity) + T - 1) / T : 0);
  }
  const int GS = p.G * p.n_row_blocks;  // segments per sequence
  const int W = GS * __builtin_amdgcn_readfirstlane(total);  // the planner bounds it to fit int32
  const int lo = (int)(((long long)w * W) / p.nwg);
  const int hi = (int)(((long long)(w + 1) * W) / p.nwg);
  int b_start = -1, pre_start = 0, L_start = 1;
  int carry = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int bb = b0 + lane;
    const int L = b0 == 0 ? L0 : (bb < p.B ? clamp_len(p.seq_lens[bb], p.capacity) : 0);
    const int gn = L > 0 ? GS * ((L + T - 1) / T) : 0;
    const int incl = carry + wave_incl_scan_i32(gn);
    const int excl = incl - gn;
    if (publish && bb < p.B) p.ws_prefix[bb] = excl;
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(L > 0 && lo >= excl && lo < incl);
    if (hit) {
      const int j = __builtin_ctzll(hit);
      b_start = b0 + j;
      pre_start = __builtin_amdgcn_readlane(excl, j);
      L_start = __builtin_amdgcn_readlane(L, j);
      if (!publish) break;
    }
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  if (publish && lane == 0) p.ws_prefix[p.B] = W;
  // wave-uniform by construction; say so, so that everything derived from the cursor
  // stays in scalar registers (and the table reads stay scalar loads)
  ScheduleStart r;
  r.lo = __builtin_amdgcn_readfirstlane(lo);
  r.count = __builtin_amdgcn_readfirstlane(hi - lo);
  r.b = __builtin_amdgcn_readfirstlane(b_start);
  r.pre = __builtin_amdgcn_readfirstlane(pre_start);
  r.L = __builtin_amdgcn_readfirstlane(L_start);
  r.W = W;
  return r;
}

}  // namespace
}  // namespace gqa
