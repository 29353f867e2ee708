// Measurement helper: the plain streaming-read rate of device memory, the ceiling a
// decode step that re-reads its whole KV cache can approach (the bandwidth-wall
// section of the llms.blog GQA/MQA page).

#include <cstdint>

#include "../../include/gqa_bench.h"
#include "../../include/gqa_decode.h"
#include <hip/hip_runtime.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kBlocks = 8192;
constexpr int kThreads = 256;
constexpr int kUnroll = 16;

// Each workgroup streams one contiguous slice with kUnroll nontemporal 16-byte loads in
// flight per thread (the pattern that reached the highest rate in our measurements).
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  constexpr size_t step = (size_t)kThreads * kUnroll;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t base = lo;
  for (; base + step <= hi; base += step) {
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = __builtin_nontemporal_load(buf + base + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= w[u][0] ^ w[u][1] ^ w[u][2] ^ w[u][3];
  }
  for (size_t i = base + threadIdx.x; i < hi; i += kThreads) {
    const u32x4 w = buf[i];
    acc ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// The decode kernel's own streaming pattern without its compute: two persistent
// workgroups per CU, each reading one contiguous share of the buffer in steps of
// direct-to-LDS loads (16 KiB = four 16-byte loads per lane, as a K + V tile of the
// 128-wide kernels; 32 KiB = eight, as a tile of the 512-wide latent), one step in
// flight while the wave issues the next. The LDS copies are not read.

__device__ __forceinline__ void dma16(const unsigned char* src, unsigned char* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 2);
#else
  (void)src;
  (void)lds_wave_base;
#endif
}

template <int kStepChunks>  // 16-byte loads per lane per step
__global__ __launch_bounds__(kThreads) void read_stream_lds_kernel(const unsigned char* __restrict__ buf, size_t n16) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][kStepChunks * kThreads * 16];
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  const int wave = threadIdx.x >> 6;
  int stage = 0;
  for (size_t base = lo; base < hi; base += (size_t)kStepChunks * kThreads) {
#pragma unroll
    for (int u = 0; u < kStepChunks; ++u) {
      const size_t i = base + (size_t)u * kThreads + threadIdx.x;
      if (i < hi) dma16(buf + i * 16, &lds[stage][u * kThreads * 16 + wave * 1024]);
    }
    // at most this step's loads stay in flight: vmcnt(kStepChunks), expcnt and lgkmcnt untouched
    __builtin_amdgcn_s_waitcnt((kStepChunks & 15) | (7 << 4) | (15 << 8));
    stage ^= 1;
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
}

}  // namespace

extern "C" int gqa_bench_read_stream_lds(const void* buf, size_t bytes, int workgroups, int step_bytes,
                                         void* stream) {
  if (!buf || bytes == 0 || (bytes % 16) != 0 || workgroups <= 0 || workgroups > (1 << 20))
    return GQA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0) return GQA_ERR_INVALID_ARGUMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned char* b = static_cast<const unsigned char*>(buf);
  if (step_bytes == 16384)
    hipLaunchKernelGGL(read_stream_lds_kernel<4>, dim3(workgroups), dim3(kThreads), 0, s, b, bytes / 16);
  else if (step_bytes == 32768)
    hipLaunchKernelGGL(read_stream_lds_kernel<8>, dim3(workgroups), dim3(kThreads), 0, s, b, bytes / 16);
  else
    return GQA_ERR_INVALID_ARGUMENT;
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

extern "C" int gqa_bench_read_stream(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || (bytes % 16) != 0) return GQA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(sink) % 4) != 0)
    return GQA_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(read_stream_kernel, dim3(kBlocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}
