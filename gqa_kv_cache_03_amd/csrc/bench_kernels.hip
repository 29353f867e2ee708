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

}  // namespace

extern "C" int gqa_bench_read_stream(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || (bytes % 16) != 0) return GQA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(sink) % 4) != 0)
    return GQA_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(read_stream_kernel, dim3(kBlocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}
