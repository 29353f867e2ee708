// Cache append for the vector-ALU decode path: write the q_len new tokens' K and V
// rows into the cache before the decode kernel reads it. A decode step appends its
// tokens' keys and values to the cache and then attends over all of it ("The KV-Cache
// Bandwidth Wall", llms.blog GQA/MQA page); in a paged cache the row of position pos
// is slot pos % P of page block_table[b][pos / P] ("PagedAttention", same page).
//
// One thread per 16-byte chunk of a (sequence, token, group) row; the matrix-core
// path does this inside its decode kernel instead.

#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

template <bool PAGED>
__global__ __launch_bounds__(kThreads) void append_kernel(DecodeParams p, int row_bytes) {
  const int cpr = row_bytes / 16;
  const long long total = (long long)p.B * p.q_len * p.G * cpr;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int ch = (int)(i % cpr);
  long long rest = i / cpr;
  const int g = (int)(rest % p.G);
  rest /= p.G;
  const int t = (int)(rest % p.q_len);
  const int b = (int)(rest / p.q_len);
  int L = p.seq_lens[b];
  L = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  const int pos = L - p.q_len + t;
  if (pos < 0) return;  // outside the documented precondition q_len <= seq_lens[b]

  const size_t src = (((size_t)b * p.q_len + t) * p.G + g) * row_bytes + (size_t)ch * 16;
  size_t dst;
  if constexpr (PAGED) {
    int page = p.table[(size_t)b * p.max_blocks + (pos >> p.page_shift)];
    page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
    const int P = 1 << p.page_shift;
    dst = (((size_t)page * p.G + g) * P + (pos & (P - 1))) * row_bytes;
  } else {
    dst = (((size_t)b * p.G + g) * p.capacity + pos) * row_bytes;
  }
  dst += (size_t)ch * 16;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.k_new) + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.v_new) + src);
  // the caches are writable in append mode (the public entry point takes them non-const)
  *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(const_cast<void*>(p.k)) + dst) = kv;
  *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(const_cast<void*>(p.v)) + dst) = vv;
}

}  // namespace

hipError_t launch_append(const DecodeParams& p, int elem_bytes, int d_h, bool paged, hipStream_t stream) {
  const int row_bytes = d_h * elem_bytes;
  const long long total = (long long)p.B * p.q_len * p.G * (row_bytes / 16);
  const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
  if (paged)
    hipLaunchKernelGGL(append_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, p, row_bytes);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, p, row_bytes);
  return hipGetLastError();
}

}  // namespace gqa
