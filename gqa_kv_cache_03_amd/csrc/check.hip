// Device-side check of the preconditions that live in device memory and that the
// decode calls document but do not verify on their fast path: every sequence length
// lies in [q_len, capacity], and every block-table entry a step reads (entry k of
// sequence b for k < ceil(seq_lens[b] / P)) names a pool page in [0, num_pages).
// A paged cache keeps each sequence's rows in fixed-size blocks found through the
// table (llms.blog GQA/MQA page, "PagedAttention"); a stray entry there is the one
// caller mistake that makes a kernel read memory it does not own, which this check
// reports instead.
//
// report (device int32[4]): [0] sequences with a bad length, [1] bad table entries
// among those read, [2] the first bad sequence, [3] the first bad entry as
// b * max_blocks + k (INT32_MAX in [2], [3] when there is none). A length outside
// [q_len, capacity] is counted, and its table row is then checked up to the clamped
// length the kernels would use.

#include <limits.h>

#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(64) void check_init_kernel(int32_t* report) {
  const int i = threadIdx.x;
  if (i < 4) report[i] = i < 2 ? 0 : INT_MAX;
}

// One workgroup per sequence: thread 0 checks the length, all threads the table row.
__global__ __launch_bounds__(kThreads) void check_inputs_kernel(CheckParams p) {
  const int b = blockIdx.x;
  const int L = p.seq_lens[b];
  if (threadIdx.x == 0 && (L < p.q_len || L > p.capacity)) {
    atomicAdd(p.report + 0, 1);
    atomicMin(p.report + 2, b);
  }
  if (!p.table) return;
  const int Lc = L < 1 ? 1 : (L > p.capacity ? p.capacity : L);
  const int n = (Lc + p.page_size - 1) / p.page_size;
  const int32_t* row = p.table + (size_t)b * p.max_blocks;
  for (int k = threadIdx.x; k < n; k += kThreads) {
    const int page = row[k];
    if (page < 0 || page >= p.num_pages) {
      atomicAdd(p.report + 1, 1);
      atomicMin(p.report + 3, b * p.max_blocks + k);
    }
  }
}

}  // namespace

hipError_t launch_check_inputs(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, p.report);
  if (p.B > 0) hipLaunchKernelGGL(check_inputs_kernel, dim3(p.B), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
