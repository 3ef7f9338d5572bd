// Optional page-id range check, run ahead of the attention kernels.
//
// rocm-libraries "one K/V resource per page on the gfx942 2D i64 path" (Not in
// this PR; review, LOW findings): page ids are bounded by slot index only and
// are never compared with the cache's page count before they form a page
// base, and that comparison needs the page count as a kernel argument.  This
// pass makes the comparison for every id a sequence will read, before any of
// them is dereferenced.  A sequence that fails (an id outside [0, num_pages),
// or a length outside [0, width * page_size], which would push the slot index
// past its row) is handed to the attention kernels with length 0, so its rows
// come out empty (0, -inf) and none of its ids is ever used as an address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCheckWaves = 4;
constexpr int kFirstThreads = 1024;

// One wave per sequence: lanes read the sequence's used slots 64 at a time.
__global__ __launch_bounds__(kCheckWaves * 64) void page_check_kernel(
    const int32_t* __restrict__ table, int64_t bt_stride, const int32_t* __restrict__ lens,
    int batch, int width, int page_size, int64_t num_pages, int32_t* __restrict__ result) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kCheckWaves + static_cast<int>(threadIdx.x >> 6);
  if (b >= batch) return;
  const int len = lens[b];
  bool ok = len >= 0 && static_cast<int64_t>(len) <= static_cast<int64_t>(width) * page_size;
  if (ok) {
    const int n = (len + page_size - 1) / page_size;
    const int32_t* row = table + static_cast<int64_t>(b) * bt_stride;
    bool bad = false;
#pragma unroll 4
    for (int s = lane; s < n; s += 64) {
      const int32_t id = row[s];
      bad |= id < 0 || static_cast<int64_t>(id) >= num_pages;
    }
    ok = __ballot(bad) == 0;
  }
  if (lane == 0) result[1 + b] = ok ? len : 0;
}

// One workgroup: the smallest b whose attended length differs from its
// length (only a failing sequence can differ: it was given 0 and read >= 1
// slot, or its length was out of range), or -1.
__global__ __launch_bounds__(kFirstThreads) void page_check_first_kernel(
    const int32_t* __restrict__ lens, int batch, int32_t* __restrict__ result) {
  __shared__ int first;
  if (threadIdx.x == 0) first = INT32_MAX;
  __syncthreads();
  int mine = INT32_MAX;
  for (int b = threadIdx.x; b < batch; b += kFirstThreads) {
    if (result[1 + b] != lens[b]) {
      mine = b;
      break;
    }
  }
  if (mine != INT32_MAX) atomicMin(&first, mine);
  __syncthreads();
  if (threadIdx.x == 0) result[0] = first == INT32_MAX ? -1 : first;
}

}  // namespace

hipError_t launch_page_check(const int32_t* block_table, int64_t bt_stride,
                             const int32_t* seq_lens, int batch, int width, int page_size,
                             int64_t num_pages, int32_t* result, hipStream_t stream) {
  const int blocks = (batch + kCheckWaves - 1) / kCheckWaves;
  hipLaunchKernelGGL(page_check_kernel, dim3(blocks), dim3(kCheckWaves * 64), 0, stream,
                     block_table, bt_stride, seq_lens, batch, width, page_size, num_pages,
                     result);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(page_check_first_kernel, dim3(1), dim3(kFirstThreads), 0, stream, seq_lens,
                     batch, result);
  return hipGetLastError();
}

}  // namespace pa
