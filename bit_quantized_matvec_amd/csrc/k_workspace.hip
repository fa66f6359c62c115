// k_workspace.hip -- zero-fill of a product workspace with a kernel.
//
// The split products keep per-tile arrival counters in the workspace and
// return them to zero at the end of every call (k_gemv_pq2.hip,
// k_gemv_ptq1.hip).  A workspace whose state is unknown -- never cleared, or
// shared by calls that overlapped -- is restored by this fill.  It is a
// kernel rather than hipMemsetAsync, so a caller may capture it in a graph.
#include <algorithm>

#include "kernels.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

// 16-byte stores over the whole 16-byte words, then single bytes for a tail;
// grid-stride, so any size launches with a bounded grid.
__global__ __launch_bounds__(kThreads) void clear_kernel(uint4* __restrict__ p, int64_t nwords, uint8_t* __restrict__ tail,
                                                         int ntail) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nwords; i += stride) p[i] = uint4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_clear(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  const int64_t nwords = bytes / 16;
  const int ntail = (int)(bytes % 16);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((nwords + kThreads - 1) / kThreads, 4096));
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, static_cast<uint4*>(p), nwords,
                     static_cast<uint8_t*>(p) + nwords * 16, ntail);
  return hipGetLastError();
}

}  // namespace tq
