// scratch.hip -- the library's own device scratch for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc): tq_gemv_f32_scratch runs the fused matrix-vector product
// with its column-split workspace in this file-scope array instead of a
// caller buffer.
//
// `scratch` is a static __device__ array.  In host code its name is only a
// host-side stand-in, so it is never passed to a kernel: the first call on a
// device looks up that device's copy with hipGetSymbolAddress (with the device
// current) and keeps the address per device; only that address is used
// afterwards.  Each GPU holds its own copy until the process ends.  Every call
// on a GPU shares the array: calls that overlap on one GPU race (their tile
// counters and partial sums collide).
#include <mutex>

#include "kernels.h"

namespace tq {

// The column split only happens below 384 row tiles (plan_gemv_pq2), so 384
// workspace blocks cover every shape the fused product accepts: 6,297,600 B.
constexpr int64_t kScratchBytes = 384 * kWsTileBytes;

namespace {

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int64_t scratch_bytes() { return kScratchBytes; }

// Device address of this device's scratch; on the first call for a device it
// is looked up and the scratch is zero-filled on `s` (a kernel, so the call
// may be captured), which leaves every tile counter at zero as the split
// product requires.  Returns hipSuccess or the HIP error of the lookup.
hipError_t scratch_ptr(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    e = launch_clear(p, kScratchBytes, s);
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
