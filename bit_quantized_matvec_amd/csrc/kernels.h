// kernels.h -- host-side launchers of the HIP kernels (internal to libtq).
// Arguments are validated by the C-ABI layer before any launcher runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace tq {

// Split of a matrix-vector product over workgroups: `slices` column slices per
// 64-row tile of `scw` superchunks (or 8-group superblocks for ptq1_0) each,
// `waves` waves per workgroup taking runs of `spw`.
struct GemvPlan {
  int slices, scw, waves, spw;
};
constexpr int kMaxSlices = 16;
// s_waitcnt immediate for "vmcnt(0)" on gfx9-family targets (vmcnt in bits
// 3:0 and 15:14 = 0; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int kWaitVmcnt0 = 0x0F70;

// Workspace of the split products: one block of kWsTileBytes per 64-row
// tile (the global tile index of a batch), at the same place for every shape,
// format and entry point, so that one workspace serves any later call whose
// tiles it covers: the tile's arrival counter (zero between calls; 16 bytes
// with padding), then room for 32 x 64 fp64 partial sums -- [slice][row] for
// pq2_0 (up to 16 slices), [superblock][row] for ptq1_0 (up to 32).
constexpr int64_t kWsTileBytes = 16 + 32 * 64 * 8;
__host__ __device__ inline unsigned* ws_counter(uint8_t* ws, int64_t tile) {
  return reinterpret_cast<unsigned*>(ws + tile * kWsTileBytes);
}
__host__ __device__ inline double* ws_partials(uint8_t* ws, int64_t tile) {
  return reinterpret_cast<double*>(ws + tile * kWsTileBytes + 16);
}
inline int64_t workspace_bytes(const Dims& d) { return d.ntiles * kWsTileBytes; }

// Zero `bytes` bytes at p (16-byte aligned) with a kernel (graph-capturable).
hipError_t launch_clear(void* p, int64_t bytes, hipStream_t s);

hipError_t launch_quantize_q8k(const float* x, int64_t nblocks, int8_t* q, float* d, int16_t* bsums, hipStream_t s);

hipError_t launch_repack_pq2(const uint8_t* src, uint8_t* dst, const Dims& dm, int32_t* bad_flag, hipStream_t s);
hipError_t launch_unrepack_pq2(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s);
hipError_t launch_repack_ptq1(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s);
hipError_t launch_unrepack_ptq1(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s);

// y[rows] (fp32) or, if idots != nullptr, the int32 group dots [rows][G].
// With a workspace (workspace_bytes, zeroed before first use) the columns are
// split over several workgroups per tile; without one, one workgroup per tile.
GemvPlan plan_gemv_pq2(const Dims& dm, bool have_workspace);
hipError_t launch_gemv_pq2_plan(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, float* y,
                                int32_t* idots, void* workspace, const GemvPlan& p, hipStream_t s);
hipError_t launch_gemv_pq2(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, void* workspace, hipStream_t s);
// The same product from fp32 activations x [cols]: every workgroup quantizes
// its slice of x to q8_K in LDS (bit-identical to launch_quantize_q8k) and
// multiplies.  Possible when one slice's q8_K fits the LDS stage.
bool gemv_pq2_fused_fits(const Dims& dm, bool have_workspace);

// Independent fused products sharing one column count, launched together:
// problem m covers workgroups [tile0[m], tile0[m + 1]).
constexpr int kMaxBatch = 4;
struct GemvBatch {
  const uint4* codes[kMaxBatch];
  const uint32_t* scales[kMaxBatch];
  const float4* x[kMaxBatch];
  float* y[kMaxBatch];
  int rows[kMaxBatch];
  int tile0[kMaxBatch + 1];
  int n;
};
// `dm` describes the whole batch: ntiles = tile0[n], cols the common count
hipError_t launch_gemv_pq2_fused_batch(const GemvBatch& b, const Dims& dm, void* workspace, hipStream_t s);
// The library's static device scratch (scratch.hip): its size, and this
// device's address (looked up and zero-filled on `s` at the first call).
int64_t scratch_bytes();
hipError_t scratch_ptr(hipStream_t s, void** out);
hipError_t launch_gemv_pq2_fused(const uint8_t* w, const Dims& dm, const float* x, float* y, void* workspace,
                                 hipStream_t s);
GemvPlan plan_gemv_ptq1(const Dims& dm, bool have_workspace);
hipError_t launch_gemv_ptq1_plan(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx,
                                 const int16_t* bsums, float* y, int32_t* idots, void* workspace, const GemvPlan& p,
                                 hipStream_t s);
hipError_t launch_gemv_ptq1(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx,
                            const int16_t* bsums, float* y, int32_t* idots, void* workspace, hipStream_t s);
// Several tokens: y[tokens][rows] or idots [tokens][rows][G], each token
// bit-identical to launch_gemv_ptq1 without a workspace.
int ptq1_token_block(const Dims& dm, int64_t tokens);
hipError_t launch_gemm_ptq1(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx,
                            const int16_t* bsums, float* y, int32_t* idots, hipStream_t s);
// The same on int8 MFMA: 16 tokens x one 64-row tile per workgroup.
hipError_t launch_gemm_ptq1_mfma(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx,
                                 const int16_t* bsums, float* y, int32_t* idots, hipStream_t s);
// y[tokens][rows] or idots [tokens][rows][G].
hipError_t launch_gemm_pq2(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx,
                           float* y, int32_t* idots, hipStream_t s);

}  // namespace tq
