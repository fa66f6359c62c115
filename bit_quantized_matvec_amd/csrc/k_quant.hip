// k_quant.hip -- q8_K activation quantizer.
//
// q8_K (ciot README, intro; page 1 "the paperwork"): per block of 256 values,
// d = max|x| / 127, q = round-to-nearest-even(x / d), and 16 partial sums of
// 16 consecutive q.  One wave64 owns one block: each lane loads 4 floats (one
// dwordx4, so the wave reads the block as one coalesced 1 KiB request); the
// block arithmetic (q8k_block.h) is shared with the matrix-vector kernel that
// quantizes its own activations; the partial sums are 4-lane butterfly adds.
#include <algorithm>

#include "kernels.h"
#include "q8k_block.h"

namespace tq {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(64 * kWavesPerBlock) void quantize_q8k_kernel(const float4* __restrict__ x, int64_t nblocks,
                                                                           int* __restrict__ q, float* __restrict__ d,
                                                                           int16_t* __restrict__ bsums) {
  const int lane = threadIdx.x & 63;
  // grid-stride over q8_K blocks, one wave per block at a time: whole waves
  // leave the loop together
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t blk = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); blk < nblocks; blk += stride) {
    const float4 v[1] = {x[blk * 64 + lane]};
    float dv[1];
    int pv[1];
    q8k_quant_batch<1>(v, dv, pv);
    const float db = dv[0];
    const int packed = pv[0];
    q[blk * 64 + lane] = packed;
    int s = (int)(int8_t)packed + (int)(int8_t)(packed >> 8) + (int)(int8_t)(packed >> 16) + (int)(int8_t)(packed >> 24);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if ((lane & 3) == 0) bsums[blk * 16 + (lane >> 2)] = (int16_t)s;
    if (lane == 0) d[blk] = db;
  }
}

}  // namespace

hipError_t launch_quantize_q8k(const float* x, int64_t nblocks, int8_t* q, float* d, int16_t* bsums, hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  // at most 2^20 workgroups (2^28 work-items); larger inputs loop
  const int64_t grid = std::min<int64_t>((nblocks + kWavesPerBlock - 1) / kWavesPerBlock, int64_t(1) << 20);
  hipLaunchKernelGGL(quantize_q8k_kernel, dim3((unsigned)grid), dim3(64 * kWavesPerBlock), 0, s,
                     reinterpret_cast<const float4*>(x), nblocks, reinterpret_cast<int*>(q), d, bsums);
  return hipGetLastError();
}

}  // namespace tq
