// k_quant.hip -- q8_K activation quantizer.
//
// q8_K (ciot README, intro; page 1 "the paperwork"): per block of 256 values,
// d = max|x| / 127, q = round-to-nearest-even(x / d), and 16 partial sums of
// 16 consecutive q.  One wave64 owns one block: each lane loads 4 floats (one
// dwordx4, so the wave reads the block as one coalesced 1 KiB request), the
// block maximum is a butterfly max-reduction across the wave, and the
// partial sums are 4-lane butterfly adds.  The divisions are IEEE fp32
// (correctly rounded; this file must not be built with fast-math), and
// rintf lowers to v_rndne_f32, so the result is bit-identical to a scalar
// reference.
#include "kernels.h"

namespace tq {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ int quant1(float x, float d) {
  if (d == 0.0f) return 0;
  float r = rintf(x / d);
  r = fminf(127.0f, fmaxf(-127.0f, r));
  return (int)r;
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void quantize_q8k_kernel(const float4* __restrict__ x, int64_t nblocks,
                                                                           int* __restrict__ q, float* __restrict__ d,
                                                                           int16_t* __restrict__ bsums) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // whole waves leave together
  const float4 v = x[blk * 64 + lane];
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  const float db = a / 127.0f;
  const int q0 = quant1(v.x, db), q1 = quant1(v.y, db), q2 = quant1(v.z, db), q3 = quant1(v.w, db);
  q[blk * 64 + lane] = (q0 & 0xff) | ((q1 & 0xff) << 8) | ((q2 & 0xff) << 16) | ((q3 & 0xff) << 24);
  int s = q0 + q1 + q2 + q3;
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  if ((lane & 3) == 0) bsums[blk * 16 + (lane >> 2)] = (int16_t)s;
  if (lane == 0) d[blk] = db;
}

}  // namespace

hipError_t launch_quantize_q8k(const float* x, int64_t nblocks, int8_t* q, float* d, int16_t* bsums, hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(quantize_q8k_kernel, dim3((unsigned)grid), dim3(64 * kWavesPerBlock), 0, s,
                     reinterpret_cast<const float4*>(x), nblocks, reinterpret_cast<int*>(q), d, bsums);
  return hipGetLastError();
}

}  // namespace tq
