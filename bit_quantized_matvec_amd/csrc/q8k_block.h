// q8k_block.h -- the q8_K arithmetic of one 256-value block held by a wave64
// (4 consecutive values per lane), shared by the standalone quantizer and the
// matrix-vector kernel that quantizes its own activations, so that both
// produce the same bits.
//
// q8_K (ciot README, intro; page 1 "the paperwork"): d = max|x| / 127 and
// q = round-to-nearest-even(x / d), both in IEEE fp32.  The divisions are
// correctly rounded (no fast-math in this library) and rintf lowers to
// v_rndne_f32, so the result is bit-identical to a scalar reference; the
// per-value divisions are replaced by one reciprocal per block wherever that
// provably gives the same integer (q8k_quant4).  The maximum is exact in any
// order, so its reduction order is free.
#pragma once
#include <hip/hip_runtime.h>

namespace tq {

// One DPP lane exchange of a float (row_mask = bank_mask = 0xf: every lane).
template <int kCtrl>
__device__ __forceinline__ float q8k_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}

// Block scale: max |x| over the wave, then / 127.  Within each 16-lane row the
// maximum travels through DPP lane swaps (quad xor 1, quad xor 2, half-row
// mirror, row mirror: VALU only, no LDS round trip); the four row maxima are
// then read into scalar registers.  The result is wave-uniform.
__device__ __forceinline__ float q8k_block_scale(const float4 v) {
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, q8k_dpp<0xB1>(a));   // quad_perm [1,0,3,2]
  a = fmaxf(a, q8k_dpp<0x4E>(a));   // quad_perm [2,3,0,1]
  a = fmaxf(a, q8k_dpp<0x141>(a));  // row_half_mirror: lanes i and 7 - i of each 8
  a = fmaxf(a, q8k_dpp<0x140>(a));  // row_mirror: lanes i and 15 - i of each 16
  const int ai = __builtin_bit_cast(int, a);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)) / 127.0f;
}

// One quantized value (d == 0: the whole block is zero).  Branch-free: the
// quotient is formed for every lane (x / 0 is an IEEE infinity or NaN, and
// fmaxf drops the NaN) and the d == 0 case is selected afterwards.
__device__ __forceinline__ int q8k_quant1(float x, float d) {
  const float r = fminf(127.0f, fmaxf(-127.0f, rintf(x / d)));
  return d == 0.0f ? 0 : (int)r;
}

// The lane's four quantized values packed little-endian into a dword.
__device__ __forceinline__ int q8k_pack4(int q0, int q1, int q2, int q3) {
  return (q0 & 0xff) | ((q1 & 0xff) << 8) | ((q2 & 0xff) << 16) | ((q3 & 0xff) << 24);
}

// The lane's four values quantized and packed, bit-identical to q8k_quant1
// on each, with one division per block instead of one per value.
//
// With r = fl(1/d), the product y = fl(x * r) is within 3 * 2^-24 * |x/d| of
// the correctly rounded quotient fl(x/d) (two roundings of relative size
// 2^-24 each, plus the quotient's own), i.e. within 2^-15 since |x/d| <= 127
// (up to rounding) in a q8_K block.  If y lies farther than 2^-15 from every
// half-integer, fl(x/d) and y round to the same integer; otherwise (and for
// non-finite y, or a block scale below 2^-100 where 1/d may overflow) the
// value takes the exact path.  A wave takes the exact path only when one of
// its lanes needs it.
__device__ __forceinline__ int q8k_quant4(const float4 v, float d) {
  if (d == 0.0f) return 0;
  const float x[4] = {v.x, v.y, v.z, v.w};
  int qv[4];
  if (d >= 0x1p-100f) {
    const float r = 1.0f / d;
    bool exact = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = x[i] * r;
      const float k = rintf(y);
      // |y - k| is the distance to the nearest integer; a half-integer is near
      // when it exceeds 0.5 - 2^-15 (NaN compares false: exact path)
      exact |= !(fabsf(y - k) < 0.5f - 0x1p-15f);
      qv[i] = (int)k;
    }
    if (!exact) return q8k_pack4(qv[0], qv[1], qv[2], qv[3]);
  }
  return q8k_pack4(q8k_quant1(x[0], d), q8k_quant1(x[1], d), q8k_quant1(x[2], d), q8k_quant1(x[3], d));
}

}  // namespace tq
