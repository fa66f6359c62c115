// q8k_block.h -- the q8_K arithmetic of 256-value blocks held by a wave64
// (4 consecutive values per lane), shared by the standalone quantizer and the
// matrix-vector kernels that quantize their own activations, so that both
// produce the same bits.
//
// q8_K (ciot README, intro; page 1 "the paperwork"): d = max|x| / 127 and
// q = round-to-nearest-even(x / d), both in IEEE fp32.  Every result here is
// the correctly rounded one (no fast-math in this library; rintf lowers to
// v_rndne_f32), so it is bit-identical to a scalar reference.  Two IEEE
// divisions per block would each be a chain of eight dependent instructions
// through the single VCC register, which no two blocks can overlap; instead:
//   * d = fl(amax / 127) comes from a product and one FMA correction
//     (q8k_div127), equal to the IEEE quotient for every amax >= 2^-93
//     (verified over every fp32 significand at exponents from 2^-126 to
//     2^127: the result depends on the significand alone while every
//     intermediate stays normal); smaller nonzero maxima take the division;
//   * q = rint(fl(x / d)) comes from y = fl(x * r) with r a refined
//     reciprocal of d wherever that provably gives the same integer
//     (q8k_quant_batch); the other values take the exact division.
// The maximum is exact in any order, so its reduction order is free.
#pragma once
#include <hip/hip_runtime.h>

namespace tq {

// One DPP lane exchange of a float (row_mask = bank_mask = 0xf: every lane).
template <int kCtrl>
__device__ __forceinline__ float q8k_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}

// fl(a / 127) for finite a >= 2^-93: c = fl(1/127), p = fl(a c), the residual
// a - 127 p is exact in one FMA, and one FMA step with c rounds to the IEEE
// quotient.  Three independent-of-VCC instructions instead of a division.
__device__ __forceinline__ float q8k_div127(float a) {
  constexpr float c = 1.0f / 127.0f;
  const float p = a * c;
  const float r = __builtin_fmaf(-p, 127.0f, a);
  return __builtin_fmaf(r, c, p);
}

// Reciprocal of d in [2^-100, 2^122): v_rcp_f32 (relative error below 2^-22)
// and one Newton step, e = 1 - d r0 (one rounding), r = r0 + e r0 (one
// rounding): |r - 1/d| <= (2^-24 + 2^-45) / d.
__device__ __forceinline__ float q8k_recip(float d) {
  const float r0 = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

// One quantized value by the definition (d == 0: the whole block is zero).
// Branch-free: the quotient is formed for every lane (x / 0 is an IEEE
// infinity or NaN, and fmaxf drops the NaN) and the d == 0 case is selected
// afterwards.
__device__ __forceinline__ int q8k_quant1(float x, float d) {
  const float r = fminf(127.0f, fmaxf(-127.0f, rintf(x / d)));
  return d == 0.0f ? 0 : (int)r;
}

// The lane's four quantized values packed little-endian into a dword.
__device__ __forceinline__ int q8k_pack4(int q0, int q1, int q2, int q3) {
  return (q0 & 0xff) | ((q1 & 0xff) << 8) | ((q2 & 0xff) << 16) | ((q3 & 0xff) << 24);
}

// NB blocks at once, one per entry of v (the lane's four values of block b in
// v[b]): the block scales d[b] (wave-uniform) and the lane's packed values,
// equal to d = fl(max|x| / 127) and q = rint(fl(x / d)) clamped to +-127.
//
// The blocks' work is one straight run with no branch between blocks, so the
// compiler interleaves the NB independent chains (maximum reduction, scale,
// reciprocal, products, rounding); a block's chain alone is mostly latency.
//
// Fast path, for d >= 2^-100: y = fl(x r) with r = q8k_recip(d).  With
// |x / d| <= 127 (1 + 2^-23) in a q8_K block, y lies within
// |x/d| (2^-23 + 2^-24)(1 + 2^-20) of x / d, and fl(x / d) within
// |x/d| 2^-24, so |y - fl(x/d)| < 381 * 2^-24 < 2^-15.  If y lies farther
// than 2^-15 from every half-integer, fl(x/d) lies strictly inside the same
// unit interval around k = rint(y), so rint(fl(x/d)) = k (and |k| <= 127, no
// clamp needed).  Values nearer a half-integer, and blocks with
// 0 < d < 2^-100, take the exact path afterwards (only the lanes and blocks
// that need it).
template <int NB>
__device__ __forceinline__ void q8k_quant_batch(const float4 (&v)[NB], float (&d)[NB], int (&packed)[NB]) {
  float a[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) a[b] = fmaxf(fmaxf(fabsf(v[b].x), fabsf(v[b].y)), fmaxf(fabsf(v[b].z), fabsf(v[b].w)));
  // maximum within each 16-lane row by DPP lane swaps (quad xor 1, quad xor 2,
  // half-row mirror, row mirror), then over the four row maxima
#pragma unroll
  for (int b = 0; b < NB; ++b) a[b] = fmaxf(a[b], q8k_dpp<0xB1>(a[b]));
#pragma unroll
  for (int b = 0; b < NB; ++b) a[b] = fmaxf(a[b], q8k_dpp<0x4E>(a[b]));
#pragma unroll
  for (int b = 0; b < NB; ++b) a[b] = fmaxf(a[b], q8k_dpp<0x141>(a[b]));
#pragma unroll
  for (int b = 0; b < NB; ++b) a[b] = fmaxf(a[b], q8k_dpp<0x140>(a[b]));
  bool tiny = false;  // wave-uniform: some block's maximum is nonzero and below 2^-93
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int ai = __builtin_bit_cast(int, a[b]);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 48));
    a[b] = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
    d[b] = q8k_div127(a[b]);
    tiny |= a[b] != 0.0f && a[b] < 0x1p-93f;
  }
  if (tiny) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (a[b] < 0x1p-93f) d[b] = a[b] / 127.0f;
  }
  unsigned slow = 0;  // bit b: this lane's values of block b take the exact path
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool fast = d[b] >= 0x1p-100f;
    const float r = q8k_recip(fast ? d[b] : 1.0f);
    const float x[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
    int qv[4];
    bool exact = !fast;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = x[i] * r;
      const float k = rintf(y);
      exact |= !(fabsf(y - k) < 0.5f - 0x1p-15f);  // NaN compares false: exact path
      qv[i] = (int)k;
    }
    packed[b] = d[b] == 0.0f ? 0 : q8k_pack4(qv[0], qv[1], qv[2], qv[3]);
    if (d[b] != 0.0f && exact) slow |= 1u << b;
  }
  if (slow) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (slow & (1u << b))
        packed[b] = q8k_pack4(q8k_quant1(v[b].x, d[b]), q8k_quant1(v[b].y, d[b]), q8k_quant1(v[b].z, d[b]),
                              q8k_quant1(v[b].w, d[b]));
    }
  }
}

}  // namespace tq
