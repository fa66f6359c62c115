// k_gemv_pq2.hip -- decode matrix-vector product, repacked pq2_0 x q8_K.
//
// What is computed (page 1, "the trick with 4 and 16"; ciot README):
//   I[r][g] = sum_{k<128} w[r][128g+k] * q[128g+k]          exact integer
//   y[r]    = sum_g d_w[r][g] * d_x[g/2] * I[r][g]          fp64, rounded once
//
// How (gfx950): the product streams every weight byte from HBM exactly once,
// so the kernel is bandwidth bound and is shaped for coalesced loads and
// memory-level parallelism rather than for ALU reuse.
//   * one lane = one row; a workgroup = one 64-row tile; its waves split the
//     columns into contiguous runs of 256-column superchunks;
//   * per superchunk a lane issues four dwordx4 loads (qd = 0..3), each a
//     fully coalesced 1 KiB wave request; UNROLL superchunks are in flight;
//   * the activation bytes a lane needs are the same for every lane of the
//     wave, so they are read with scalar loads into SGPRs and fed to
//     v_dot4_i32_i8 directly -- no LDS traffic, no VGPRs;
//   * each code dword yields four dot4 operands with one shift and one mask
//     each ((d << (6-2s)) & 0xC0C0C0C0 = 64*w for four columns, the slot
//     masking idea of the pages with two's-complement codes, so no +1
//     correction is needed); the factor 64 is removed exactly by a shift;
//   * per group: term = (d_w * d_x) * I in fp64 (exact), accumulated in fp64;
//     the wave partials are combined in LDS in wave order and rounded once.
#include "kernels.h"

namespace tq {
namespace {

constexpr int kMaxWaves = 16;

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h));
}

__device__ __forceinline__ int slot64(uint32_t d, int s) {
  // field s of every byte, moved to bits 6..7: the byte reads as 64 * w
  return (int)((d << (6 - 2 * s)) & 0xC0C0C0C0u);
}

// Integer dots of one superchunk: i0 for group 2 sc (dwords c = 0, 1), i1 for
// group 2 sc + 1 (c = 2, 3).  `a` points at the superchunk's 64 activation
// dwords (wave-uniform).
__device__ __forceinline__ void superchunk_dots(const uint4 (&v)[4], const int* __restrict__ a, int& i0, int& i1) {
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const uint32_t dw[4] = {v[qd].x, v[qd].y, v[qd].z, v[qd].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int act = a[16 * c + 4 * qd + s];
        if (c < 2)
          i0 = __builtin_amdgcn_sdot4(slot64(dw[c], s), act, i0, false);
        else
          i1 = __builtin_amdgcn_sdot4(slot64(dw[c], s), act, i1, false);
      }
    }
  }
}

template <int UNROLL, bool IDOTS>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_pq2_kernel(const uint4* __restrict__ codes,
                                                                  const uint32_t* __restrict__ scales,
                                                                  const int* __restrict__ q, const float* __restrict__ dx,
                                                                  float* __restrict__ y, int32_t* __restrict__ idots,
                                                                  int rows, int nsc, int G8, int spw) {
  __shared__ double red[kMaxWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int tile = blockIdx.x;
  const int row = tile * 64 + lane;
  const int G = 2 * nsc;
  const int sc0 = wave * spw;
  const int sc1 = min(nsc, sc0 + spw);

  const uint4* cp = codes + (size_t)tile * nsc * 256 + lane;
  const uint32_t* sp = scales + (size_t)tile * G8 * 256 + lane * 4;
  double acc = 0.0;

  auto epilogue = [&](int sc, int i0, int i1) {
    const int I0 = i0 >> 6, I1 = i1 >> 6;  // exact: both are 64 * I
    if (IDOTS) {
      if (row < rows) {
        idots[(size_t)row * G + 2 * sc] = I0;
        idots[(size_t)row * G + 2 * sc + 1] = I1;
      }
    } else {
      const uint32_t s2 = sp[(sc >> 2) * 256 + (sc & 3)];  // fp16 scales of groups 2sc, 2sc+1
      const double dxs = (double)dx[sc];
      acc += ((double)half_bits_to_float(s2 & 0xffffu) * dxs) * (double)I0;
      acc += ((double)half_bits_to_float(s2 >> 16) * dxs) * (double)I1;
    }
  };

  int sc = sc0;
  for (; sc + UNROLL <= sc1; sc += UNROLL) {
    uint4 v[UNROLL][4];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) v[u][qd] = cp[(size_t)((sc + u) * 4 + qd) * 64];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      int i0 = 0, i1 = 0;
      superchunk_dots(v[u], q + (size_t)(sc + u) * 64, i0, i1);
      epilogue(sc + u, i0, i1);
    }
  }
  for (; sc < sc1; ++sc) {
    uint4 v[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) v[qd] = cp[(size_t)(sc * 4 + qd) * 64];
    int i0 = 0, i1 = 0;
    superchunk_dots(v, q + (size_t)sc * 64, i0, i1);
    epilogue(sc, i0, i1);
  }

  if (IDOTS) return;
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    double s = red[0][lane];
    for (int w = 1; w < nw; ++w) s += red[w][lane];
    if (row < rows) y[row] = (float)s;
  }
}

}  // namespace

hipError_t launch_gemv_pq2(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s) {
  constexpr int kUnroll = 4;
  const int nsc = (int)dm.nsc;
  // Split the columns over up to 8 waves, each taking a contiguous run.
  int waves = nsc < 8 ? nsc : 8;
  const int spw = (nsc + waves - 1) / waves;
  waves = (nsc + spw - 1) / spw;
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint32_t* scales = reinterpret_cast<const uint32_t*>(w + pq2_code_bytes(dm));
  const dim3 grid((unsigned)dm.ntiles), block(64 * waves);
  if (idots)
    hipLaunchKernelGGL((gemv_pq2_kernel<kUnroll, true>), grid, block, 0, s, codes, scales,
                       reinterpret_cast<const int*>(q), dx, y, idots, (int)dm.rows, nsc, (int)dm.G8, spw);
  else
    hipLaunchKernelGGL((gemv_pq2_kernel<kUnroll, false>), grid, block, 0, s, codes, scales,
                       reinterpret_cast<const int*>(q), dx, y, idots, (int)dm.rows, nsc, (int)dm.G8, spw);
  return hipGetLastError();
}

}  // namespace tq
