// k_gemm_pq2.hip -- prompt (small-batch) product, repacked pq2_0 x q8_K,
// on int8 MFMA.
//
// Same arithmetic per token as the matrix-vector product (page 1, "prefill
// wants a different shape": with many tokens in flight a loaded weight is
// reused, so instruction count matters; "the leftovers": token counts that
// are not a multiple of the tile are zero-padded and only real outputs are
// written).
//
// How (gfx950):
//   * A = weights: the lane (row r16, k-block qd) loads the dwordx4 of its
//     row at (superchunk, qd); dword c expands with one shift and one mask per
//     field into the 16 int8 values 64*w of columns 64c + 16qd + [0, 16), which
//     is exactly one A operand of v_mfma_i32_16x16x64_i8 for chunk c.
//   * B = activations: the lane (token t16, qd) loads the 16 contiguous bytes
//     q[t][256 sc + 64 c + 16 qd ...] -- one dwordx4, no shuffle.
//   * The MFMA accumulators restart every 128-group (two chunks), because the
//     weight scale changes per group; the group epilogue converts 64*I to the
//     fp64 term d_w * d_x * I and accumulates it in fp64.
//   * Workgroup = 4 waves on one 64-row tile and up to 64 tokens; the waves
//     split the superchunks (contiguous runs) and each covers all 64 rows, so
//     every B operand it loads feeds 4 row blocks.  The four fp64 partial
//     tiles are summed in LDS in wave order and rounded once.
//   * Padded tokens (t >= tokens) have B = 0 and are never stored.
#include "kernels.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kRowBlocks = 4;  // 4 x 16 rows = the 64-row tile

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h));
}

__device__ __forceinline__ v4i expand64(uint32_t d) {
  v4i a;
  a[0] = (int)((d << 6) & 0xC0C0C0C0u);
  a[1] = (int)((d << 4) & 0xC0C0C0C0u);
  a[2] = (int)((d << 2) & 0xC0C0C0C0u);
  a[3] = (int)(d & 0xC0C0C0C0u);
  return a;
}

template <int NT, bool IDOTS>
__global__ __launch_bounds__(64 * kWaves, 1) void gemm_pq2_kernel(const uint4* __restrict__ codes,
                                                                  const uint16_t* __restrict__ scales,
                                                                  const int8_t* __restrict__ q, const float* __restrict__ dx,
                                                                  float* __restrict__ y, int32_t* __restrict__ idots,
                                                                  int rows, int nsc, int G8, int tokens, int spw) {
  // fp64 partial tiles of waves 1..3 for one row block, [wave-1][n][v][lane]
  __shared__ double red[kWaves - 1][NT * 4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  const int tok0 = blockIdx.y * (16 * NT);
  const int l16 = lane & 15;
  const int qd = lane >> 4;
  const int K = nsc * 256;
  const int G = nsc * 2;
  const int B = nsc;
  const int sc0 = wave * spw;
  const int sc1 = min(nsc, sc0 + spw);

  // B-operand rows of this lane (one token per n-tile) and output tokens
  const int8_t* qrow[NT];
  bool tok_ok[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int t = tok0 + 16 * n + l16;
    tok_ok[n] = t < tokens;
    qrow[n] = q + (size_t)(tok_ok[n] ? t : 0) * K + 16 * qd;
  }

  double yacc[kRowBlocks][NT][4];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 4; ++v) yacc[rb][n][v] = 0.0;

  const uint4* cp = codes + (size_t)tile * nsc * 256 + qd * 64 + l16;

  for (int sc = sc0; sc < sc1; ++sc) {
    uint4 wv[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) wv[rb] = cp[(size_t)sc * 256 + rb * 16];
    double dxs[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
      dxs[n] = (!IDOTS && tok_ok[n]) ? (double)dx[(size_t)(tok0 + 16 * n + l16) * B + sc] : 0.0;

#pragma unroll
    for (int half = 0; half < 2; ++half) {  // group g = 2 sc + half: chunks c = 2 half, 2 half + 1
      const int g = 2 * sc + half;
      v4i acc[kRowBlocks][NT];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[rb][n] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = 2 * half + cc;
        v4i bop[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint4 b = tok_ok[n] ? *reinterpret_cast<const uint4*>(qrow[n] + sc * 256 + 64 * c) : uint4{0, 0, 0, 0};
          bop[n] = v4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
        }
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
          const uint32_t d = c == 0 ? wv[rb].x : c == 1 ? wv[rb].y : c == 2 ? wv[rb].z : wv[rb].w;
          const v4i a = expand64(d);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[rb][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bop[n], acc[rb][n], 0, 0, 0);
        }
      }
      // epilogue of group g: lane holds rows 16 rb + 4 qd + v, token 16 n + l16
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 16 * rb + 4 * qd + v;
          const double dw = (double)half_bits_to_float(scales[(((size_t)tile * G8 + g / 8) * 64 + r) * 8 + (g & 7)]);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int I = acc[rb][n][v] >> 6;  // exact: the MFMA sums 64 * w * q
            if (IDOTS) {
              const int row = tile * 64 + r;
              if (tok_ok[n] && row < rows) idots[((size_t)(tok0 + 16 * n + l16) * rows + row) * G + g] = I;
            } else {
              yacc[rb][n][v] += (dw * dxs[n]) * (double)I;
            }
          }
        }
      }
    }
  }
  if (IDOTS) return;

  // Sum the four waves' partial tiles in wave order, one row block at a time.
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    if (wave > 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave - 1][n * 4 + v][lane] = yacc[rb][n][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          double s = yacc[rb][n][v];
#pragma unroll
          for (int w = 0; w < kWaves - 1; ++w) s += red[w][n * 4 + v][lane];
          const int row = tile * 64 + 16 * rb + 4 * qd + v;
          const int t = tok0 + 16 * n + l16;
          if (row < rows && t < tokens) y[(size_t)t * rows + row] = (float)s;
        }
    }
    __syncthreads();
  }
}

template <int NT>
hipError_t launch_nt(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                     int32_t* idots, hipStream_t s) {
  const int nsc = (int)dm.nsc;
  const int spw = (nsc + kWaves - 1) / kWaves;
  const dim3 grid((unsigned)dm.ntiles, (unsigned)((tokens + 16 * NT - 1) / (16 * NT))), block(64 * kWaves);
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(w + pq2_code_bytes(dm));
  if (idots)
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, true>), grid, block, 0, s, codes, scales, q, dx, y, idots, (int)dm.rows, nsc,
                       (int)dm.G8, (int)tokens, spw);
  else
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, false>), grid, block, 0, s, codes, scales, q, dx, y, idots, (int)dm.rows, nsc,
                       (int)dm.G8, (int)tokens, spw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_pq2(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s) {
  if (tokens <= 16) return launch_nt<1>(w, dm, tokens, q, dx, y, idots, s);
  if (tokens <= 32) return launch_nt<2>(w, dm, tokens, q, dx, y, idots, s);
  return launch_nt<4>(w, dm, tokens, q, dx, y, idots, s);
}

}  // namespace tq
