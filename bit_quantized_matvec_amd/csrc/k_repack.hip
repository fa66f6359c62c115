// k_repack.hip -- load-time repack of canonical pq2_0 / ptq1_0 matrices into
// the device layouts described in layout.h, and the inverse (for tests and
// export).
//
// The pages repack once at model load, in place, at the same size
// ("the layout", page 1; ciot README layout paragraph).  Here the repack is
// out of place (an in-place permutation on the GPU would need scratch) and
// also keeps the total size.  Every kernel is pure byte / bit movement with
// one thread per output dword, so the cost is a copy of the matrix.
#include "kernels.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
// Every kernel below loops over its items with a grid stride, so a launch
// covers any item count with at most kMaxBlocks workgroups (2^28 work-items,
// far below the 2^32 limit of one launch dimension).
constexpr int64_t kMaxBlocks = int64_t(1) << 20;

inline unsigned grid_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (unsigned)(b < kMaxBlocks ? (b > 0 ? b : 1) : kMaxBlocks);
}

#define TQ_FOR_ITEMS(i, n) \
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < (n); i += (int64_t)gridDim.x * kThreads)

// ---------------------------------------------------------------- pq2_0 codes
// Code dword index i -> (tile, sc, qd, row, c), stored in unit (tile, sc) at
// dword (qd * 64 + row) * 4 + c.  Its byte j, field s holds
// the weight of column 256 sc + 64 c + 16 qd + 4 s + j, i.e. (in group
// g = 2 sc + c/2, position k = 64 (c&1) + 16 qd + 4 s + j) field j of
// canonical byte 16 (c&1) + 4 qd + s.  So the output dword is the 4x4
// transpose of the 2-bit fields of four consecutive canonical bytes, each
// field re-coded from u = w + 1 to two's-complement w.
__global__ void repack_pq2_codes(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t rows, int64_t nsc,
                                 int64_t ndw, int32_t* __restrict__ bad_flag) {
  TQ_FOR_ITEMS(i, ndw) {
  const int c = (int)(i & 3);
  const int r = (int)((i >> 2) & 63);
  const int qd = (int)((i >> 8) & 3);
  const int64_t rest = i >> 10;  // the unit, tile * nsc + sc
  const int64_t sc = rest % nsc;
  const int64_t tile = rest / nsc;
  const int64_t row = tile * kRowTile + r;
  uint32_t out = 0;  // padded rows: w = 0 everywhere
  if (row < rows) {
    const int64_t G = nsc * 2;
    const int64_t g = 2 * sc + (c >> 1);
    const uint8_t* qs = src + (row * G + g) * 34 + 2 + 16 * (c & 1) + 4 * qd;
    bool bad = false;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t cb = qs[s];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = (cb >> (2 * j)) & 3u;
        bad |= (u == 3u);
        const uint32_t code = (u + 3u) & 3u;  // w = u - 1 as 2-bit two's complement
        out |= code << (8 * j + 2 * s);
      }
    }
    if (bad && bad_flag) *bad_flag = 1;
  }
  dst[rest * (kPq2UnitBytes / 4) + (i & 1023)] = out;
  }
}

// Inverse: one thread per canonical 34-byte block.
__global__ void unrepack_pq2_codes(const uint32_t* __restrict__ units, uint8_t* __restrict__ dst, int64_t rows,
                                   int64_t nsc) {
  const int64_t G = nsc * 2;
  TQ_FOR_ITEMS(b, rows * G) {
  const int64_t row = b / G, g = b % G;
  const int64_t tile = row / kRowTile;
  const int r = (int)(row % kRowTile);
  const int64_t sc = g >> 1;
  uint8_t* out = dst + b * 34;
  const uint32_t* unit = units + (tile * nsc + sc) * (kPq2UnitBytes / 4);
  const uint32_t pair = unit[kPq2ScaleOffset / 4 + r];
  const uint32_t h = (g & 1) ? pair >> 16 : pair & 0xffffu;
  out[0] = (uint8_t)(h & 0xff);
  out[1] = (uint8_t)(h >> 8);
  for (int qd = 0; qd < 4; ++qd) {
    for (int cc = 0; cc < 2; ++cc) {
      const int c = 2 * (int)(g & 1) + cc;
      const uint32_t dw = unit[(qd * 64 + r) * 4 + c];
      for (int s = 0; s < 4; ++s) {
        uint32_t byte = 0;
        for (int j = 0; j < 4; ++j) {
          const uint32_t code = (dw >> (8 * j + 2 * s)) & 3u;
          const uint32_t u = (code + 1u) & 3u;  // two's-complement w back to u = w + 1
          byte |= u << (2 * j);
        }
        out[2 + 16 * cc + 4 * qd + s] = (uint8_t)byte;
      }
    }
  }
  }
}

// ------------------------------------------------------------- pq2_0 scales
// fp16 scales of groups 2 sc, 2 sc + 1 of a row into dword `row` of unit
// (tile, sc)'s scale pairs; zero for padding rows.
__global__ void repack_pq2_scales(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t rows, int64_t nsc,
                                  int64_t n) {
  TQ_FOR_ITEMS(i, n) {
  const int r = (int)(i & 63);
  const int64_t rest = i >> 6;
  const int64_t sc = rest % nsc;
  const int64_t tile = rest / nsc;
  const int64_t row = tile * kRowTile + r;
  uint32_t v = 0;
  if (row < rows) {
    const uint8_t* b0 = src + (row * 2 * nsc + 2 * sc) * 34;
    const uint8_t* b1 = b0 + 34;
    v = (uint32_t)(b0[0] | (b0[1] << 8)) | ((uint32_t)(b1[0] | (b1[1] << 8)) << 16);
  }
  dst[rest * (kPq2UnitBytes / 4) + kPq2ScaleOffset / 4 + r] = v;
  }
}

// ------------------------------------------------------------- ptq1_0 scales
// fp16 scale of (row, group) into [row][8] of unit (tile, g8); zero for
// padding.
__global__ void repack_scales(const uint8_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t rows, int64_t G,
                              int64_t G8, int block_bytes, int64_t n) {
  TQ_FOR_ITEMS(i, n) {
  const int gi = (int)(i & 7);
  const int r = (int)((i >> 3) & 63);
  const int64_t rest = i >> 9;
  const int64_t g8 = rest % G8;
  const int64_t tile = rest / G8;
  const int64_t row = tile * kRowTile + r;
  const int64_t g = g8 * 8 + gi;
  uint16_t h = 0;
  if (row < rows && g < G) {
    const uint8_t* blk = src + (row * G + g) * block_bytes;
    h = (uint16_t)(blk[0] | (blk[1] << 8));
  }
  dst[rest * (kPtq1UnitBytes / 2) + kPtq1ScaleOffset / 2 + (i & 511)] = h;
  }
}

// --------------------------------------------------------------- ptq1_0 codes
__device__ __forceinline__ int64_t ptq1_src_byte(int D, int bi, int64_t sb, int64_t* g_out) {
  // byte bi (0..3) of superblock dword D -> (group within matrix, byte within qs)
  if (D < 48) {
    const int gi = D / 6, m = D % 6;
    *g_out = sb * 8 + gi;
    return 4 * m + bi;
  }
  const int p = D - 48;
  *g_out = sb * 8 + 2 * p + (bi >> 1);
  return 24 + (bi & 1);
}

__global__ void repack_ptq1_codes(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t rows, int64_t G,
                                  int64_t G8, int64_t ndw) {
  TQ_FOR_ITEMS(i, ndw) {
  const int c = (int)(i & 3);
  const int r = (int)((i >> 2) & 63);
  const int64_t rest = i >> 8;
  const int L = (int)(rest % kPtqLoads);
  const int64_t rest2 = rest / kPtqLoads;
  const int64_t sb = rest2 % G8;
  const int64_t tile = rest2 / G8;
  const int64_t row = tile * kRowTile + r;
  const int D = 4 * L + c;
  uint32_t out = 0;
  if (row < rows) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      int64_t g;
      const int64_t byte = ptq1_src_byte(D, bi, sb, &g);
      if (g < G) out |= (uint32_t)src[(row * G + g) * 28 + 2 + byte] << (8 * bi);
    }
  }
  // unit rest2 = tile * G8 + sb holds 13 * 256 code dwords, then its scales
  dst[rest2 * (kPtq1UnitBytes / 4) + (i - rest2 * (kPtqLoads * 256))] = out;
  }
}

__global__ void unrepack_ptq1_codes(const uint8_t* __restrict__ units, uint8_t* __restrict__ dst, int64_t rows, int64_t G,
                                    int64_t G8) {
  TQ_FOR_ITEMS(b, rows * G) {
  const int64_t row = b / G, g = b % G;
  const int64_t tile = row / kRowTile;
  const int r = (int)(row % kRowTile);
  const int64_t sb = g / 8;
  const int gi = (int)(g % 8);
  uint8_t* out = dst + b * 28;
  const uint8_t* base = units + (tile * G8 + sb) * kPtq1UnitBytes;
  const uint16_t h = reinterpret_cast<const uint16_t*>(base + kPtq1ScaleOffset)[r * 8 + gi];
  out[0] = (uint8_t)(h & 0xff);
  out[1] = (uint8_t)(h >> 8);
  for (int byte = 0; byte < 26; ++byte) {
    int D, bi;
    if (byte < 24) {
      D = 6 * gi + byte / 4;
      bi = byte % 4;
    } else {
      D = 48 + gi / 2;
      bi = 2 * (gi & 1) + (byte - 24);
    }
    const int L = D / 4, c = D % 4;
    const int64_t dw = ((int64_t)L * 64 + r) * 4 + c;
    out[2 + byte] = base[dw * 4 + bi];
  }
  }
}

}  // namespace

hipError_t launch_repack_pq2(const uint8_t* src, uint8_t* dst, const Dims& dm, int32_t* bad_flag, hipStream_t s) {
  const int64_t ndw = pq2_code_bytes(dm) / 4;
  hipLaunchKernelGGL(repack_pq2_codes, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src, reinterpret_cast<uint32_t*>(dst),
                     dm.rows, dm.nsc, ndw, bad_flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = pq2_scale_bytes(dm) / 4;
  hipLaunchKernelGGL(repack_pq2_scales, dim3(grid_for(ns)), dim3(kThreads), 0, s, src, reinterpret_cast<uint32_t*>(dst),
                     dm.rows, dm.nsc, ns);
  return hipGetLastError();
}

hipError_t launch_unrepack_pq2(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s) {
  const int64_t nb = dm.rows * dm.G;
  hipLaunchKernelGGL(unrepack_pq2_codes, dim3(grid_for(nb)), dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(src),
                     dst, dm.rows, dm.nsc);
  return hipGetLastError();
}

hipError_t launch_repack_ptq1(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s) {
  const int64_t ndw = ptq1_code_bytes(dm) / 4;
  hipLaunchKernelGGL(repack_ptq1_codes, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src, reinterpret_cast<uint32_t*>(dst),
                     dm.rows, dm.G, dm.G8, ndw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = ptq1_scale_bytes(dm) / 2;
  hipLaunchKernelGGL(repack_scales, dim3(grid_for(ns)), dim3(kThreads), 0, s, src, reinterpret_cast<uint16_t*>(dst),
                     dm.rows, dm.G, dm.G8, 28, ns);
  return hipGetLastError();
}

hipError_t launch_unrepack_ptq1(const uint8_t* src, uint8_t* dst, const Dims& dm, hipStream_t s) {
  const int64_t nb = dm.rows * dm.G;
  hipLaunchKernelGGL(unrepack_ptq1_codes, dim3(grid_for(nb)), dim3(kThreads), 0, s, src, dst, dm.rows, dm.G, dm.G8);
  return hipGetLastError();
}

}  // namespace tq
