// k_gemm_pq2.hip -- prompt (small-batch) product, repacked pq2_0 x q8_K,
// on int8 MFMA.
//
// Same arithmetic per token as the matrix-vector product (page 1, "prefill
// wants a different shape": with many tokens in flight a loaded weight is
// reused, so instruction count matters; "the leftovers": token counts that
// are not a multiple of the tile are padded and only real outputs are
// written).
//
// How (gfx950):
//   * Workgroup = 4 waves on one 64-row tile and 16 * NT tokens; wave w owns
//     rows 16w..16w+15 for every token and both 128-groups of a superchunk.
//   * Each wave loads its own operands straight into registers: per
//     superchunk one 16-byte code load per lane (lane (row, qd) gets the four
//     dwords whose fields are columns 64c + 16qd + [0, 16), c = 0..3 -- the A
//     operands of four v_mfma_i32_16x16x64_i8 after one shift and one mask
//     per field) and one 16-byte load of its four rows' scale pairs.
//   * The activations of the superchunk (16 * NT tokens x 256 bytes) are
//     shared by the four waves through a double-buffered LDS stage: fetched
//     row by row (coalesced), stored at [token][piece ^ (token & 15)] so that
//     neither the stores nor the operand reads (16 tokens, one piece) collide
//     in LDS banks; one barrier per superchunk.  The tokens' d_x for every
//     superchunk are copied into LDS once, before the loop.
//   * Codes, scales and activations are fetched D superchunks ahead (4 for
//     16-token blocks, 2 for 32-token blocks) into
//     register rings with literal indices.  A prologue fills the ring and the
//     main loop runs only while every fetch is real, so its body has no
//     branch and the compiler's wait counts stay exact (no drain per pass);
//     the last passes run in a separate tail loop.
//   * Epilogue per superchunk, in fp64 (every product exact, sums rounded
//     once per operation): inner = d_w(2sc+1) * I1 + d_w(2sc) * I0, then
//     y += (d_x / 64) * inner; the 1/64 removes the scale of the
//     two's-complement codes and is exact.
//   * Several token blocks of one tile run on one XCD (workgroup id modulo
//     8) and are dispatched together, so their code reads after the first
//     hit that XCD's L2 instead of HBM.
//   * Tokens past the end read a valid token (the last one) and are never
//     stored; rows past the end have zero codes and scales.
#include <algorithm>

#include "kernels.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
// Native vector types (not HIP's uint4 struct) keep copies in registers.
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Register-ring depth in superchunks: measured on 17408 x 5120, 4 is best for
// 16-token blocks (4 and 16 tokens; 2: 15.7 us at 4 tokens vs 12.4) and 2 for
// 32-token blocks (64 tokens: 23.9 us vs 24.4); deeper rings are slower.
template <int NT>
constexpr int kDepth = NT == 1 ? 4 : 2;

// Workgroups per token block of the balanced grid: one per compute unit.
constexpr int kBalancedWgs = 256;

// LDS of the d_x copy: 16 * NT tokens x nsc superchunks of fp32, at most
// 32 KiB (rows of up to 65536 columns with 32-token blocks)
constexpr size_t gemm_dx_bytes(int nsc, int nt) { return (size_t)nsc * 16 * nt * 4; }
constexpr size_t kMaxDxBytes = 32 * 1024;

__device__ __forceinline__ v4i expand64(uint32_t d) {
  v4i a;
  a[0] = (int)((d << 6) & 0xC0C0C0C0u);
  a[1] = (int)((d << 4) & 0xC0C0C0C0u);
  a[2] = (int)((d << 2) & 0xC0C0C0C0u);
  a[3] = (int)(d & 0xC0C0C0C0u);
  return a;
}

__device__ __forceinline__ double lo_half(uint32_t p) {
  return (double)static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(p & 0xffffu)));
}
__device__ __forceinline__ double hi_half(uint32_t p) {
  return (double)static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(p >> 16)));
}

// Grid: ntb token blocks per tile, laid out so that the blocks of one tile
// share blockIdx.x % 8: id = (grp * ntb + tb) * 8 + (tile % 8), grp = tile / 8.
//
// BAL (a little over 256 tiles, where one workgroup per tile would leave
// some compute units with two and most with one): 256 workgroups per token
// block of 5 waves each, each taking 4 or 5 consecutive 16-row blocks (one
// per wave; a fifth wave without a block only takes part in the barriers), evenly
// over the XCDs.  Every wave still runs the whole row of superchunks, so the
// sums are the same.
template <int NT, bool IDOTS, bool BAL>
__global__ __launch_bounds__(BAL ? 320 : 256) void gemm_pq2_kernel(const v4u* __restrict__ codes,
                                                                  const uint32_t* __restrict__ scales,
                                                                  const int8_t* __restrict__ q,
                                                                  const float* __restrict__ dx, float* __restrict__ y,
                                                                  int32_t* __restrict__ idots, int rows, int ntiles,
                                                                  int nsc, int tokens, int ntb, int spw, int nwg) {
  constexpr int NTOK = 16 * NT;
  constexpr int BPIECES = NTOK * 16;  // 16-byte activation pieces per superchunk
  constexpr int BPT = BPIECES / 256;  // per staging thread (the first 256)
  constexpr int D = kDepth<NT>;
  __shared__ v4u lds_b[2][BPIECES];
  extern __shared__ float lds_x[];  // d_x of the block's tokens, [superchunk][token]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, qd = lane >> 4;
  const int id = blockIdx.x;
  const int grp = id / (8 * ntb), rem = id % (8 * ntb);
  const int unit = grp * 8 + (rem % 8);
  const int tb = rem / 8;
  if (unit >= (BAL ? nwg : ntiles)) return;  // padding of the last group of 8 (uniform)
  int tile = unit, rb = wv;
  bool active = true;  // this wave owns a 16-row block
  if (BAL) {
    // XCD x = unit % 8 (the dispatch order) gets blocks [x nblk / 8,
    // (x + 1) nblk / 8), split over its nwg / 8 workgroups, so that every XCD
    // and every compute unit gets the same share
    const int nblk = 4 * ntiles, x = unit & 7, l = unit >> 3, nx = nwg >> 3;
    const int x0 = x * nblk / 8, xn = (x + 1) * nblk / 8 - x0;
    const int base = xn / nx, extra = xn - base * nx;  // the first `extra` workgroups take one more
    const int b0 = x0 + base * l + min(l, extra), nb = base + (l < extra ? 1 : 0);
    active = wv < nb;
    const int b = b0 + min(wv, nb - 1);
    tile = b >> 2;
    rb = b & 3;
  }
  const bool stager = tid < 256;
  if (BAL && !active && !stager) {
    // a fifth wave without a block: only the per-superchunk barriers
    for (int j = 0; j < nsc; ++j) __syncthreads();
    return;
  }
  const int tok0 = tb * NTOK;
  const int K = nsc * 256, G = 2 * nsc;

  const v4u* a_src = codes + (size_t)tile * nsc * 256 + qd * 64 + 16 * rb + l16;                      // + sc * 256
  const v4u* s_src = reinterpret_cast<const v4u*>(scales + (size_t)tile * nsc * 64 + 16 * rb + 4 * qd);  // + sc * 16
  const int8_t* b_src[BPT];
  int b_dst[BPT];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int slot = k * 256 + (tid & 255);  // the fifth wave re-reads the first's pieces and stores none
    const int t = slot >> 4, p = slot & 15;
    b_src[k] = q + (size_t)min(tok0 + t, tokens - 1) * K + 16 * p;  // + sc * 256
    b_dst[k] = t * 16 + (p ^ (t & 15));
  }
  v4u ra[D], rs[D], rbv[D][BPT];
  // Fetches past the last superchunk read cache-resident activation bytes in
  // place of codes and scales (no HBM traffic); every load stays
  // unconditional so that the wait counts stay exact.
  const v4u* dummy = reinterpret_cast<const v4u*>(q) + (tid & 15);
#define TQ_FETCH(J, SC)                                                                  \
  {                                                                                      \
    const bool real = (SC) < nsc;                                                        \
    const int scf = min((SC), nsc - 1);                                                  \
    ra[J] = __builtin_nontemporal_load(real ? a_src + (size_t)scf * 256 : dummy);        \
    rs[J] = *(real ? s_src + (size_t)scf * 16 : dummy);                                  \
    _Pragma("unroll") for (int k = 0; k < BPT; ++k) rbv[J][k] =                          \
        *reinterpret_cast<const v4u*>(b_src[k] + (size_t)scf * 256);                     \
  }

  // yacc sums the superchunks of one run of spw, ytot the finished runs in
  // order: the summation order of the matrix-vector product (one run per
  // wave, waves added in order), so each token's output is bit-identical to
  // a tq_gemv call without a workspace
  double yacc[NT][4], ytot[NT][4];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v) yacc[n][v] = ytot[n][v] = 0.0;
  auto fold_run = [&](int j) __attribute__((always_inline)) {
    if (j + 1 == nsc || (j + 1) % spw == 0) {  // uniform
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          ytot[n][v] = j < spw ? yacc[n][v] : ytot[n][v] + yacc[n][v];
          yacc[n][v] = 0.0;
        }
    }
  };

  auto compute = [&](int buf, const v4u c4, const v4u s4, int sc) __attribute__((always_inline)) {
    v4i acc[2][NT];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[hh][n] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v4i a = expand64(c4[c]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const v4i b = __builtin_bit_cast(v4i, lds_b[buf][(16 * n + l16) * 16 + ((4 * c + qd) ^ l16)]);
        acc[c >> 1][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c >> 1][n], 0, 0, 0);
      }
    }
    // lane holds rows 16 rb + 4 qd + v and token 16 n + l16
    if (IDOTS) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = tile * 64 + 16 * rb + 4 * qd + v;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int t = tok0 + 16 * n + l16;
          if (t < tokens && row < rows) {
            int32_t* o = idots + ((size_t)t * rows + row) * G + 2 * sc;
            o[0] = acc[0][n][v] >> 6;
            o[1] = acc[1][n][v] >> 6;
          }
        }
      }
    } else {
      double xd[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) xd[n] = (double)lds_x[sc * NTOK + 16 * n + l16] * 0.015625;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double d0 = lo_half(s4[v]), d1 = hi_half(s4[v]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const double inner = __builtin_fma(d1, (double)acc[1][n][v], d0 * (double)acc[0][n][v]);
          yacc[n][v] = __builtin_fma(xd[n], inner, yacc[n][v]);
        }
      }
    }
  };

  // d_x of every superchunk for the block's tokens, copied into LDS once (the
  // group-dot variant has no d_x).  The first 4 * 256 values are loaded into
  // registers ahead of the ring's first fetches (an index past the end
  // re-copies the last value: same bits, same place, no branch); the rest, for
  // long rows only, after them.
  constexpr int XPT = 4;
  const int nx = nsc * NTOK;
  float xr[XPT];
  auto x_at = [&](int i) { return dx[(size_t)min(tok0 + i % NTOK, tokens - 1) * nsc + i / NTOK]; };
  if (!IDOTS) {
#pragma unroll
    for (int k = 0; k < XPT; ++k) xr[k] = x_at(min(tid + 256 * k, nx - 1));
  }

  // Step J of a pass: publish superchunk j's activations in LDS buffer j & 1,
  // multiply, then fetch superchunk j + D into the freed ring slot.  The
  // barrier also guarantees that every wave is done with buffer j & 1 from
  // two steps back before it is overwritten (and, at the first step, that
  // the d_x copy is complete).
#define TQ_STEP(J, LIVE)                                                                \
  {                                                                                     \
    const int j = base + J;                                                             \
    if (LIVE) {                                                                         \
      const int buf = j & 1;                                                            \
      if (stager) {                                                                     \
        _Pragma("unroll") for (int k = 0; k < BPT; ++k) lds_b[buf][b_dst[k]] = rbv[J][k]; \
      }                                                                                 \
      __syncthreads();                                                                  \
      if (active) {                                                                     \
        compute(buf, ra[J], rs[J], j);                                                  \
        if (!IDOTS) fold_run(j);                                                        \
      }                                                                                 \
    }                                                                                   \
    TQ_FETCH(J, j + D)                                                                  \
  }

  TQ_FETCH(0, 0) TQ_FETCH(1, 1)
  if constexpr (D > 2) { TQ_FETCH(2, 2) TQ_FETCH(3, 3) }
  if (!IDOTS) {
#pragma unroll
    for (int k = 0; k < XPT; ++k) lds_x[min(tid + 256 * k, nx - 1)] = xr[k];
    for (int i = tid + 256 * XPT; i < nx; i += 256) lds_x[i] = x_at(i);
  }
  int base = 0;
  for (; base + 2 * D <= nsc; base += D) {
    TQ_STEP(0, true) TQ_STEP(1, true)
    if constexpr (D > 2) { TQ_STEP(2, true) TQ_STEP(3, true) }
  }
  for (; base < nsc; base += D) {
    TQ_STEP(0, j < nsc) TQ_STEP(1, j < nsc)
    if constexpr (D > 2) { TQ_STEP(2, j < nsc) TQ_STEP(3, j < nsc) }
  }
#undef TQ_STEP
#undef TQ_FETCH

  if (IDOTS || !active) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = tile * 64 + 16 * rb + 4 * qd + v;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = tok0 + 16 * n + l16;
      if (row < rows && t < tokens) y[(size_t)t * rows + row] = (float)ytot[n][v];
    }
  }
}
static_assert(kDepth<1> == 4 && kDepth<2> == 2, "the passes in gemm_pq2_kernel are written out for two or four steps");

template <int NT, bool BAL>
hipError_t launch_gemm_ntb(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s) {
  const int nsc = (int)dm.nsc;
  const int ntb = (int)((tokens + 16 * NT - 1) / (16 * NT));
  const int nwg = BAL ? kBalancedWgs : (int)dm.ntiles;
  const int64_t groups = (nwg + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * ntb)), block(BAL ? 320 : 256);
  const v4u* codes = reinterpret_cast<const v4u*>(w);
  const uint32_t* scales = reinterpret_cast<const uint32_t*>(w + pq2_code_bytes(dm));
  // the run length of the matrix-vector product without a workspace
  const int spw = plan_gemv_pq2(dm, false).spw;
  if (idots)
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, true, BAL>), grid, block, 0, s, codes, scales, q, dx, y, idots,
                       (int)dm.rows, (int)dm.ntiles, nsc, (int)tokens, ntb, spw, nwg);
  else
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, false, BAL>), grid, block, (unsigned)gemm_dx_bytes(nsc, NT), s, codes,
                       scales, q, dx, y, idots, (int)dm.rows, (int)dm.ntiles, nsc, (int)tokens, ntb, spw, nwg);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_gemm_nt(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                          int32_t* idots, hipStream_t s) {
  // a little over 256 tiles: the balanced grid (4 or 5 row blocks per
  // workgroup, 256 workgroups per token block)
  if (dm.ntiles > kBalancedWgs && dm.ntiles * 4 <= kBalancedWgs * 5)
    return launch_gemm_ntb<NT, true>(w, dm, tokens, q, dx, y, idots, s);
  return launch_gemm_ntb<NT, false>(w, dm, tokens, q, dx, y, idots, s);
}

}  // namespace

hipError_t launch_gemm_pq2(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s) {
  // 16-token blocks up to 32 tokens, 32-token blocks beyond (measured on the
  // 17408 x 5120 prompt shape: the 16-token kernel has more independent
  // workgroups per CU, the 32-token one shares each code expansion and scale
  // conversion between twice the tokens)
  const int nt = tokens <= 32 ? 1 : 2;
  if (gemm_dx_bytes((int)dm.nsc, nt) > kMaxDxBytes) {
    // rows longer than the d_x copy allows: one matrix-vector product per token
    for (int64_t t = 0; t < tokens; ++t) {
      const hipError_t e = launch_gemv_pq2(w, dm, q + t * dm.cols, dx + t * dm.nsc, y + t * dm.rows,
                                           idots ? idots + t * dm.rows * 2 * dm.nsc : nullptr, nullptr, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // One launch covers at most 2^22 workgroups (row-tile groups x token
  // blocks, so that the grid stays far below 2^32 work-items); longer prompts
  // go in chunks of whole token blocks, each with its tokens' activations and
  // outputs.  The token blocking does not change the summation order.
  const int64_t wgs_per_block = std::max<int64_t>(dm.ntiles, kBalancedWgs) + 7;
  const int64_t chunk = std::max<int64_t>(1, (int64_t(1) << 22) / wgs_per_block) * 16 * nt;
  for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
    const int64_t tc = std::min(chunk, tokens - t0);
    const int8_t* qc = q + t0 * dm.cols;
    const float* dxc = dx ? dx + t0 * dm.nsc : nullptr;
    float* yc = y ? y + t0 * dm.rows : nullptr;
    int32_t* ic = idots ? idots + t0 * dm.rows * 2 * dm.nsc : nullptr;
    const hipError_t e = nt == 1 ? launch_gemm_nt<1>(w, dm, tc, qc, dxc, yc, ic, s)
                                 : launch_gemm_nt<2>(w, dm, tc, qc, dxc, yc, ic, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
