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
//   * Workgroup = 4 waves on one 64-row tile and 16 * NT tokens.  The
//     superchunks (256 columns) stream through the workgroup: every thread
//     loads its share of a superchunk (16 bytes of codes, NT x 16 activation
//     bytes, its rows' scale pairs and its tokens' d_x) ahead of use into
//     rings of registers -- codes, scales and d_x twelve superchunks ahead,
//     the activations (L2 hits) six -- then stores them into one of two LDS
//     buffers, one barrier per superchunk.  The loads are
//     unconditional, so the compiler's wait counts stay exact and the rings
//     really hide the memory latency.
//   * Wave w owns row block w (16 rows) for all tokens: A operand = one dword
//     of its codes expanded with one shift and one mask per field into the
//     16 int8 values 64*w (columns 64c + 16qd + [0, 16) for chunk c), exactly
//     one A operand of v_mfma_i32_16x16x64_i8; B operand = 16 activation
//     bytes read from LDS.  Activations are fetched token-row by token-row
//     (coalesced) and stored [token][16-byte piece], the piece index
//     XOR-swizzled by the token so that neither the stores nor the operand
//     reads (16 tokens, same piece) hit the same LDS banks.
//   * The MFMA accumulators restart every 128-group (two chunks) because the
//     weight scale changes per group; the group epilogue converts the integer
//     sum to fp64 and accumulates (d_w / 64) * d_x * sum in fp64 (every term
//     exact; the 1/64 of the two's-complement codes folded into d_w).
//   * Tokens past the end read a valid row (the last token) and are never
//     stored.
#include "kernels.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
// Native vector types (not HIP's uint4 struct) keep copies in registers.
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;

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

__device__ __forceinline__ uint32_t pick(const v4u v, int c) { return v[c]; }

}  // namespace

template <int NT, bool IDOTS>
__global__ __launch_bounds__(64 * kWaves) void gemm_pq2_kernel(const uint4* __restrict__ codes,
                                                              const uint32_t* __restrict__ scales,
                                                              const int8_t* __restrict__ q, const float* __restrict__ dx,
                                                              float* __restrict__ y, int32_t* __restrict__ idots,
                                                              int rows, int nsc, int tokens) {
  __shared__ v4u lds_a[2][256];              // codes: [qd][row] x 16 B, as in global memory
  __shared__ v4u lds_b[2][16 * NT * 16];     // activations: [token][piece ^ (token & 15)] x 16 B
  __shared__ uint32_t lds_s[2][64];          // scale pair (groups 2 sc, 2 sc + 1) of each row
  __shared__ float lds_x[2][64];             // d_x of each token of the tile (padded to 64)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x;
  const int tok0 = blockIdx.y * (16 * NT);
  const int l16 = lane & 15;
  const int qd = lane >> 4;
  const int K = nsc * 256;
  const int G = nsc * 2;

  // ---- per-thread sources (offsets per superchunk added at fetch time)
  const v4u* a_src = reinterpret_cast<const v4u*>(codes) + (size_t)tile * nsc * 256 + tid;  // + sc * 256
  // Activations: 16 consecutive threads read one token's 256 bytes (piece p =
  // 16-byte column block, = 4 c + qd of the MFMA operand); they are stored at
  // LDS slot token * 16 + (p ^ (token & 15)), which keeps both these stores
  // and the operand reads (16 tokens, one piece) free of bank conflicts.
  const int8_t* b_src[NT];
  int b_dst[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int slot = k * 256 + tid;
    const int t = slot >> 4, p = slot & 15;
    const int tt = min(tok0 + t, tokens - 1);
    b_src[k] = q + (size_t)tt * K + 16 * p;  // + sc * 256
    b_dst[k] = t * 16 + (p ^ (t & 15));
  }
  // One extra dword per thread and superchunk: threads 64..127 fetch the d_x of
  // token tid - 64 (of the tile, clamped to a valid token), the others the
  // scale pair of row tid & 63 (only threads 0..63 keep theirs).  The load is
  // unconditional for every thread.
  const bool x_thread = !IDOTS && tid >= 64 && tid < 128;
  const uint32_t* sx_src = x_thread ? reinterpret_cast<const uint32_t*>(dx) +
                                          (size_t)min(tok0 + min(tid - 64, 16 * NT - 1), tokens - 1) * nsc  // + sc
                                    : scales + (size_t)tile * nsc * 64 + lane;                             // + sc * 64
  const int sx_step = x_thread ? 1 : 64;

  // Register rings.  The weight codes (the HBM stream, 4 VGPRs per stage) and
  // the scale / d_x dword are fetched twelve superchunks ahead, so that ~48 KiB
  // per CU are in flight; the activations (L2 hits, 4 NT VGPRs per stage) six
  // ahead.  Every ring index is a literal, so the rings stay in VGPRs and the
  // compiler's waits stay exact.
  constexpr int kDepthA = 12, kDepthB = 6;
  v4u ra[kDepthA], rb[kDepthB][NT];
  uint32_t rsx[kDepthA];
#define TQ_FETCH_A(J, SC)                                                                 \
  {                                                                                       \
    const int scf = min((SC), nsc - 1); /* past the end: reload the last one (unused) */ \
    ra[J] = a_src[(size_t)scf * 256];                                                     \
    rsx[J] = sx_src[(size_t)scf * sx_step];                                               \
  }
#define TQ_FETCH_B(J, SC)                                                                 \
  {                                                                                       \
    const int scf = min((SC), nsc - 1);                                                   \
    _Pragma("unroll") for (int k = 0; k < NT; ++k) rb[J][k] =                             \
        *reinterpret_cast<const v4u*>(b_src[k] + (size_t)scf * 256);                      \
  }

  double yacc[NT][4];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v) yacc[n][v] = 0.0;

  auto compute = [&](int buf, int sc) __attribute__((always_inline)) {
    const v4u codes4 = lds_a[buf][qd * 64 + wave * 16 + l16];
    const v4u s4 = *reinterpret_cast<const v4u*>(&lds_s[buf][wave * 16 + 4 * qd]);
    const uint32_t sp[4] = {s4[0], s4[1], s4[2], s4[3]};
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // group g = 2 sc + half: chunks c = 2 half, 2 half + 1
      v4i acc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = 2 * half + cc;
        const v4i a = expand64(pick(codes4, c));
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const v4i b = __builtin_bit_cast(v4i, lds_b[buf][(16 * n + l16) * 16 + ((4 * c + qd) ^ l16)]);
          acc[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[n], 0, 0, 0);
        }
      }
      // lane holds rows 16 wave + 4 qd + v and token 16 n + l16
      const int g = 2 * sc + half;
      if (IDOTS) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = tile * 64 + wave * 16 + 4 * qd + v;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int t = tok0 + 16 * n + l16;
            if (t < tokens && row < rows) idots[((size_t)t * rows + row) * G + g] = acc[n][v] >> 6;
          }
        }
      } else {
        double xd[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) xd[n] = (double)lds_x[buf][16 * n + l16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // (d_w / 64): exact, it removes the factor 64 of the codes
          const double dw = (double)half_bits_to_float(half ? (sp[v] >> 16) : (sp[v] & 0xffffu)) * 0.015625;
#pragma unroll
          for (int n = 0; n < NT; ++n) yacc[n][v] += (dw * xd[n]) * (double)acc[n][v];
        }
      }
    }
  };

  // One superchunk: publish its codes, activations, scales and d_x in LDS
  // buffer sc & 1, multiply, then refill both ring slots (twelve and six
  // ahead).  The barrier also guarantees that every wave is done with buffer
  // sc & 1 from two steps back before it is overwritten.
#define TQ_STEP(J, JA, JB)                                                        \
  {                                                                               \
    const int scj = sc + J;                                                       \
    const int buf = scj & 1;                                                      \
    lds_a[buf][tid] = ra[JA];                                                     \
    _Pragma("unroll") for (int k = 0; k < NT; ++k) lds_b[buf][b_dst[k]] = rb[JB][k];     \
    if (tid < 64) lds_s[buf][tid] = rsx[JA];                                      \
    else if (tid < 128) lds_x[buf][tid - 64] = __builtin_bit_cast(float, rsx[JA]); \
    __syncthreads();                                                              \
    if (scj < nsc) compute(buf, scj);                                             \
    TQ_FETCH_A(JA, scj + kDepthA)                                                 \
    TQ_FETCH_B(JB, scj + kDepthB)                                                 \
  }

  {
    const int sc = 0;
    TQ_FETCH_A(0, sc) TQ_FETCH_A(1, sc + 1) TQ_FETCH_A(2, sc + 2) TQ_FETCH_A(3, sc + 3)
    TQ_FETCH_A(4, sc + 4) TQ_FETCH_A(5, sc + 5) TQ_FETCH_A(6, sc + 6) TQ_FETCH_A(7, sc + 7)
    TQ_FETCH_A(8, sc + 8) TQ_FETCH_A(9, sc + 9) TQ_FETCH_A(10, sc + 10) TQ_FETCH_A(11, sc + 11)
    TQ_FETCH_B(0, sc) TQ_FETCH_B(1, sc + 1) TQ_FETCH_B(2, sc + 2)
    TQ_FETCH_B(3, sc + 3) TQ_FETCH_B(4, sc + 4) TQ_FETCH_B(5, sc + 5)
  }
  for (int sc = 0; sc < nsc; sc += kDepthA) {
    TQ_STEP(0, 0, 0) TQ_STEP(1, 1, 1) TQ_STEP(2, 2, 2) TQ_STEP(3, 3, 3)
    TQ_STEP(4, 4, 4) TQ_STEP(5, 5, 5) TQ_STEP(6, 6, 0) TQ_STEP(7, 7, 1)
    TQ_STEP(8, 8, 2) TQ_STEP(9, 9, 3) TQ_STEP(10, 10, 4) TQ_STEP(11, 11, 5)
  }
#undef TQ_STEP
#undef TQ_FETCH_A
#undef TQ_FETCH_B

  if (IDOTS) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = tile * 64 + wave * 16 + 4 * qd + v;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = tok0 + 16 * n + l16;
      if (row < rows && t < tokens) y[(size_t)t * rows + row] = (float)yacc[n][v];
    }
  }
}

template <int NT>
hipError_t launch_gemm_nt(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                          int32_t* idots, hipStream_t s) {
  const int nsc = (int)dm.nsc;
  const dim3 grid((unsigned)dm.ntiles, (unsigned)((tokens + 16 * NT - 1) / (16 * NT))), block(64 * kWaves);
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint32_t* scales = reinterpret_cast<const uint32_t*>(w + pq2_code_bytes(dm));
  if (idots)
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, true>), grid, block, 0, s, codes, scales, q, dx, y, idots, (int)dm.rows, nsc,
                       (int)tokens);
  else
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, false>), grid, block, 0, s, codes, scales, q, dx, y, idots, (int)dm.rows, nsc,
                       (int)tokens);
  return hipGetLastError();
}

template hipError_t launch_gemm_nt<1>(const uint8_t*, const Dims&, int64_t, const int8_t*, const float*, float*, int32_t*, hipStream_t);
template hipError_t launch_gemm_nt<2>(const uint8_t*, const Dims&, int64_t, const int8_t*, const float*, float*, int32_t*, hipStream_t);
template hipError_t launch_gemm_nt<4>(const uint8_t*, const Dims&, int64_t, const int8_t*, const float*, float*, int32_t*, hipStream_t);

hipError_t launch_gemm_pq2(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s) {
  if (tokens <= 16) return launch_gemm_nt<1>(w, dm, tokens, q, dx, y, idots, s);
  if (tokens <= 32) return launch_gemm_nt<2>(w, dm, tokens, q, dx, y, idots, s);
  return launch_gemm_nt<4>(w, dm, tokens, q, dx, y, idots, s);
}

}  // namespace tq
