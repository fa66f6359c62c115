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
//   * v_mfma_i32_16x16x64_i8 on 16 tokens x 16 rows x 64 columns: lane
//     (r, qd) = (lane % 16, lane / 16) supplies the columns 16 qd .. 16 qd + 15
//     of each 64-column step for row r and for the token in MFMA row r.  The
//     row side comes from one 16-byte code load per row block and superchunk
//     (dword c = step c, one shift and one mask per 2-bit field); the token
//     side is 16 bytes of q per token.  Token t of a block of 16 sits in MFMA
//     row 4 (t % 4) + t / 4, so result slot v of lane (r, qd) holds token
//     4 v + qd: with at most 4 (8) tokens only slot 0 (slots 0 and 1) hold
//     real tokens, and the epilogue and the final run sums skip the others.
//   * Work split.  The matrix-vector product sums each row's superchunks in
//     runs (one run per wave of its plan without a workspace) and adds the
//     runs in order.  Here each wave owns one run, for all the row blocks
//     and tokens of its workgroup: no two waves read the same codes or
//     activations; at the end the workgroup adds its runs in run order
//     through LDS, so every token's output is the matrix-vector product's,
//     bit for bit.
//   * Rows: the 16-row blocks of the matrix are split into contiguous,
//     nearly equal ranges.  Up to 16 tokens: ranges of at most 3 blocks, at
//     least 512 of them, two workgroups per compute unit.  17 to 48 tokens:
//     ranges of at most 5 blocks, at least 256, each range once per group of
//     16 tokens.  More: the same ranges once per group of 32 tokens, again
//     two workgroups per compute unit.  A wave's fp64 sums (5 row blocks x
//     32 tokens) fill a third of its registers.
//   * Data flow per wave: every operand (codes, scale pairs, activations,
//     d_x) streams through a ring of RD superchunks in registers by raw
//     buffer loads: a per-lane offset, a uniform offset and a resource over
//     just this workgroup's rows or tokens, so a load costs no address
//     arithmetic, and a load that must not happen (a superchunk past the
//     run, a row block past the range, a token past the end) reads an empty
//     or short resource and returns zeros without touching memory.  All
//     loads are unconditional, so the compiler's wait counts follow the ring
//     slot by slot.  With 16-token groups (up to 48 tokens) the activations
//     (cache hits) have a ring of their own, one slot deep and issued ahead
//     of the codes.
//   * Epilogue per superchunk, in fp64 (every product exact, sums rounded
//     once per operation): inner = d_w(2sc+1) * I1 + d_w(2sc) * I0, then
//     y += (d_x / 64) * inner; the MFMA sums are 64 I (two's-complement codes
//     masked to the top two bits of each byte), and the 1/64 is exact.
//   * What bounds it: the epilogue (5 fp64-pipe instructions per row, token
//     and superchunk) and the code expansion (7 per code dword and token
//     group) are VALU work that no layout removes; at 64 tokens they exceed
//     the time to stream the codes from HBM.
//   * Rows past the end have zero codes and scales; tokens past the end
//     read zeros and are never stored.
#include <algorithm>

#include "kernels.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
// Native vector types (not HIP's uint4 struct) keep copies in registers.
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kMaxRb = 5;           // 16-row blocks per workgroup (at most, over all variants)
constexpr int kMaxRuns = 4;         // waves per workgroup: the matrix-vector plan's runs
constexpr int kRbSmall = 3;         // blocks per workgroup at up to 16 tokens (two workgroups per compute unit)
constexpr int kMinRowGroups = 256;  // one row range per compute unit where the blocks allow

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

typedef __amdgpu_buffer_rsrc_t buf_t;
// A raw buffer resource over `bytes` bytes at p (stride 0, 32-bit data
// format word of gfx9-family targets).
__device__ __forceinline__ buf_t make_buf(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ v4u load16(buf_t r, int voff, int soff) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Streamed once: non-temporal.
__device__ __forceinline__ v4u load16_nt(buf_t r, int voff, int soff) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ uint32_t load4(buf_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Launch geometry, shared by host and device.
struct GemmShape {
  int nrg;    // row ranges (workgroups per token group), a multiple of 8 with padding
  int nreal;  // real row ranges
  int base;   // blocks per range: base, the first `extra` ranges one more
  int extra;
  int ntg;    // token groups of 16 NT tokens
};

// grid = 1-D, nrg * ntg workgroups, the token groups of one row range on one
// XCD (workgroup id modulo 8), so that their code reads after the first hit
// that XCD's L2: id = ((rg / 8) * ntg + tg) * 8 + rg % 8.
// Block = nruns waves; wave w sums superchunks [w spw, min(nsc, (w + 1) spw)).
// The MFMA's first operand is the activations (16 tokens x 64 columns), the
// second the expanded codes (64 columns x 16 rows): lane (l16, qd) of the
// result holds tokens qd, 4 + qd, 8 + qd, 12 + qd of row l16 (slots 0..VT-1
// of them are used), so a lane needs one scale pair per row block, and 16
// consecutive rows of a token are stored together.
// Every operand streams through a ring of RD superchunks in registers.
template <int NT, int RD, bool SPLIT, int MRB, int VT, bool IDOTS>
__global__ __launch_bounds__(64 * kMaxRuns, IDOTS ? 1 : 2) void gemm_pq2_kernel(
    const v4u* __restrict__ codes, const int8_t* __restrict__ q,
    const float* __restrict__ dx, float* __restrict__ y, int32_t* __restrict__ idots, int rows, int nsc, int tokens,
    int spw, GemmShape gs) {
  static_assert(VT == 1 || VT == 2 || VT == 4, "result slots per lane");
  constexpr int kAcc = MRB * NT * VT;  // fp64 sums per lane
  extern __shared__ double sums[];       // run sums of one phase [wave][kPer][lane]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nruns = blockDim.x >> 6;
  const int l16 = lane & 15, qd = lane >> 4;
  const int id = blockIdx.x;
  const int grp = id / (8 * gs.ntg), rem = id % (8 * gs.ntg);
  const int rg = grp * 8 + (rem % 8), tg = rem / 8;
  if (rg >= gs.nreal) return;  // padding of the last group of 8 (whole workgroup)
  const int b0 = rg * gs.base + min(rg, gs.extra);
  const int nrb = gs.base + (rg < gs.extra ? 1 : 0);  // uniform, 1..MRB
  const int K = nsc * 256, G = 2 * nsc;
  const int sc0 = wave * spw;
  const int n = min(nsc, sc0 + spw) - sc0;  // superchunks of this wave's run (>= 1)
  const int tok0 = tg * 16 * NT;

  // Raw buffer loads: a resource over this workgroup's own rows (at most two
  // tiles) or tokens, a per-lane VGPR offset and a uniform SGPR offset, so no
  // per-load address arithmetic.  A lane whose offset lies past the
  // resource's size reads 0 without a memory access: tokens past the end, and
  // every load of `none` (size 0), which stands in for superchunks past the
  // run and row blocks past nrb.  Every load is then unconditional.
  const int tile0 = b0 >> 2;
  const int ntl = min(2, (rows + 63) / 64 - tile0);  // tiles of this row range
  const int ntok = min(16 * NT, tokens - tok0);
  const buf_t none = make_buf(codes, 0);
  // units (tile, sc) of kPq2UnitBytes: codes, then the scale pairs
  constexpr int kUnit = (int)kPq2UnitBytes;
  const uint8_t* units = reinterpret_cast<const uint8_t*>(codes) + (size_t)tile0 * nsc * kUnit;
  const buf_t a_buf = make_buf(units, ntl * nsc * kUnit);
  const buf_t s_buf = make_buf(units + kPq2ScaleOffset, ntl * nsc * kUnit - (int)kPq2ScaleOffset);
  const buf_t b_buf = make_buf(q + (size_t)tok0 * K, ntok * K);
  const buf_t x_buf = make_buf(dx + (size_t)tok0 * nsc, ntok * nsc * 4);
  // byte offsets: codes of row block i at superchunk sc are at a_off[i] +
  // kUnit sc, lane (l16, qd) reading 16 bytes at (64 qd + l16) * 16; its
  // scale pair at s_off[i] + kUnit sc + 4 l16; token block nb's activations at
  // (16 nb + trow) K + 16 qd + 256 sc + 64 c, trow the token in MFMA row l16;
  // d_x of token `lane` at 4 (lane nsc + sc), lanes past 16 NT out of range
  int a_off[MRB], s_off[MRB];
#pragma unroll
  for (int i = 0; i < MRB; ++i) {
    const int b = b0 + i, tl = (b >> 2) - tile0, rbi = b & 3;
    a_off[i] = tl * nsc * kUnit + 16 * rbi * 16;
    s_off[i] = tl * nsc * kUnit + 16 * rbi * 4;
  }
  const int a_lane = (64 * qd + l16) * 16, s_lane = 4 * l16;
  const int trow = 4 * (l16 & 3) + (l16 >> 2);
  const int x_lane = lane < 16 * NT ? 4 * lane * nsc : 0x7fffff00;

  // Ring slots: RD for the codes and scales; RD for the activations and d_x,
  // or one with SPLIT (see the loop below).
  constexpr int RA = SPLIT ? 1 : RD;
  v4u ra[RD][MRB];
  uint32_t rs[RD][MRB];
  v4u rb[RA][NT][4];
  float rx[RA];
  // Loads of superchunk k: its codes and scale pairs into code slot J and/or
  // its activations and d_x into activation slot JA (one lambda: two nested
  // ones made the compiler keep 58 more VGPRs live).
  auto fetch = [&](int J, int JA, int k, bool codes, bool acts) __attribute__((always_inline)) {
    const bool real = k < n;  // uniform
    const int sc = sc0 + k;
    if (codes) {
#pragma unroll
      for (int i = 0; i < MRB; ++i) {
        const bool use = real && i < nrb;
        ra[J][i] = load16_nt(use ? a_buf : none, a_lane, a_off[i] + kUnit * sc);
        if (!IDOTS) rs[J][i] = load4(use ? s_buf : none, s_lane, s_off[i] + kUnit * sc);
      }
    }
    if (acts) {
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) {
        const int vo = (16 * nb + trow) * K + 16 * qd;
#pragma unroll
        for (int c = 0; c < 4; ++c) rb[JA][nb][c] = load16(real ? b_buf : none, vo + 64 * c, 256 * sc);
      }
      if (!IDOTS) rx[JA] = __builtin_bit_cast(float, load4(real ? x_buf : none, x_lane, 4 * sc));
    }
  };

  double yacc[MRB][NT][VT];
#pragma unroll
  for (int i = 0; i < MRB; ++i)
#pragma unroll
    for (int nb = 0; nb < NT; ++nb)
#pragma unroll
      for (int v = 0; v < VT; ++v) yacc[i][nb][v] = 0.0;

  // superchunk j from code slot J and activation slot JA
  auto step = [&](int J, int JA, int j) __attribute__((always_inline)) {
    double xd[NT][VT];
    if (!IDOTS) {
      // d_x of token 16 nb + 4 v + qd, from the lane that loaded it
      const int xi = __builtin_bit_cast(int, rx[JA]);
#pragma unroll
      for (int nb = 0; nb < NT; ++nb)
#pragma unroll
        for (int v = 0; v < VT; ++v)
          xd[nb][v] = (double)__builtin_bit_cast(float, __shfl(xi, 16 * nb + 4 * v + qd, 64)) * 0.015625;
    }
    const int sc = sc0 + j;
#pragma unroll
    for (int i = 0; i < MRB; ++i) {
      if (i >= nrb) continue;  // uniform
      v4i acc[NT][2];
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) acc[nb][0] = acc[nb][1] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const v4i a = expand64(ra[J][i][c]);
#pragma unroll
        for (int nb = 0; nb < NT; ++nb)
          acc[nb][c >> 1] =
              __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, rb[JA][nb][c]), a, acc[nb][c >> 1], 0, 0, 0);
      }
      const int row = (b0 + i) * 16 + l16;
      if (IDOTS) {
#pragma unroll
        for (int nb = 0; nb < NT; ++nb)
#pragma unroll
          for (int v = 0; v < VT; ++v) {
            const int t = tok0 + 16 * nb + 4 * v + qd;
            if (t < tokens && row < rows) {
              int32_t* o = idots + ((size_t)t * rows + row) * G + 2 * sc;
              o[0] = acc[nb][0][v] >> 6;
              o[1] = acc[nb][1][v] >> 6;
            }
          }
      } else {
        const double d0 = lo_half(rs[J][i]), d1 = hi_half(rs[J][i]);
#pragma unroll
        for (int nb = 0; nb < NT; ++nb)
#pragma unroll
          for (int v = 0; v < VT; ++v) {
            const double inner = __builtin_fma(d1, (double)acc[nb][1][v], d0 * (double)acc[nb][0][v]);
            yacc[i][nb][v] = __builtin_fma(xd[nb][v], inner, yacc[i][nb][v]);
          }
      }
    }
  };

  // The ring is indexed by literal slots: the prologue fills it, each pass of
  // the loop consumes slots 0 .. RD-1 and refills each RD superchunks ahead,
  // and the last n mod RD superchunks sit in slots 0, 1, ... after it.  No
  // step inside the loop is conditional, so the compiler's wait counts stay
  // per slot instead of draining the ring at a join.  Vector loads complete
  // in issue order, so a wait for one load is a wait for every earlier one.
  //   * Plain: superchunk k's codes then its activations, RD ahead.
  //   * SPLIT: the codes RD ahead, the activations (cache hits, one slot) one
  //     ahead and issued before the codes of the same pass, so that waiting
  //     for them never waits for the codes' HBM round trip.
  const int full = n / RD;
  const int left = n - full * RD;
  if constexpr (!SPLIT) {
#pragma unroll
    for (int J = 0; J < RD; ++J) fetch(J, J, J, true, true);
    for (int c = 0; c < full; ++c) {
#pragma unroll
      for (int J = 0; J < RD; ++J) {
        step(J, J, c * RD + J);
        fetch(J, J, c * RD + J + RD, true, true);
      }
    }
#pragma unroll
    for (int J = 0; J + 1 < RD; ++J)
      if (J < left) step(J, J, full * RD + J);  // uniform
  } else {
    fetch(0, 0, 0, true, true);
#pragma unroll
    for (int J = 1; J < RD; ++J) fetch(J, 0, J, true, false);
    for (int c = 0; c < full; ++c) {
#pragma unroll
      for (int J = 0; J < RD; ++J) {
        step(J, 0, c * RD + J);
        fetch(J, 0, c * RD + J + 1, false, true);
        fetch(J, 0, c * RD + J + RD, true, false);
      }
    }
#pragma unroll
    for (int J = 0; J + 1 < RD; ++J)
      if (J < left) {  // uniform
        step(J, 0, full * RD + J);
        fetch(J, 0, full * RD + J + 1, false, true);
      }
  }
  if (IDOTS) return;

  // Runs added in run order: y = ((s0 + s1) + s2) + s3, each token's order in
  // the matrix-vector product.  In each of kPh phases every wave stores its
  // sums of a share of the (row block, token block, v) slots; wave w then
  // finishes every nruns-th slot of that share.
  constexpr int kPh = kAcc > 20 ? 2 : 1;  // two phases halve the LDS
  constexpr int kPer = kAcc / kPh;
  static_assert(kAcc % kPh == 0, "phases split the slots evenly");
#pragma unroll
  for (int p = 0; p < kPh; ++p) {
    if (p > 0) __syncthreads();  // the previous phase's reads are done
#pragma unroll
    for (int i = 0; i < MRB; ++i)
#pragma unroll
      for (int nb = 0; nb < NT; ++nb)
#pragma unroll
        for (int v = 0; v < VT; ++v) {
          const int sl = (i * NT + nb) * VT + v;
          if (sl / kPer == p) sums[((size_t)wave * kPer + sl % kPer) * 64 + lane] = yacc[i][nb][v];
        }
    __syncthreads();
    for (int sl = p * kPer + wave; sl < (p + 1) * kPer; sl += nruns) {
      const int i = sl / (NT * VT), nb = (sl / VT) % NT, v = sl % VT;
      if (i >= nrb) continue;
      // every run's sum read before the first add (a read and an add per run
      // waited an LDS round trip each); runs past the last repeat it unused
      double rv[kMaxRuns];
#pragma unroll
      for (int w = 0; w < kMaxRuns; ++w) rv[w] = sums[((size_t)min(w, nruns - 1) * kPer + sl % kPer) * 64 + lane];
      double t = rv[0];
#pragma unroll
      for (int w = 1; w < kMaxRuns; ++w)
        if (w < nruns) t += rv[w];
      const int row = (b0 + i) * 16 + l16, tk = tok0 + 16 * nb + 4 * v + qd;
      if (row < rows && tk < tokens) y[(size_t)tk * rows + row] = (float)t;
    }
  }
}

template <int NT, int MRB, int VT>
size_t gemm_lds_bytes(int nruns) {
  constexpr int acc = MRB * NT * VT;
  return (size_t)nruns * (acc > 20 ? acc / 2 : acc) * 64 * 8;
}

// Row ranges of at most mrb blocks, at least min_groups of them where the
// blocks allow (one or two per compute unit), as even as possible.
GemmShape gemm_shape(const Dims& dm, int64_t tokens, int nt, int mrb, int min_groups) {
  GemmShape gs;
  const int nblk = (int)(4 * dm.ntiles);
  const int want = std::max((nblk + mrb - 1) / mrb, std::min(nblk, min_groups));
  gs.nreal = want;
  gs.base = nblk / want;
  gs.extra = nblk - gs.base * want;
  gs.nrg = (want + 7) / 8 * 8;
  gs.ntg = (int)((tokens + 16 * nt - 1) / (16 * nt));
  return gs;
}

template <int NT, int RD, bool SPLIT, int MRB, int VT>
hipError_t launch_gemm_t(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                         int32_t* idots, int min_groups, hipStream_t s) {
  const GemmShape gs = gemm_shape(dm, tokens, NT, MRB, min_groups);
  const GemvPlan p = plan_gemv_pq2(dm, false);  // the runs of the matrix-vector product
  const int nruns = (int)((dm.nsc + p.spw - 1) / p.spw);
  const dim3 grid((unsigned)((int64_t)gs.nrg * gs.ntg)), block(64 * nruns);
  const size_t lds = gemm_lds_bytes<NT, MRB, VT>(nruns);
  const v4u* codes = reinterpret_cast<const v4u*>(w);
  if (idots)
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, RD, SPLIT, MRB, VT, true>), grid, block, lds, s, codes, q, dx, y, idots,
                       (int)dm.rows, (int)dm.nsc, (int)tokens, p.spw, gs);
  else
    hipLaunchKernelGGL((gemm_pq2_kernel<NT, RD, SPLIT, MRB, VT, false>), grid, block, lds, s, codes, q, dx, y, idots,
                       (int)dm.rows, (int)dm.nsc, (int)tokens, p.spw, gs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_pq2(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, hipStream_t s) {
  static_assert(kMaxRuns == 4, "the matrix-vector plan uses at most 4 waves per row tile");
  // Token groups and row ranges, measured on 17408 x 5120 (2 tokens per
  // point, us): up to 16 tokens one group of 16 over ranges of at most 3
  // blocks (at least 512 ranges), codes two superchunks ahead and
  // activations one (at 4 tokens 7.8 with both two ahead, 7.5 split), and up
  // to 4 (8) tokens only the result slots that hold real tokens are
  // finished; 17 to 48 tokens groups of 16 over ranges of at most 5 blocks
  // (at least 256), two or three groups keeping two workgroups per compute
  // unit (17 / 32 / 48 tokens: 13.5 / 13.7 / 17.9, one or two groups of 32:
  // 14.7 / 15.5 / 19.2); more, groups of 32 (two MFMA blocks) over ranges of
  // at most 5 blocks, one superchunk in flight per wave, the other wave on
  // the SIMD covering its latency (64 tokens: 19.3, groups of 16: 22.4).
  // One launch covers at most 2^22 workgroups (far below 2^32 work-items);
  // longer prompts go in chunks of whole token groups, each with its tokens'
  // activations and outputs.  The token grouping does not change the
  // summation order.  Buffer offsets are 32-bit: the largest, 32 tokens of
  // activations, is 32 cols bytes.
  if (dm.cols > (int64_t(1) << 25)) return hipErrorInvalidValue;
  const int mode = tokens <= 16 ? 0 : tokens <= 48 ? 1 : 2;  // fixed for every chunk
  const int nt = mode == 2 ? 2 : 1;
  const int mrb = mode == 0 ? kRbSmall : kMaxRb;
  const int ranges = mode == 0 ? 2 * kMinRowGroups : kMinRowGroups;
  const int64_t group = 16 * nt;
  const int64_t rgs = gemm_shape(dm, 1, nt, mrb, ranges).nrg;
  const int64_t chunk = std::max<int64_t>(1, (int64_t(1) << 22) / rgs) * group;
  for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
    const int64_t tc = std::min(chunk, tokens - t0);
    const int8_t* qc = q + t0 * dm.cols;
    const float* dxc = dx ? dx + t0 * dm.nsc : nullptr;
    float* yc = y ? y + t0 * dm.rows : nullptr;
    int32_t* ic = idots ? idots + t0 * dm.rows * 2 * dm.nsc : nullptr;
    const hipError_t e =
        mode == 2  ? launch_gemm_t<2, 1, false, kMaxRb, 4>(w, dm, tc, qc, dxc, yc, ic, ranges, s)
        : mode == 1 ? launch_gemm_t<1, 2, true, kMaxRb, 4>(w, dm, tc, qc, dxc, yc, ic, ranges, s)
        : tc <= 4  ? launch_gemm_t<1, 2, true, kRbSmall, 1>(w, dm, tc, qc, dxc, yc, ic, ranges, s)
        : tc <= 8  ? launch_gemm_t<1, 2, true, kRbSmall, 2>(w, dm, tc, qc, dxc, yc, ic, ranges, s)
                   : launch_gemm_t<1, 2, true, kRbSmall, 4>(w, dm, tc, qc, dxc, yc, ic, ranges, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
