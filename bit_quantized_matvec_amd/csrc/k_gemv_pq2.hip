// k_gemv_pq2.hip -- decode matrix-vector product, repacked pq2_0 x q8_K.
//
// What is computed (page 1, "the trick with 4 and 16"; ciot README):
//   I[r][g] = sum_{k<128} w[r][128g+k] * q[128g+k]          exact integer
//   y[r]    = sum_g d_w[r][g] * d_x[g/2] * I[r][g]          fp64, rounded once
//
// How (gfx950): the product streams every weight byte from HBM exactly once,
// so the kernel is bandwidth bound and is shaped for coalesced loads and
// memory-level parallelism rather than for ALU reuse.
//   * one lane = one row; a workgroup = one 64-row tile and one slice of the
//     columns; its waves split the slice into runs of 256-column superchunks;
//   * per superchunk a lane issues four non-temporal dwordx4 loads (qd = 0..3),
//     each a fully coalesced 1 KiB wave request (the codes are never reused),
//     plus its row's scale pair from the 256 bytes that follow the codes in
//     the same 4352-byte unit, one or two superchunks ahead of their use
//     (the ring's depth: two, or one for short runs on a full grid);
//   * the activation bytes a lane needs are the same for every lane of the
//     wave: the workgroup stages its slice of them in LDS once, and each
//     superchunk's 256 bytes are read from there with broadcast 16-byte
//     reads, all issued before its products;
//   * each code dword yields four dot4 operands with one shift and one mask
//     each ((d << (6-2s)) & 0xC0C0C0C0 = 64*w for four columns: the pages'
//     slot masking, with two's-complement codes so that no +1 correction is
//     needed); the factor 64 is removed exactly by a shift;
//   * per group: term = (d_w * d_x) * I in fp64 (exact), accumulated in fp64;
//   * the wave partials of a workgroup are summed in LDS in wave order.  With
//     several column slices per tile (more, smaller workgroups, so the
//     hardware can balance them over the CUs), each workgroup stores its fp64
//     partial in a workspace and bumps the tile's counter; the last one to
//     arrive sums the slices in slice order, writes y and resets the counter.
//     The result is therefore deterministic, and no memset is needed between
//     calls (safe inside a captured graph).
#include <algorithm>

#include "kernels.h"
#include "q8k_block.h"

namespace tq {
namespace {

constexpr int kPlanWaves = 4;  // waves per workgroup (at most)
constexpr int kMaxWaves = kPlanWaves;
constexpr size_t kMaxStageBytes = 32 * 1024;  // LDS for one slice's staged activations

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Weight codes are read once and never reused: non-temporal loads keep them
// from displacing reusable lines and stream measurably faster on gfx950.
template <bool NT>
__device__ __forceinline__ v4u load_codes(const uint4* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return *reinterpret_cast<const v4u*>(p);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h));
}

__device__ __forceinline__ int slot64(uint32_t d, int s) {
  // field s of every byte, moved to bits 6..7: the byte reads as 64 * w
  return (int)((d << (6 - 2 * s)) & 0xC0C0C0C0u);
}

// Integer dots of one superchunk: i0 for group 2 sc (dwords c = 0, 1), i1 for
// group 2 sc + 1 (c = 2, 3).  `a` points at the superchunk's 64 activation
// dwords (wave-uniform); they are fetched first, in one batch of 16-byte
// reads, so that the wave waits for memory (LDS or cache) once per
// superchunk rather than once per few products.
__device__ __forceinline__ void superchunk_dots(const v4u (&v)[4], const int* __restrict__ a, int& i0, int& i1) {
  v4i act[16];  // act[4c + qd][s] = activation dword 16c + 4qd + s
#pragma unroll
  for (int k = 0; k < 16; ++k) act[k] = *reinterpret_cast<const v4i*>(a + 4 * k);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const uint32_t dw = v[qd][c];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (c < 2)
          i0 = __builtin_amdgcn_sdot4(slot64(dw, s), act[4 * c + qd][s], i0, false);
        else
          i1 = __builtin_amdgcn_sdot4(slot64(dw, s), act[4 * c + qd][s], i1, false);
      }
    }
  }
}

}  // namespace

// grid = (ntiles, slices).  Workgroup (tile, slice) covers superchunks
// [slice * scw, min(nsc, (slice + 1) * scw)); its waves take runs of spw.
// LDSQ: the slice's q is copied into LDS first, XB 16-byte pieces per thread
// (XB at least the pieces per thread).  FX: the activations come in as fp32 x
// (`xf`, `q` and `dx` unused) and each wave quantizes the blocks of its own
// run to q8_K itself, into LDS (requires LDSQ), in batches of XB blocks (up
// to 8).
// The body of one workgroup: `tile` is the row tile within the matrix,
// `ptile` the index of its arrival counter and partial sums in the workspace.
template <int RING, bool IDOTS, bool NT, bool LDSQ, bool FX, int XB>
__device__ __forceinline__ void gemv_pq2_body(const uint4* __restrict__ codes, const uint32_t* __restrict__ scales,
                                              const int* __restrict__ q, const float* __restrict__ dx,
                                              const float4* __restrict__ xf, float* __restrict__ y,
                                              int32_t* __restrict__ idots, int rows, int nsc, int G8, int scw, int spw,
                                              uint8_t* __restrict__ ws, int tile,
                                              int ptile) {
  __shared__ double red[kMaxWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int slice = blockIdx.y;
  const int nslices = gridDim.y;
  const int row = tile * 64 + lane;
  const int G = 2 * nsc;
  const int wg0 = slice * scw;
  const int wg1 = min(nsc, wg0 + scw);
  const int sc0 = min(wg1, wg0 + wave * spw);
  const int sc1 = min(wg1, sc0 + spw);

  // unit (tile, sc): 272 uint4 (256 of codes, then the 16 holding the 64
  // scale pairs); `scales` points at the first unit's scale pairs
  constexpr int kUnitU4 = (int)(kPq2UnitBytes / 16), kUnitDw = (int)(kPq2UnitBytes / 4);
  const uint4* cp = codes + (size_t)tile * nsc * kUnitU4 + lane;
  const uint32_t* sp = scales + (size_t)tile * nsc * kUnitDw + lane;
  double acc = 0.0;

  // The activations were typically written by the previous kernel, so every
  // line of them misses in this XCD's caches.  Read where they are used (one
  // scalar load per superchunk), those misses would serialize behind each
  // superchunk (measured: +6 us on 32768 x 8192 after the quantizer); instead
  // the workgroup first brings its slice's activations into LDS (a copy of q,
  // or with FX its own q8_K of x), and the products read them from there.
  static_assert(!FX || LDSQ, "the fused quantization writes its q8_K into the LDS stage");
  extern __shared__ int stage[];  // LDSQ: nb * 64 activation dwords; FX: then nb d_x
  const int nb = wg1 - wg0;       // superchunks of the slice (= q8_K blocks of 256 columns)
  const int* qa = q + (size_t)wg0 * 64;  // activations of the slice, indexed by sc - wg0
  const float* xa = dx + wg0;            // d_x of the slice, indexed by sc - wg0

  auto epilogue = [&](int sc, int i0, int i1, uint32_t s2) {
    const int I0 = i0 >> 6, I1 = i1 >> 6;  // exact: both are 64 * I
    if (IDOTS) {
      if (row < rows) {
        idots[(size_t)row * G + 2 * sc] = I0;
        idots[(size_t)row * G + 2 * sc + 1] = I1;
      }
    } else {
      // s2: fp16 scales of groups 2sc (low half) and 2sc+1.  The pair's
      // inner sum d0 I0 + d1 I1 (the first product exact) is rounded once,
      // then scaled by d_x into the accumulator: the prompt product's
      // epilogue, so that both give the same bits
      const double dxs = (double)xa[sc - wg0];
      const double inner = __builtin_fma((double)half_bits_to_float(s2 >> 16), (double)I1,
                                         (double)half_bits_to_float(s2 & 0xffffu) * (double)I0);
      acc = __builtin_fma(dxs, inner, acc);
    }
  };

  // The wave's superchunks [sc0, sc1) stream through a ring of RD slots: the
  // codes and the scale pair of superchunk j + RD are fetched while j is
  // multiplied.  The prologue fills the ring, so the state at the loop
  // header is the steady state and the compiler's wait counts stay exact.
  // Two slots (8 KiB in flight per wave), or one for short runs on a full
  // grid (fused_ring), measured fastest: deeper rings put
  // more requests in flight per CU than HBM serves better.
  constexpr int RD = RING;
  static_assert(RD == 1 || RD == 2, "the passes below are written out for one or two slots");
  const int n = sc1 - sc0;
  v4u rc[RD][4];
  uint32_t rsc[RD];
  // Fetches past the end of the run read 256 bytes of the (cache-resident)
  // activation vector instead of reloading codes from HBM; the loads stay
  // unconditional so that the wait counts stay exact.
  const void* hot = FX ? static_cast<const void*>(xf) : static_cast<const void*>(q);  // >= 256 cache-resident bytes
  const uint4* dummy_c = static_cast<const uint4*>(hot) + (lane & 15);
  const uint32_t* dummy_s = static_cast<const uint32_t*>(hot) + lane;
#define TQ_FETCH(J, K)                                                                                   \
  {                                                                                                      \
    const bool real = (K) < n;                                                                           \
    const int scf = sc0 + max(min((K), n - 1), 0);                                                       \
    const uint4* c0 = real ? cp + (size_t)scf * kUnitU4 : dummy_c;                                       \
    const uint32_t* s0 = real ? sp + (size_t)scf * kUnitDw : dummy_s;                                    \
    _Pragma("unroll") for (int qd = 0; qd < 4; ++qd) rc[J][qd] = load_codes<NT>(c0 + (real ? qd * 64 : 0)); \
    rsc[J] = *s0;                                                                                        \
  }
#define TQ_STEP(J)                                                                                       \
  {                                                                                                      \
    const int j = base + J;                                                                              \
    if (j < n) {                                                                                         \
      int i0 = 0, i1 = 0;                                                                                \
      superchunk_dots(rc[J], qa + (size_t)(sc0 + j - wg0) * 64, i0, i1);                                 \
      epilogue(sc0 + j, i0, i1, rsc[J]);                                                                 \
    }                                                                                                    \
    TQ_FETCH(J, j + RD)                                                                                  \
  }

  // Prologue: the activation loads go out first and the ring's first fetches
  // right behind them; staging then waits only for the activations (loads
  // complete in order), so it overlaps the HBM latency of the codes.
  if (FX) {
    // q8_K of the blocks (one per superchunk) of this wave's own run, in
    // batches of XB whose loads are all in flight together; the same
    // arithmetic as the standalone quantizer (q8k_block.h).  A wave reads only
    // its own blocks from the stage, so no barrier follows: each wave starts
    // its products as soon as its own part of x has arrived (measured on
    // 17408 x 5120: 8.73 -> 8.48 us; blocks interleaved over the waves needed
    // the whole workgroup's x first).  A batch slot past the run redoes the
    // run's last block, and a wave without a run the slice's last block: the
    // same bits to the same place, no branch, so the compiler keeps the loads
    // where they are.
    constexpr int kXB = XB;
    float* sd = reinterpret_cast<float*>(stage + nb * 64);
    float4 v[kXB];
    auto blk = [&](int i) { return n > 0 ? (sc0 - wg0) + min(i, n - 1) : nb - 1; };
    auto load_batch = [&](int b0) {
#pragma unroll
      for (int i = 0; i < kXB; ++i) v[i] = xf[(size_t)(wg0 + blk(b0 + i)) * 64 + lane];
    };
    auto quant_batch = [&](int b0) {
      float db[kXB];
      int pk[kXB];
      q8k_quant_batch<kXB>(v, db, pk);
#pragma unroll
      for (int i = 0; i < kXB; ++i) {
        const int b = blk(b0 + i);
        stage[b * 64 + lane] = pk[i];
        if (lane == 0) sd[b] = db[i];
      }
    };
    load_batch(0);
    TQ_FETCH(0, 0)
    if constexpr (RD > 1) TQ_FETCH(1, 1)
    __builtin_amdgcn_sched_barrier(0);  // all of those loads issue before the first quantization
    quant_batch(0);
    for (int b0 = kXB; b0 < n; b0 += kXB) {
      load_batch(b0);
      quant_batch(b0);
    }
    qa = stage;
    xa = sd;
  } else if (LDSQ) {
    // copy of the slice's q: XB 16-byte pieces per thread, all loaded before
    // the ring's first fetches; a piece index past the slice re-copies its
    // last piece (same bits to the same place, no branch)
    const int nd4 = nb * 16;
    const v4i* src = reinterpret_cast<const v4i*>(qa);
    v4i* dst = reinterpret_cast<v4i*>(stage);
    v4i v[XB];
#pragma unroll
    for (int i = 0; i < XB; ++i) v[i] = src[min((int)threadIdx.x + i * (int)blockDim.x, nd4 - 1)];
    TQ_FETCH(0, 0)
    if constexpr (RD > 1) TQ_FETCH(1, 1)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < XB; ++i) dst[min((int)threadIdx.x + i * (int)blockDim.x, nd4 - 1)] = v[i];
    __syncthreads();
    qa = stage;
  } else {
    TQ_FETCH(0, 0)
    if constexpr (RD > 1) TQ_FETCH(1, 1)
  }
  for (int base = 0; base < n; base += RD) {
    TQ_STEP(0)
    if constexpr (RD > 1) TQ_STEP(1)
  }
#undef TQ_STEP
#undef TQ_FETCH

  if (IDOTS) return;
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  double s = red[0][lane];
  for (int w = 1; w < nw; ++w) s += red[w][lane];
  if (nslices == 1) {
    if (row < rows) y[row] = (float)s;
    return;
  }
  // The partial goes out with an agent-scope atomic store (written through
  // to the level shared by all XCDs, so no whole-L2 write-back is needed);
  // the counter is bumped only after the store has completed (vmcnt = 0).
  double* partials = ws_partials(ws, ptile);
  unsigned* counter = ws_counter(ws, ptile);
  __hip_atomic_store(&partials[slice * 64 + lane], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, 64);
  if (prev != (unsigned)(nslices - 1)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // every slice's partial is requested before the first add (one loop with
  // a load and an add per slice waited a full round trip per slice); the
  // indices past the last slice repeat it and are not added
  double pv[kMaxSlices];
#pragma unroll
  for (int k = 0; k < kMaxSlices; ++k)
    pv[k] = __hip_atomic_load(&partials[min(k, nslices - 1) * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxSlices; ++k)
    if (k < nslices) t += pv[k];
  if (row < rows) y[row] = (float)t;
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Launch bounds: at most kMaxWaves waves, and two workgroups per compute unit
// (the decode grid of 512 row tiles on 256 compute units), so up to 256 VGPRs.
template <int RING, bool IDOTS, bool NT, bool LDSQ, bool FX, int XB = 1>
__global__ __launch_bounds__(64 * kMaxWaves, 2) void gemv_pq2_kernel(const uint4* __restrict__ codes,
                                                                  const uint32_t* __restrict__ scales,
                                                                  const int* __restrict__ q, const float* __restrict__ dx,
                                                                  const float4* __restrict__ xf,
                                                                  float* __restrict__ y, int32_t* __restrict__ idots,
                                                                  int rows, int nsc, int G8, int scw, int spw,
                                                                  uint8_t* __restrict__ ws) {
  gemv_pq2_body<RING, IDOTS, NT, LDSQ, FX, XB>(codes, scales, q, dx, xf, y, idots, rows, nsc, G8, scw, spw, ws,
                                               blockIdx.x, blockIdx.x);
}

// Several independent fused products with the same column count in one
// launch: workgroup x belongs to problem m with tile0[m] <= x < tile0[m + 1].
template <int RING, int XB>
__global__ __launch_bounds__(64 * kMaxWaves, 2) void gemv_pq2_batch_kernel(GemvBatch b, int nsc, int G8, int scw, int spw,
                                                                        uint8_t* __restrict__ ws) {
  const int x = blockIdx.x;
  int m = 0;
#pragma unroll
  for (int k = 1; k < kMaxBatch; ++k) m += (k < b.n && x >= b.tile0[k]) ? 1 : 0;
  gemv_pq2_body<RING, false, true, true, true, XB>(b.codes[m], b.scales[m], nullptr, nullptr, b.x[m], b.y[m], nullptr,
                                                b.rows[m], nsc, G8, scw, spw, ws, x - b.tile0[m], x);
}

GemvPlan plan_gemv_pq2(const Dims& dm, bool have_workspace) {
  // Measured on MI355X: with 384 or more row tiles one workgroup per tile is
  // fastest (32768 x 8192: 13.7 us; split in 2 or 4 slices: 15.4, 17.1).
  // With fewer tiles the columns are split.  Of the slice counts that give
  // each wave a run of 2 or 3 superchunks (at least 4 superchunks per
  // slice), the one with the least work on the busiest compute unit --
  // ceil(workgroups / 256) x superchunks per slice -- is taken, ties going to
  // more slices; without such a count, runs of any length from 2.  Fused
  // kernel, us per slice count 2 / 3 / 4 / 5 / 6 / 9 / 12 (rule's pick *):
  // 17408 x 5120 9.60 / 8.99 / 8.93* / 9.75 / 9.75 / 9.61 / 9.54; 7168 x
  // 5120 6.58 / 6.56 / 5.93* / 6.43 / 6.43 / 6.34 / 6.17; 5120 x 6144 6.45 /
  // 5.24* / 6.15 / 5.91 / 5.37 / 6.02 / 5.49; 5120 x 17408 12.70 / 9.21 /
  // 11.11 / 9.01 / 8.17 / 8.10 / 8.09*.  A tiny row is not split (256 x
  // 1024 takes 2.9 us unsplit, 4.2 split).
  GemvPlan p;
  const int nsc = (int)dm.nsc;
  int slices = 1;
  if (have_workspace && dm.ntiles < 384) {
    const int most_slices = std::min(kMaxSlices, std::max(1, nsc / 4));
    for (int pass = 0; pass < 2 && slices == 1; ++pass) {
      const int longest = pass == 0 ? 3 : nsc;  // runs of 2 or 3 superchunks, else of any length from 2
      int64_t best_cost = -1;
      for (int sl = 2; sl <= most_slices; ++sl) {
        const int scw = (nsc + sl - 1) / sl;
        const int w = std::min(scw, kPlanWaves);
        const int run = (scw + w - 1) / w;
        if (run < 2 || run > longest) continue;
        const int64_t cost = (dm.ntiles * sl + 255) / 256 * scw;
        if (best_cost < 0 || cost <= best_cost) {
          best_cost = cost;
          slices = sl;
        }
      }
    }
  }
  p.scw = (nsc + slices - 1) / slices;
  p.slices = (nsc + p.scw - 1) / p.scw;
  const int waves = p.scw < kPlanWaves ? p.scw : kPlanWaves;
  p.spw = (p.scw + waves - 1) / waves;
  p.waves = (p.scw + p.spw - 1) / p.spw;
  return p;
}

hipError_t launch_gemv_pq2_plan(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, float* y,
                                int32_t* idots, void* workspace, const GemvPlan& p, hipStream_t s) {
  constexpr int kRing = 2;
  const int nsc = (int)dm.nsc;
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint32_t* scales = reinterpret_cast<const uint32_t*>(w + kPq2ScaleOffset);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const dim3 grid((unsigned)dm.ntiles, (unsigned)p.slices), block(64 * p.waves);
  // one slice's activations are staged in LDS when they fit (always with the
  // column splits a workspace allows for matrices of up to 128 Ki columns)
  const size_t stage = (size_t)p.scw * 256;
  const bool ldsq = stage <= kMaxStageBytes;
  const int* qi = reinterpret_cast<const int*>(q);
  const int ns = (int)dm.G8;
  // 16-byte pieces of q per thread in the LDS copy
  const int pieces = (p.scw * 16 + 64 * p.waves - 1) / (64 * p.waves);
#define TQ_LAUNCH(ID, LQ, XB)                                                                                     \
  hipLaunchKernelGGL((gemv_pq2_kernel<kRing, ID, true, LQ, false, XB>), grid, block, LQ ? (unsigned)stage : 0u, s, \
                     codes, scales, qi, dx, nullptr, y, idots, (int)dm.rows, nsc, ns, p.scw, p.spw, ws)
#define TQ_LAUNCH_Q(ID)                          \
  if (!ldsq) TQ_LAUNCH(ID, false, 1);            \
  else if (pieces <= 1) TQ_LAUNCH(ID, true, 1);  \
  else if (pieces <= 2) TQ_LAUNCH(ID, true, 2);  \
  else if (pieces <= 4) TQ_LAUNCH(ID, true, 4);  \
  else TQ_LAUNCH(ID, true, 8);
  if (idots) {
    TQ_LAUNCH_Q(true)
  } else {
    TQ_LAUNCH_Q(false)
  }
#undef TQ_LAUNCH_Q
#undef TQ_LAUNCH
  return hipGetLastError();
}

bool gemv_pq2_fused_fits(const Dims& dm, bool have_workspace) {
  const GemvPlan p = plan_gemv_pq2(dm, have_workspace);
  return (size_t)p.scw * (256 + 4) <= kMaxStageBytes;
}

// Ring slots of the fused kernels (measured on MI355X, fused product, 2 / 1
// slots): 17408 x 5120 (544 workgroups, runs of 3) 10.10 / 9.60 us and
// 5120 x 17408 (480, runs of 3) 10.31 / 9.51 us take one slot; 32768 x 8192
// (512, runs of 8) 13.6 / 15.3 us, 7168 x 5120 (224) 6.49 / 6.72 us and
// 5120 x 6144 (240, runs of 2) 5.56 / 5.80 us keep two.  With short runs and
// at least two workgroups per compute unit, a second slot in flight only
// adds to the burst of requests at the start.
int fused_ring(const Dims& dm, const GemvPlan& p) { return dm.ntiles * p.slices >= 448 && p.spw <= 3 ? 1 : 2; }

hipError_t launch_gemv_pq2_fused(const uint8_t* w, const Dims& dm, const float* x, float* y, void* workspace,
                                 hipStream_t s) {
  const GemvPlan p = plan_gemv_pq2(dm, workspace != nullptr);
  const size_t stage = (size_t)p.scw * (256 + 4);
  if (stage > kMaxStageBytes) return hipErrorInvalidValue;  // the caller checks gemv_pq2_fused_fits first
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint32_t* scales = reinterpret_cast<const uint32_t*>(w + kPq2ScaleOffset);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const dim3 grid((unsigned)dm.ntiles, (unsigned)p.slices), block(64 * p.waves);
  // quantization batch: a wave's run of blocks, no more than 8 at once (a
  // batch no longer than the run: the gate + up launch of 17408 x 5120 runs
  // of 5 took 13.33 us with batches of 8, 12.67 with batches of 6)
  const int ring = fused_ring(dm, p);
#define TQ_LAUNCH(RG, XB)                                                                                       \
  hipLaunchKernelGGL((gemv_pq2_kernel<RG, false, true, true, true, XB>), grid, block, (unsigned)stage, s, codes, \
                     scales, nullptr, nullptr, reinterpret_cast<const float4*>(x), y, nullptr, (int)dm.rows,     \
                     (int)dm.nsc, (int)dm.G8, p.scw, p.spw, ws)
  if (p.spw <= 2) { if (ring == 1) TQ_LAUNCH(1, 2); else TQ_LAUNCH(2, 2); }
  else if (p.spw <= 4) { if (ring == 1) TQ_LAUNCH(1, 4); else TQ_LAUNCH(2, 4); }
  else if (p.spw <= 6) { if (ring == 1) TQ_LAUNCH(1, 6); else TQ_LAUNCH(2, 6); }
  else { if (ring == 1) TQ_LAUNCH(1, 8); else TQ_LAUNCH(2, 8); }
#undef TQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemv_pq2_fused_batch(const GemvBatch& b, const Dims& dm, void* workspace, hipStream_t s) {
  const GemvPlan p = plan_gemv_pq2(dm, workspace != nullptr);
  const size_t stage = (size_t)p.scw * (256 + 4);
  if (stage > kMaxStageBytes) return hipErrorInvalidValue;  // the caller checks gemv_pq2_fused_fits first
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const dim3 grid((unsigned)dm.ntiles, (unsigned)p.slices), block(64 * p.waves);
  const int ring = fused_ring(dm, p);
  // quantization batch as in launch_gemv_pq2_fused
#define TQ_LAUNCH(RG, XB)                                                                                         \
  hipLaunchKernelGGL((gemv_pq2_batch_kernel<RG, XB>), grid, block, (unsigned)stage, s, b, (int)dm.nsc, (int)dm.G8, \
                     p.scw, p.spw, ws)
  if (p.spw <= 2) { if (ring == 1) TQ_LAUNCH(1, 2); else TQ_LAUNCH(2, 2); }
  else if (p.spw <= 4) { if (ring == 1) TQ_LAUNCH(1, 4); else TQ_LAUNCH(2, 4); }
  else if (p.spw <= 6) { if (ring == 1) TQ_LAUNCH(1, 6); else TQ_LAUNCH(2, 6); }
  else { if (ring == 1) TQ_LAUNCH(1, 8); else TQ_LAUNCH(2, 8); }
#undef TQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemv_pq2(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, float* y,
                           int32_t* idots, void* workspace, hipStream_t s) {
  const GemvPlan p = plan_gemv_pq2(dm, workspace != nullptr && idots == nullptr);
  return launch_gemv_pq2_plan(w, dm, q, dx, y, idots, workspace, p, s);
}

}  // namespace tq
