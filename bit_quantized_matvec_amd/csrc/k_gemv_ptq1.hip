// k_gemv_ptq1.hip -- decode matrix-vector product, repacked ptq1_0 x q8_K.
//
// Base-3 weights (page 1, "the detour that lost"; ciot README ptq1_0
// paragraph): trit j of byte b is floor(3 * ((b * 3^j) mod 256) / 256), and
// w = trit - 1.  The trits follow from one another: with v0 = b,
// t_j = (3 v_j) >> 8 and v_{j+1} = (3 v_j) & 255.
//
// How (gfx950):
//   * one lane = one row, a workgroup = a 64-row tile, waves split the
//     8-group superblocks; 13 fully coalesced dwordx4 loads per row and
//     superblock (1.75 bits per weight, bytes only reordered by the repack);
//   * the four bytes of a code dword are split into two pairs of 16-bit lanes
//     (bytes 0, 2 and bytes 1, 3), so one 32-bit multiply-by-3 advances two
//     bytes at once without carries between them; after it the high byte of
//     each lane is that byte's trit, and one v_perm_b32 gathers the four into
//     a dword = one dot4 operand;
//   * the trits are w + 1, so I = dot(t, q) - sum(q), the group sum coming
//     from the q8_K partial sums (page 1, "the trick with 4 and 16": sum(y)
//     over 128 values is one add over 8 partial sums);
//   * the dot4 partner of trit j of four consecutive code bytes is the four
//     activations 5 apart; each workgroup first writes this permuted copy of
//     q into LDS, and the main loop reads it with wave-uniform (broadcast)
//     LDS loads.  The two bytes per group that do not fill a dword are paired
//     with the next group's, and their padding trits meet zero activations.
#include "kernels.h"

namespace tq {
namespace {

constexpr int kMaxWaves = 8;   // the kernel's limit
constexpr int kPlanWaves = 4;  // what the plan uses
constexpr int kTableDwords = 48 * 8 + 4 * 16;  // per superblock
constexpr int kQChunk = 4;                      // superblocks of q copied into LDS at a time

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h));
}

// Permuted activation table.  Entry (D < 48, j): bytes i = 0..3 hold
// q[col(group gi, byte 4m + i, trit j)] with D = 6 gi + m.  Entry (48 + p, j, h):
// the leftover dword p pairs bytes 24, 25 of groups 2p (h = 0) and 2p + 1
// (h = 1); only the half of the dword that belongs to group 2p + h is non-zero.
// `qs` is the workgroup's copy of q in LDS, starting at group g0.
__device__ uint32_t table_entry(const uint8_t* __restrict__ qs, int g0, int G, int sb, int e) {
  auto act = [&](int g, int byte, int j) -> uint32_t {
    const int k = 5 * byte + j;  // position inside the group
    if (g >= G || k >= 128) return 0u;
    return (uint32_t)qs[(g - g0) * 128 + k];
  };
  if (e < 48 * 8) {
    const int D = e >> 3, j = e & 7;
    if (j >= 5) return 0u;
    const int g = sb * 8 + D / 6, m = D % 6;
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) r |= act(g, 4 * m + i, j) << (8 * i);
    return r;
  }
  const int f = e - 48 * 8;
  const int p = f >> 4, jj = f & 15;
  if (jj >= 10) return 0u;
  const int j = jj >> 1, h = jj & 1;
  const int g = sb * 8 + 2 * p + h;
  const uint32_t lo = act(g, 24, j) | (act(g, 25, j) << 8);
  return h ? lo << 16 : lo;
}

}  // namespace

// grid = (ntiles, slices).  Workgroup (tile, slice) covers superblocks
// [slice * scw, min(G8, (slice + 1) * scw)); its waves take runs of spw.
template <bool IDOTS>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_ptq1_kernel(const uint4* __restrict__ codes,
                                                                   const uint4* __restrict__ scales,
                                                                   const int8_t* __restrict__ q, const float* __restrict__ dx,
                                                                   const int16_t* __restrict__ bsums, float* __restrict__ y,
                                                                   int32_t* __restrict__ idots, int rows, int G, int G8,
                                                                   int scw, int spw, double* __restrict__ partials,
                                                                   unsigned* __restrict__ counters) {
  extern __shared__ uint32_t table[];
  __shared__ double red[kMaxWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int tile = blockIdx.x;
  const int slice = blockIdx.y;
  const int nslices = gridDim.y;
  const int row = tile * 64 + lane;
  const int wg0 = slice * scw;
  const int wg1 = min(G8, wg0 + scw);

  // Permuted activations of this workgroup's superblocks, built kQChunk
  // superblocks at a time: that part of q is first copied into LDS with
  // coalesced 16-byte loads (the table gathers single bytes, which straight
  // from global memory would cost one round trip each), then its table
  // entries are built from the copy.
  uint8_t* qs = reinterpret_cast<uint8_t*>(table + (wg1 - wg0) * kTableDwords);
  for (int c0 = wg0; c0 < wg1; c0 += kQChunk) {
    const int c1 = min(wg1, c0 + kQChunk);
    const int g0 = c0 * 8, g1 = min(G, c1 * 8);
    const uint4* src = reinterpret_cast<const uint4*>(q + (size_t)g0 * 128);
    uint4* dst = reinterpret_cast<uint4*>(qs);
    for (int i = threadIdx.x; i < (g1 - g0) * 8; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
    for (int e = threadIdx.x; e < (c1 - c0) * kTableDwords; e += blockDim.x) {
      const int sb = c0 + e / kTableDwords;
      table[(sb - wg0) * kTableDwords + e % kTableDwords] = table_entry(qs, g0, G, sb, e % kTableDwords);
    }
    __syncthreads();
  }

  const int sb0 = min(wg1, wg0 + wave * spw);
  const int sb1 = min(wg1, sb0 + spw);
  double acc = 0.0;
  for (int sb = sb0; sb < sb1; ++sb) {
    // Loads 0..11 hold the 48 full dwords (3 loads per group pair), load 12
    // the four leftover dwords.  One group pair is decoded per iteration,
    // with the next pair's three loads already in flight.
    const uint4* cp = codes + ((size_t)(tile * G8 + sb) * 13) * 64 + lane;
    const uint4 left = cp[12 * 64];
    const uint4 sc8 = scales[(size_t)(tile * G8 + sb) * 64 + lane];
    const uint32_t* tb = table + (sb - wg0) * kTableDwords;
    uint4 cur[3] = {cp[0], cp[64], cp[128]};
#pragma unroll 1
    for (int gp = 0; gp < 4; ++gp) {
      uint4 nxt[3] = {cur[0], cur[1], cur[2]};
      if (gp < 3) {
        nxt[0] = cp[(3 * gp + 3) * 64];
        nxt[1] = cp[(3 * gp + 4) * 64];
        nxt[2] = cp[(3 * gp + 5) * 64];
      }
      const uint32_t dws[13] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y, cur[1].z,
                                cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                                gp == 0 ? left.x : gp == 1 ? left.y : gp == 2 ? left.z : left.w};
      int ia = 0, ib = 0;  // groups 2 gp and 2 gp + 1
#pragma unroll
      for (int m = 0; m < 13; ++m) {
        const uint32_t d = dws[m];
        uint32_t tv[10];
        if (m < 12) {
          const uint32_t* te = tb + (12 * gp + m) * 8;
          const uint4 t0 = *reinterpret_cast<const uint4*>(te);
          tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w; tv[4] = te[4];
        } else {
          const uint4* lt = reinterpret_cast<const uint4*>(tb + 48 * 8 + gp * 16);
          const uint4 t0 = lt[0], t1 = lt[1];
          const uint2 t2 = *reinterpret_cast<const uint2*>(lt + 2);
          tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w;
          tv[4] = t1.x; tv[5] = t1.y; tv[6] = t1.z; tv[7] = t1.w; tv[8] = t2.x; tv[9] = t2.y;
        }
        uint32_t e = d & 0x00FF00FFu;
        uint32_t o = (d >> 8) & 0x00FF00FFu;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          e *= 3u;
          o *= 3u;
          // each 16-bit lane now holds 3v < 768, so its high byte is the trit:
          // one byte permute gathers the four (bytes 1, 3 of e and of o)
          const int t = (int)__builtin_amdgcn_perm(o, e, 0x07030501u);
          if (m < 6) {
            ia = __builtin_amdgcn_sdot4(t, (int)tv[j], ia, false);
          } else if (m < 12) {
            ib = __builtin_amdgcn_sdot4(t, (int)tv[j], ib, false);
          } else {
            ia = __builtin_amdgcn_sdot4(t, (int)tv[2 * j], ia, false);
            ib = __builtin_amdgcn_sdot4(t, (int)tv[2 * j + 1], ib, false);
          }
          e &= 0x00FF00FFu;
          o &= 0x00FF00FFu;
        }
      }
      const uint32_t s2 = gp == 0 ? sc8.x : gp == 1 ? sc8.y : gp == 2 ? sc8.z : sc8.w;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = sb * 8 + 2 * gp + h;
        if (g < G) {
          const int16_t* bs = bsums + (size_t)g * 8;
          const int qsum = bs[0] + bs[1] + bs[2] + bs[3] + bs[4] + bs[5] + bs[6] + bs[7];
          const int I = (h ? ib : ia) - qsum;
          if (IDOTS) {
            if (row < rows) idots[(size_t)row * G + g] = I;
          } else {
            acc += ((double)half_bits_to_float(h ? (s2 >> 16) : (s2 & 0xffffu)) * (double)dx[g >> 1]) * (double)I;
          }
        }
      }
      cur[0] = nxt[0];
      cur[1] = nxt[1];
      cur[2] = nxt[2];
    }
  }
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
  // several slices per tile: the last workgroup to arrive sums them in order
  // The partial goes out with an agent-scope atomic store (written through
  // to the level shared by all XCDs, so no whole-L2 write-back is needed);
  // the counter is bumped only after the store has completed (vmcnt = 0).
  __hip_atomic_store(&partials[((size_t)tile * nslices + slice) * 64 + lane], s, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, 64);
  if (prev != (unsigned)(nslices - 1)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  double t = 0.0;
  for (int k = 0; k < nslices; ++k)
    t += __hip_atomic_load(&partials[((size_t)tile * nslices + k) * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (row < rows) y[row] = (float)t;
  if (lane == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

GemvPlan plan_gemv_ptq1(const Dims& dm, bool have_workspace) {
  // As for pq2_0: one workgroup per tile when there are many tiles, else split
  // the 8-group superblocks until there are ~384 workgroups.
  GemvPlan p;
  const int G8 = (int)dm.G8;
  int slices = 1;
  if (have_workspace && dm.ntiles < 384) {
    slices = (int)((384 + dm.ntiles - 1) / dm.ntiles);
    slices = slices < kMaxSlices ? slices : kMaxSlices;
    slices = slices < G8 ? slices : G8;
  }
  p.scw = (G8 + slices - 1) / slices;
  p.slices = (G8 + p.scw - 1) / p.scw;
  // up to 4 waves (measured on 32768 x 8192: 4 waves of two superblocks each
  // beat 8 waves of one, which cannot share a CU two workgroups at a time)
  const int waves = p.scw < kPlanWaves ? p.scw : kPlanWaves;
  p.spw = (p.scw + waves - 1) / waves;
  p.waves = (p.scw + p.spw - 1) / p.spw;
  return p;
}

hipError_t launch_gemv_ptq1_plan(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx,
                                 const int16_t* bsums, float* y, int32_t* idots, void* workspace, const GemvPlan& p,
                                 hipStream_t s) {
  // the table, then room for kQChunk superblocks of q to build it from
  const size_t lds = (size_t)p.scw * kTableDwords * sizeof(uint32_t) + (size_t)kQChunk * 1024;
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint4* scales = reinterpret_cast<const uint4*>(w + ptq1_code_bytes(dm));
  unsigned* counters = reinterpret_cast<unsigned*>(workspace);
  double* partials =
      workspace ? reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + workspace_counter_bytes(dm)) : nullptr;
  const dim3 grid((unsigned)dm.ntiles, (unsigned)p.slices), block(64 * p.waves);
  if (idots)
    hipLaunchKernelGGL(gemv_ptq1_kernel<true>, grid, block, lds, s, codes, scales, q, dx, bsums, y, idots, (int)dm.rows,
                       (int)dm.G, (int)dm.G8, p.scw, p.spw, partials, counters);
  else
    hipLaunchKernelGGL(gemv_ptq1_kernel<false>, grid, block, lds, s, codes, scales, q, dx, bsums, y, idots, (int)dm.rows,
                       (int)dm.G, (int)dm.G8, p.scw, p.spw, partials, counters);
  return hipGetLastError();
}

hipError_t launch_gemv_ptq1(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, const int16_t* bsums,
                            float* y, int32_t* idots, void* workspace, hipStream_t s) {
  const GemvPlan p = plan_gemv_ptq1(dm, workspace != nullptr && idots == nullptr);
  return launch_gemv_ptq1_plan(w, dm, q, dx, bsums, y, idots, workspace, p, s);
}

}  // namespace tq
