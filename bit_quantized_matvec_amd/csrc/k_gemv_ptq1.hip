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
//     superblock (1.75 bits per weight, bytes only reordered by the repack),
//     requested in two halves;
//   * the four bytes of a code dword are spread over the four 16-bit lanes of
//     a 64-bit register, so one 64-bit shift-and-add (x + 2x) advances all
//     four at once without carries between them, and one v_perm_b32 gathers
//     the four high bytes into a dword = one dot4 operand.  Without masking
//     between the multiplications the high byte after j + 1 of them is
//     h_j = floor(b 3^(j+1) / 256), and trit j is h_j - 3 h_(j-1):
//     summation by parts turns the trit dot into h dots against the
//     activations and their next-trit neighbours (no masks); the leftover
//     dword, whose halves belong to two groups, is masked trit by trit;
//   * the trits are w + 1, so I = dot(t, q) - sum(q), the group sum coming
//     from the q8_K partial sums (page 1, "the trick with 4 and 16": sum(y)
//     over 128 values is one add over 8 partial sums);
//   * the dot4 partner of trit j of four consecutive code bytes is the four
//     activations 5 apart; each workgroup first writes this permuted copy of
//     q into LDS (20 consecutive bytes of q give the 5 entries of one code
//     dword: a 4 x 5 byte transpose), and the main loop reads it with
//     wave-uniform (broadcast) LDS loads.  The two bytes per group that do
//     not fill a dword are paired with the next group's, and their padding
//     trits meet zero activations.  The table also holds each group's sum of
//     q and its d_x, so the products read nothing but LDS (scalar loads in
//     the loop would make every LDS wait a full one: they return out of
//     order);
//   * the fp64 sum has one fixed order whatever the launch: per group pair
//     (groups 2p, 2p + 1 share one q8_K block) inner = d_w(2p+1) I1 +
//     d_w(2p) I0 and acc = d_x inner + acc, each with one rounding, acc from
//     zero per superblock in pair order, and the superblock sums in
//     superblock order.  Waves, column slices (with a workspace) and token
//     blocks only change who computes which superblock sum, so every launch
//     shape -- and the MFMA prompt product, which uses the same sequence --
//     gives the same bits;
//   * one token: up to 8 waves per workgroup, one superblock each where the
//     columns allow;
//   * a prompt of up to 7 tokens runs NT tokens per workgroup (NT = 1 or
//     2): each code dword is decoded once and its trits meet the NT tokens'
//     tables, whose entries are interleaved by token.  Longer prompts go to
//     the MFMA kernel of k_gemm_ptq1.hip.
#include "kernels.h"

namespace tq {
namespace {

constexpr int kMaxWaves = 8;   // the kernel's limit
constexpr int kTableDwords = 48 * 8 + 4 * 16;  // per superblock and token
constexpr int kTasks = 48 + 8;                  // table-building tasks per superblock and token
constexpr int kMaxTokBlock = 2;                 // tokens per workgroup
constexpr int kMfmaMinTokens = 8;               // from here on prompts go to the MFMA kernel
constexpr size_t kLdsBudget = 80 * 1024;        // two workgroups per compute unit

// Dynamic LDS of a workgroup: the tables of scw superblocks for nt tokens.
// Once a superblock's products are done, the start of its table holds its
// fp64 sums [token][lane] (512 bytes per token, within the 1792 of the table).
size_t ptq1_lds_bytes(int scw, int nt) { return (size_t)nt * scw * kTableDwords * sizeof(uint32_t); }

// LDS-typed pointers, so that an address passed through an asm statement
// still yields LDS reads.
typedef __attribute__((address_space(3))) const uint32_t* lds_cptr;
typedef unsigned lds_v4 __attribute__((ext_vector_type(4)));
typedef unsigned lds_v2 __attribute__((ext_vector_type(2)));

// `L` consecutive dwords of LDS from a 16-byte aligned address, in as few
// reads as the alignment allows.
template <int L>
__device__ __forceinline__ void lds_run(lds_cptr p, uint32_t* v) {
  typedef __attribute__((address_space(3))) const lds_v4* P4;
  typedef __attribute__((address_space(3))) const lds_v2* P2;
  const P4 p4 = (P4)p;
#pragma unroll
  for (int i = 0; i < L / 4; ++i) {
    const lds_v4 t = p4[i];
    v[4 * i] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
  if constexpr (L % 4 >= 2) {
    const lds_v2 t = *(P2)(p + L / 4 * 4);
    v[L / 4 * 4] = t.x;
    v[L / 4 * 4 + 1] = t.y;
  }
  if constexpr (L % 2 == 1) v[L - 1] = p[L - 1];
}

__device__ __forceinline__ uint64_t times3(uint64_t x) {
  uint64_t r;
  asm("v_lshl_add_u64 %0, %1, 1, %1" : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h));
}

// Permuted activation table of one superblock and token.  Entry (D, j),
// D = 6 gi + m < 48, j < 5, at dword 8 D + j: bytes i = 0..3 hold
// q[group 8 sb + gi][5 (4m + i) + j], the partners of trit j of code bytes
// 4m .. 4m + 3 of that group.  Entry (p, h, j) at dword 384 + 16 p + 2 j + h:
// the leftover code dword p pairs bytes 24, 25 of groups 2p (low half) and
// 2p + 1 (high half); entry h holds group 2p + h's partners of trit j of
// those two bytes in its half and zeros in the other.  Groups past G and
// positions past 128 (the padding trits of byte 25) are zero.
//
// Task t < 48 (D = t) reads the 20 bytes q[g][20m .. 20m + 19] and writes
// the five entries (D, 0..4), a 4 x 5 byte transpose; task 48 + 2p + h reads
// q[g][120 .. 127] and writes the five entries (p, h, 0..4).  The spare
// dwords 8D + 6 and 8D + 7 of D = 6 gi (m = 0) hold group gi's sum of q (the
// sum of its 8 partial sums) and its d_x (as bits), so that the products
// read nothing but LDS.  `qt`, `bst`, `dxt` are the token's rows of q, the
// partial sums and d_x (dxt may be null: group dots only); `out` the
// superblock's table, `nt` tokens interleaved.
__device__ __forceinline__ void build_task(const int8_t* __restrict__ qt, const int16_t* __restrict__ bst,
                                           const float* __restrict__ dxt, int G, int sb, int task, uint32_t* out,
                                           int nt) {
  auto byte = [](uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; };
  if (task < 48) {
    const int g = sb * 8 + task / 6, m = task % 6;
    uint32_t w[5] = {0u, 0u, 0u, 0u, 0u};
    if (g < G) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(qt + (size_t)g * 128 + 20 * m);
#pragma unroll
      for (int k = 0; k < 5; ++k) w[k] = src[k];
    }
    if (m == 0) {
      int qsum = 0;
      float d = 0.0f;
      if (g < G) {
#pragma unroll
        for (int k = 0; k < 8; ++k) qsum += bst[(size_t)g * 8 + k];
        if (dxt) d = dxt[g >> 1];
      }
      out[(task * 8 + 6) * nt] = (uint32_t)qsum;
      out[(task * 8 + 7) * nt] = __builtin_bit_cast(uint32_t, d);
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      uint32_t r = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 5 * i + j;  // byte of the 20
        r |= byte(w[b >> 2], b & 3) << (8 * i);
      }
      out[(task * 8 + j) * nt] = r;
    }
  } else {
    const int p = (task - 48) >> 1, h = (task - 48) & 1;
    const int g = sb * 8 + 2 * p + h;
    uint32_t u0 = 0u, u1 = 0u;  // q[g][120 .. 123], q[g][124 .. 127]
    if (g < G) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(qt + (size_t)g * 128 + 120);
      u0 = src[0];
      u1 = src[1];
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint32_t a = j < 4 ? byte(u0, j) : byte(u1, 0);  // q[120 + j]
      const uint32_t b = j < 3 ? byte(u1, j + 1) : 0u;       // q[125 + j]; 128, 129 are padding
      const uint32_t lo = a | (b << 8);
      out[(384 + 16 * p + 2 * j + h) * nt] = h ? lo << 16 : lo;
    }
  }
}

}  // namespace

// grid = (ntiles, slices, token blocks).  Workgroup (tile, slice, tb) covers
// superblocks [slice * scw, min(G8, (slice + 1) * scw)) for tokens
// [tb * NT, tb * NT + NT) (those past `tokens` are padding: zero tables,
// outputs not written); its waves take runs of spw superblocks.  Several
// slices are used with NT == 1 only.
template <bool IDOTS, int NT>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_ptq1_kernel(const uint4* __restrict__ codes,
                                                                   const uint4* __restrict__ scales,
                                                                   const int8_t* __restrict__ q, const float* __restrict__ dx,
                                                                   const int16_t* __restrict__ bsums, float* __restrict__ y,
                                                                   int32_t* __restrict__ idots, int rows, int G, int G8,
                                                                   int scw, int spw, uint8_t* __restrict__ ws,
                                                                   int tokens) {
  extern __shared__ __align__(16) uint32_t table[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int tile = blockIdx.x;
  const int slice = blockIdx.y;
  const int nslices = gridDim.y;
  const int tok0 = blockIdx.z * NT;
  const int row = tile * 64 + lane;
  const int wg0 = slice * scw;
  const int wg1 = min(G8, wg0 + scw);
  const size_t K = (size_t)G * 128;

  // Permuted activations of this workgroup's superblocks: entry e of
  // superblock sb for token n sits at ((sb - wg0) * kTableDwords + e) * NT + n.
  for (int i = threadIdx.x; i < (wg1 - wg0) * kTasks * NT; i += blockDim.x) {
    const int n = i % NT, r = i / NT;
    const int sb = wg0 + r / kTasks, task = r % kTasks;
    uint32_t* out = table + (size_t)(sb - wg0) * kTableDwords * NT + n;
    if (tok0 + n < tokens) {
      const size_t t = (size_t)(tok0 + n);
      build_task(q + t * K, bsums + t * K / 16, dx ? dx + t * K / 256 : nullptr, G, sb, task, out, NT);
    } else {
      build_task(q, bsums, nullptr, 0, sb, task, out, NT);  // padding token: G = 0 gives zero entries
    }
  }
  __syncthreads();

  const int sb0 = min(wg1, wg0 + wave * spw);
  const int sb1 = min(wg1, sb0 + spw);
  for (int sb = sb0; sb < sb1; ++sb) {
    double acc[NT];  // this superblock's sums, from zero
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = 0.0;
    // Loads 0..11 hold the 48 full dwords (3 loads per group pair), load 12
    // the four leftover dwords.  Group pairs 0 and 1 (with the leftover
    // dwords and the scales) are requested first, pairs 2 and 3 once pair 0
    // is done: with every wave of the chip starting its superblock at once,
    // half the requests in flight stream faster than the whole superblock's
    // (measured on 32768 x 8192: 16.3 us -> 15.7-16.0 us).
    constexpr int kUnitU4 = (int)(kPtq1UnitBytes / 16);  // 13 code loads x 64 rows, then 64 scale rows
    const uint4* cp = codes + (size_t)(tile * G8 + sb) * kUnitU4 + lane;
    uint4 cw[13];
#pragma unroll
    for (int k = 0; k < 3; ++k) cw[k] = cp[k * 64];
    cw[12] = cp[12 * 64];
    const uint4 sc8 = scales[(size_t)(tile * G8 + sb) * kUnitU4 + lane];
#pragma unroll
    for (int k = 3; k < 6; ++k) cw[k] = cp[k * 64];
    const uint4 left = cw[12];
    const uint32_t* tb = table + (size_t)(sb - wg0) * kTableDwords * NT;
#pragma unroll
    for (int gp = 0; gp < 4; ++gp) {
      if (gp == 1) {
#pragma unroll
        for (int k = 6; k < 12; ++k) cw[k] = cp[k * 64];
      }
      const uint4* cur = cw + 3 * gp;
      const uint32_t dws[13] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y, cur[1].z,
                                cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                                gp == 0 ? left.x : gp == 1 ? left.y : gp == 2 ? left.z : left.w};
      // groups 2 gp (a) and 2 gp + 1 (b), per token: i = sum h x + t4 x4 and
      // j = sum h x_next, the group's dot(t, q) being i - 3 j
      int ia[NT], ib[NT], ja[NT], jb[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) ia[n] = ib[n] = ja[n] = jb[n] = 0;
      // Table entries of dword m: 5 levels (10 level-halves for the leftover
      // dword m = 12) x NT tokens, entry (level, token) at te[level * NT + token].
      // The reads of dword m + 1 are issued before the products of dword m
      // and no earlier, so that two dwords' entries at most are held in
      // registers: the table's base address passes through an empty asm
      // statement once per dword, which keeps the compiler from merging or
      // hoisting reads across dwords (the constant offsets still fold into
      // the read instructions).
      constexpr int kLev = 5 * NT, kLeft = 10 * NT;
      auto te_off = [&](int m) { return m < 12 ? (12 * gp + m) * 8 * NT : (48 * 8 + gp * 16) * NT; };
      uint32_t tnext[kLeft];
      lds_cptr tbl = (lds_cptr)tb;
      asm volatile("" : "+v"(tbl));
      lds_run<kLev>(tbl + te_off(0), tnext);
#pragma unroll
      for (int m = 0; m < 13; ++m) {
        const uint32_t d = dws[m];
        uint32_t tv[kLeft];
#pragma unroll
        for (int i = 0; i < kLeft; ++i) tv[i] = tnext[i];
        if (m + 1 < 13) {
          asm volatile("" : "+v"(tbl));
          if (m + 1 < 12) lds_run<kLev>(tbl + te_off(m + 1), tnext);
          else lds_run<kLeft>(tbl + te_off(m + 1), tnext);
        }
        // the four bytes of the code dword in the four 16-bit lanes of E
        // (bytes 0, 1 in the low dword, 2, 3 in the high one); after each
        // multiplication by 3 the high bytes of the lanes, bytes 1, 3 of each
        // dword, are gathered in byte order by one v_perm_b32
        uint64_t E = ((uint64_t)__builtin_amdgcn_perm(0u, d, 0x0C030C02u) << 32) |
                     (uint64_t)__builtin_amdgcn_perm(0u, d, 0x0C010C00u);
        auto high_bytes = [](uint64_t v) { return __builtin_amdgcn_perm((uint32_t)(v >> 32), (uint32_t)v, 0x07050301u); };
        if (m < 12) {
          // Summation by parts.  With h_j = floor(b 3^(j+1) / 256), the high
          // byte of the 16-bit lane after j + 1 multiplications by 3 (b 3^5
          // < 2^16, so nothing spills into the next lane), trit j is
          // h_j - 3 h_(j-1).  Hence sum_j t_j x_j = sum_{j<4} h_j x_j
          // - 3 sum_{j<3} h_j x_(j+1) + t_4 x_4, and h_0..h_3 <= 80 are valid
          // signed dot4 operands: no masking between the multiplications.
          uint32_t hprev = 0;
#pragma unroll
          for (int j = 0; j < 5; ++j) {
            E = times3(E);
            const uint32_t hj = high_bytes(E);
            if (j < 4) {
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                int& a1 = m < 6 ? ia[n] : ib[n];
                int& a3 = m < 6 ? ja[n] : jb[n];
                a1 = __builtin_amdgcn_sdot4((int)hj, (int)tv[j * NT + n], a1, false);
                if (j < 3) a3 = __builtin_amdgcn_sdot4((int)hj, (int)tv[(j + 1) * NT + n], a3, false);
              }
            } else {
              // t_4 = h_4 - 3 h_3 byte by byte, without borrows (each byte is 0..2)
              const int t4 = (int)(hj - 3u * hprev);
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                int& a1 = m < 6 ? ia[n] : ib[n];
                a1 = __builtin_amdgcn_sdot4(t4, (int)tv[4 * NT + n], a1, false);
              }
            }
            hprev = hj;
          }
        } else {
          // trit by trit: each 16-bit lane holds v < 256, after the
          // multiplication 3v < 768 and its high byte is the trit; the mask
          // keeps v_(j+1) = 3v mod 256 (the leftover dword pairs two groups)
#pragma unroll
          for (int j = 0; j < 5; ++j) {
            E = times3(E);
            const int t = (int)high_bytes(E);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              if (m < 6) {
                ia[n] = __builtin_amdgcn_sdot4(t, (int)tv[j * NT + n], ia[n], false);
              } else if (m < 12) {
                ib[n] = __builtin_amdgcn_sdot4(t, (int)tv[j * NT + n], ib[n], false);
              } else {
                ia[n] = __builtin_amdgcn_sdot4(t, (int)tv[2 * j * NT + n], ia[n], false);
                ib[n] = __builtin_amdgcn_sdot4(t, (int)tv[(2 * j + 1) * NT + n], ib[n], false);
              }
            }
            E &= 0x00FF00FF00FF00FFull;
          }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          asm volatile("" : "+v"(ia[n]), "+v"(ib[n]));
          asm volatile("" : "+v"(ja[n]), "+v"(jb[n]));
        }
      }
      const uint32_t s2 = gp == 0 ? sc8.x : gp == 1 ? sc8.y : gp == 2 ? sc8.z : sc8.w;
      const int g0 = sb * 8 + 2 * gp;
      if (g0 < G) {  // G is even: both groups of the pair exist
        // the groups' sums of q, then their d_x (the same q8_K block)
        const uint32_t* gs0 = tb + (8 * 6 * (2 * gp) + 6) * NT;
        const uint32_t* gs1 = tb + (8 * 6 * (2 * gp + 1) + 6) * NT;
        const double dw0 = (double)half_bits_to_float(s2 & 0xffffu);
        const double dw1 = (double)half_bits_to_float(s2 >> 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int I0 = ia[n] - 3 * ja[n] - (int)gs0[n];
          const int I1 = ib[n] - 3 * jb[n] - (int)gs1[n];
          if (IDOTS) {
            if (row < rows && tok0 + n < tokens) {
              const size_t o = ((size_t)(tok0 + n) * rows + row) * G + g0;
              idots[o] = I0;
              idots[o + 1] = I1;
            }
          } else {
            // inner = d_w1 I1 + d_w0 I0 (d_w0 I0 exact, one rounding), then
            // acc = d_x inner + acc (one rounding)
            const double inner = __builtin_fma(dw1, (double)I1, dw0 * (double)I0);
            acc[n] = __builtin_fma((double)__builtin_bit_cast(float, gs0[NT + n]), inner, acc[n]);
          }
        }
      }
    }
    if (!IDOTS) {
      // this wave has read the last of the superblock's table (LDS operations
      // of one wave complete in order): its sums take the table's place
      double* red = reinterpret_cast<double*>(table + (size_t)(sb - wg0) * kTableDwords * NT);
#pragma unroll
      for (int n = 0; n < NT; ++n) red[n * 64 + lane] = acc[n];
    }
  }
  if (IDOTS) return;
  __syncthreads();
  auto sb_sum = [&](int sb, int n) {
    return reinterpret_cast<const double*>(table + (size_t)(sb - wg0) * kTableDwords * NT)[n * 64 + lane];
  };
  if (nslices == 1) {
    // token n is summed by wave n mod nw, superblock by superblock
    for (int n = wave; n < NT; n += nw) {
      double s = sb_sum(wg0, n);
      for (int sb = wg0 + 1; sb < wg1; ++sb) s += sb_sum(sb, n);
      if (row < rows && tok0 + n < tokens) y[(size_t)(tok0 + n) * rows + row] = (float)s;
    }
    return;
  }
  if (wave != 0) return;
  // Several slices per tile (one token): the superblock sums go to the
  // workspace with agent-scope atomic stores (written through to the level
  // shared by all XCDs, so no whole-L2 write-back is needed); the counter is
  // bumped only after the stores have completed (vmcnt = 0).  The last
  // workgroup to arrive adds all the tile's superblock sums in order.
  double* partials = ws_partials(ws, tile);
  unsigned* counter = ws_counter(ws, tile);
  for (int sb = wg0; sb < wg1; ++sb)
    __hip_atomic_store(&partials[sb * 64 + lane], sb_sum(sb, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, 64);
  if (prev != (unsigned)(nslices - 1)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // eight superblock sums requested at a time before they are added (one
  // load and one add per superblock waited a full round trip each); indices
  // past the last superblock repeat it and are not added
  double t = 0.0;
  for (int sb0 = 0; sb0 < G8; sb0 += 8) {
    double pv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      pv[k] = __hip_atomic_load(&partials[min(sb0 + k, G8 - 1) * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (sb0 + k < G8) t = sb0 + k == 0 ? pv[0] : t + pv[k];
  }
  if (row < rows) y[row] = (float)t;
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  // up to 8 waves of one or more superblocks (measured on 32768 x 8192: 8
  // waves of one superblock, 19.4 us, beat 4 waves of two, 20.8 us)
  const int waves = p.scw < kMaxWaves ? p.scw : kMaxWaves;
  p.spw = (p.scw + waves - 1) / waves;
  p.waves = (p.scw + p.spw - 1) / p.spw;
  return p;
}

namespace {

template <bool IDOTS, int NT>
void launch_ptq1(const dim3& grid, const dim3& block, size_t lds, hipStream_t s, const uint4* codes,
                 const uint4* scales, const int8_t* q, const float* dx, const int16_t* bsums, float* y, int32_t* idots,
                 const Dims& dm, const GemvPlan& p, uint8_t* ws, int tokens) {
  hipLaunchKernelGGL((gemv_ptq1_kernel<IDOTS, NT>), grid, block, lds, s, codes, scales, q, dx, bsums, y, idots,
                     (int)dm.rows, (int)dm.G, (int)dm.G8, p.scw, p.spw, ws, tokens);
}

template <int NT>
void launch_ptq1_nt(bool idots_out, const dim3& grid, const dim3& block, size_t lds, hipStream_t s,
                    const uint4* codes, const uint4* scales, const int8_t* q, const float* dx, const int16_t* bsums,
                    float* y, int32_t* idots, const Dims& dm, const GemvPlan& p, uint8_t* ws, int tokens) {
  if (idots_out)
    launch_ptq1<true, NT>(grid, block, lds, s, codes, scales, q, dx, bsums, y, idots, dm, p, ws, tokens);
  else
    launch_ptq1<false, NT>(grid, block, lds, s, codes, scales, q, dx, bsums, y, idots, dm, p, ws, tokens);
}

}  // namespace

hipError_t launch_gemv_ptq1_plan(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx,
                                 const int16_t* bsums, float* y, int32_t* idots, void* workspace, const GemvPlan& p,
                                 hipStream_t s) {
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint4* scales = reinterpret_cast<const uint4*>(w + kPtq1ScaleOffset);  // the first unit's scales
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const dim3 grid((unsigned)dm.ntiles, (unsigned)p.slices), block(64 * p.waves);
  launch_ptq1_nt<1>(idots != nullptr, grid, block, ptq1_lds_bytes(p.scw, 1), s, codes, scales, q, dx, bsums, y, idots,
                    dm, p, ws, 1);
  return hipGetLastError();
}

hipError_t launch_gemv_ptq1(const uint8_t* w, const Dims& dm, const int8_t* q, const float* dx, const int16_t* bsums,
                            float* y, int32_t* idots, void* workspace, hipStream_t s) {
  const GemvPlan p = plan_gemv_ptq1(dm, workspace != nullptr && idots == nullptr);
  return launch_gemv_ptq1_plan(w, dm, q, dx, bsums, y, idots, workspace, p, s);
}

int ptq1_token_block(const Dims& dm, int64_t tokens) {
  // Blocks of 2 tokens where the LDS budget allows (measured on 17408 x 5120
  // with blocks of 1 / 2 / 4: 4 tokens 29.0 / 20.9 / 21.9 us): one decode
  // serves two tokens, and two tokens take summation by parts.
  const GemvPlan p = plan_gemv_ptq1(dm, false);
  int nt = 1;
  while (nt < kMaxTokBlock && nt < tokens && ptq1_lds_bytes(p.scw, 2 * nt) <= kLdsBudget) nt *= 2;
  return nt;
}

hipError_t launch_gemm_ptq1(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx,
                            const int16_t* bsums, float* y, int32_t* idots, hipStream_t s) {
  // From 8 tokens on the MFMA kernel (measured on 17408 x 5120, vector
  // units / MFMA: 4 tokens 20.2 / 28.3 us, 8 tokens 34.2 / 28.1, 16 tokens
  // 48.6 / 28.4, 64 tokens 163 / 56.6); it sums in the same order.
  if (tokens >= kMfmaMinTokens) return launch_gemm_ptq1_mfma(w, dm, tokens, q, dx, bsums, y, idots, s);
  // one workgroup per tile and token block, with the one-token plan's waves
  // (the summation order does not depend on the split)
  const GemvPlan p = plan_gemv_ptq1(dm, false);
  const int nt = ptq1_token_block(dm, tokens);
  const uint4* codes = reinterpret_cast<const uint4*>(w);
  const uint4* scales = reinterpret_cast<const uint4*>(w + kPtq1ScaleOffset);  // the first unit's scales
  const dim3 grid((unsigned)dm.ntiles, 1u, (unsigned)((tokens + nt - 1) / nt)), block(64 * p.waves);
  const size_t lds = ptq1_lds_bytes(p.scw, nt);
  const bool io = idots != nullptr;
  const int T = (int)tokens;
  if (nt == 1)
    launch_ptq1_nt<1>(io, grid, block, lds, s, codes, scales, q, dx, bsums, y, idots, dm, p, nullptr, T);
  else
    launch_ptq1_nt<2>(io, grid, block, lds, s, codes, scales, q, dx, bsums, y, idots, dm, p, nullptr, T);
  return hipGetLastError();
}

}  // namespace tq
