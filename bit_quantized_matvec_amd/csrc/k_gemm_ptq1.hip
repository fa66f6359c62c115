// k_gemm_ptq1.hip -- prompt (several-token) product, repacked ptq1_0 x q8_K,
// on int8 MFMA.
//
// Same arithmetic per token as the matrix-vector product of k_gemv_ptq1.hip
// (page 1, "the detour that lost": trit j of code byte b is
// floor(3 ((b 3^j) mod 256) / 256) and w = trit - 1; "prefill wants a
// different shape": with many tokens a decoded weight is reused, so the dot
// products belong on the matrix cores).
//
// How (gfx950):
//   * v_mfma_i32_16x16x64_i8: a wave owns 16 rows of a 64-row tile and the
//     workgroup's 16 tokens; lane (r, qd) = (lane % 16, lane / 16) supplies
//     row r's k-slots 16 qd .. 16 qd + 15 of A and token r's of B.
//   * A group (128 weights, 6 full code dwords and half of a leftover dword)
//     takes three MFMAs.  Lane qd decodes two code dwords into trit dwords
//     (byte i of trit dword j = trit j of code byte i): X = dword qd and
//     Y = dword qd + 4 (qd < 2), the leftover dword (qd = 2) or nothing
//     useful (qd = 3).  Its three A pieces are [X0..X3], [X4, Y0..Y2],
//     [Y3, Y4, 0, 0]; B holds zeros wherever A holds nothing of the group
//     (qd = 3's Y, the other group's half of the leftover dword, the padding
//     trits of byte 25), so C = the group's sum of trit x q and the integer
//     dot is C minus the group's sum of q (trit = w + 1).
//   * B is the matching permutation of q: for trit dword (c, j) the four
//     activations 5 apart, q[20 c + j + 5 i], i = 0..3.  Per superblock each
//     lane builds the three B pieces of one (token, slot) for two groups from
//     40 bytes of q held in registers (loaded a superblock ahead, two byte
//     permutes per entry) and stores them in [group][step][token][qd] order,
//     so that one MFMA's B is one 16-byte read per lane.
//   * The fp64 epilogue per group pair (groups 2p, 2p + 1 share d_x):
//     inner = d_w(2p+1) I1 + d_w(2p) I0 (one rounding), acc = d_x inner + acc
//     (one rounding), acc from zero per superblock, superblock sums added in
//     order.  The matrix-vector product uses the same sequence, so every
//     token's output is bit-identical to it.
//   * Workgroup = 4 waves = one 64-row tile and 16 tokens (29 KiB of LDS,
//     142 VGPRs: three workgroups per compute unit); each lane loads exactly
//     the code dwords it decodes (16 per superblock), and those and the q
//     bytes and scales of the next superblock are loaded while the current
//     ones are used.
//   * Tokens past the end read a valid token (the last) and rows past the
//     end have zero codes and scales; neither is stored.
#include <algorithm>

#include "kernels.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;  // tokens per workgroup (MFMA columns)

struct Stage {
  v4u bimg[8][3][kTok][4];  // B pieces [group][step][token][qd], 24 KiB
  double dw[8][64];         // d_w [group][row of the tile], 4 KiB
  int qs[8][kTok];          // sum of q per group
  double dxs[4][kTok];      // d_x per q8_K block of the superblock
};

__device__ __forceinline__ uint64_t times3(uint64_t x) {
  uint64_t r;
  asm("v_lshl_add_u64 %0, %1, 1, %1" : "=v"(r) : "v"(x));
  return r;
}

// The five trit dwords of a code dword: byte i of t[j] is trit j of byte i.
// The four bytes sit in the 16-bit lanes of a 64-bit register; each
// multiplication by 3 moves the next trit into the high byte of every lane,
// and the mask keeps (b 3^j) mod 256 for the next level.
__device__ __forceinline__ void trits5(uint32_t d, uint32_t* t) {
  uint64_t E = ((uint64_t)__builtin_amdgcn_perm(0u, d, 0x0C030C02u) << 32) |
               (uint64_t)__builtin_amdgcn_perm(0u, d, 0x0C010C00u);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    E = times3(E);
    t[j] = __builtin_amdgcn_perm((uint32_t)(E >> 32), (uint32_t)E, 0x07050301u);
    if (j < 4) E &= 0x00FF00FF00FF00FFull;
  }
}

__device__ __forceinline__ double half_to_double(uint32_t h) {
  return (double)static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h));
}

// grid = (ntiles, ceil(tokens / 16)); wave w owns rows 16 w .. 16 w + 15 of
// its tile.
template <bool IDOTS>
__global__ __launch_bounds__(256) void gemm_ptq1_kernel(const v4u* __restrict__ codes, const v4u* __restrict__ scales,
                                                        const int8_t* __restrict__ q, const float* __restrict__ dx,
                                                        const int16_t* __restrict__ bsums, float* __restrict__ y,
                                                        int32_t* __restrict__ idots, int rows, int G, int G8,
                                                        int tokens) {
  __shared__ Stage st;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;  // row of A, token of B and C
  const int qd = lane >> 4;
  const int tile = blockIdx.x;
  const int tok0 = blockIdx.y * kTok;
  const size_t K = (size_t)G * 128;

  // ---- staging inputs of a superblock, loaded a superblock ahead
  // q for the B pieces: lane (n, qd) = (lane / 4, lane % 4) of wave w builds
  // token n's pieces of slot qd for groups w and w + 4 (item k = 0, 1).  It
  // reads the 20 bytes of code dword qd's partners (X) and those of code
  // dword qd + 4 (Y, qd < 2) or the group's last 20 bytes (qd >= 2: bytes
  // 120 .. 127 are the leftover dword's partners; qd = 3 uses none of it).
  // Groups past G and tokens past the end read valid bytes that no stored
  // output uses.
  const int bn = lane >> 2, bq = lane & 3;
  const int bx = 20 * bq, by = bq < 2 ? 20 * (bq + 4) : 108;
  uint32_t qx[2][5], qy[2][5];
  auto load_q = [&](int sb) {
    const size_t t = (size_t)min(tok0 + bn, tokens - 1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int g = min(sb * 8 + wave + 4 * k, G - 1);
      const uint32_t* src = reinterpret_cast<const uint32_t*>(q + t * K + (size_t)g * 128);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        qx[k][i] = src[bx / 4 + i];
        qy[k][i] = src[by / 4 + i];
      }
    }
  };
  // scales (threads 0..63: one row's 8 fp16), partial sums (threads 0..127:
  // one token and group), d_x (threads 0..63: one token and q8_K block)
  v4u sc_in;
  uint32_t bs_in[4];
  float dx_in;
  auto load_side = [&](int sb) {
    sc_in = scales[((size_t)tile * G8 + sb) * (kPtq1UnitBytes / 16) + lane];
    {
      const int n = (tid & 127) >> 3, g = min(sb * 8 + (tid & 7), G - 1);
      const size_t t = (size_t)min(tok0 + n, tokens - 1);
      // the 8 partial sums as words (the hardware's unaligned global loads
      // cover a buffer that is only 2-byte aligned)
      const uint32_t* src = reinterpret_cast<const uint32_t*>(bsums + t * (K / 16) + (size_t)g * 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) bs_in[k] = src[k];
    }
    {
      const int n = lane >> 2, kb = min(sb * 4 + (lane & 3), G / 2 - 1);
      const size_t t = (size_t)min(tok0 + n, tokens - 1);
      dx_in = dx ? dx[t * (K / 256) + kb] : 0.0f;
    }
  };
  auto store_side = [&]() {
    if (tid < 64) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t w = sc_in[g >> 1];
        st.dw[g][tid] = half_to_double((g & 1) ? (w >> 16) : (w & 0xffffu));
      }
      st.dxs[tid & 3][tid >> 2] = (double)dx_in;
    }
    if (tid < 128) {
      int s = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) s += (int)(int16_t)(bs_in[k] & 0xffffu) + ((int)bs_in[k] >> 16);
      st.qs[tid & 7][tid >> 3] = s;
    }
  };
  // B pieces from the q registers.  Trit dword j of a code dword is partnered
  // by its bytes' activations 5 apart: from 20 bytes w (5 dwords) entry e[j]
  // holds bytes j, 5 + j, 10 + j, 15 + j (two byte permutes of two dwords
  // each, merged).  Pieces of slot qd: [X0..X3], [X4, Y0..Y2], [Y3, Y4, 0, 0]
  // with X = code dword qd's entries and Y = code dword qd + 4's (qd < 2),
  // the leftover dword's (qd = 2: the group's bytes 24, 25 in its half of the
  // dword -- low half for an even group -- and zeros in the other half, the
  // padding trits of byte 25 meeting zeros) or zeros (qd = 3).
  auto entries = [](const uint32_t* w, uint32_t* e) __attribute__((always_inline)) {
    e[0] = __builtin_amdgcn_perm(w[1], w[0], 0x0C0C0500u) | __builtin_amdgcn_perm(w[3], w[2], 0x07020C0Cu);
    e[1] = __builtin_amdgcn_perm(w[1], w[0], 0x0C0C0601u) | __builtin_amdgcn_perm(w[4], w[2], 0x04030C0Cu);
    e[2] = __builtin_amdgcn_perm(w[1], w[0], 0x0C0C0702u) | __builtin_amdgcn_perm(w[4], w[3], 0x05000C0Cu);
    e[3] = __builtin_amdgcn_perm(w[2], w[0], 0x0C0C0403u) | __builtin_amdgcn_perm(w[4], w[3], 0x06010C0Cu);
    e[4] = __builtin_amdgcn_perm(w[2], w[1], 0x0C0C0500u) | __builtin_amdgcn_perm(w[4], w[3], 0x07020C0Cu);
  };
  auto build_b = [&]() {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int g = wave + 4 * k;
      uint32_t ex[5], ey[5];
      entries(qx[k], ex);
      if (bq < 2) {
        entries(qy[k], ey);
      } else if (bq == 2) {
        // bytes 120 .. 123 and 124 .. 127 of the group are qy[k][3], qy[k][4]
        const uint32_t u_lo = qy[k][3], u_hi = qy[k][4];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const uint32_t a = j < 4 ? (u_lo >> (8 * j)) & 0xffu : u_hi & 0xffu;  // q[120 + j]: byte 24
          const uint32_t b = j < 3 ? (u_hi >> (8 * (j + 1))) & 0xffu : 0u;      // q[125 + j]: byte 25
          const uint32_t lo = a | (b << 8);
          ey[j] = (g & 1) ? lo << 16 : lo;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 5; ++j) ey[j] = 0u;
      }
      st.bimg[g][0][bn][bq] = v4u{ex[0], ex[1], ex[2], ex[3]};
      st.bimg[g][1][bn][bq] = v4u{ex[4], ey[0], ey[1], ey[2]};
      st.bimg[g][2][bn][bq] = v4u{ey[3], ey[4], 0u, 0u};
    }
  };

  // ---- codes: each lane loads exactly the code dwords it decodes, a
  // superblock ahead.  Dword D of a row's superblock is component D % 4 of
  // uint4 D / 4 (the repacked [L][row] order); for pair p lane qd needs
  // X_a = D(12 p + qd), X_b = D(12 p + 6 + qd) and Y_a = D(12 p + 4 + qd),
  // Y_b = D(12 p + 10 + qd) (qd < 2) or the leftover D(48 + p) (qd >= 2).
  const uint8_t* cb = reinterpret_cast<const uint8_t*>(codes) + (size_t)tile * G8 * kPtq1UnitBytes + (16 * wave + r) * 16;
  const int xa0 = 4 * qd, xb0 = (1 + (qd >> 1)) * 1024 + 4 * ((2 + qd) & 3);
  const int ya0 = qd < 2 ? 1024 + 4 * qd : 12 * 1024, yb0 = qd < 2 ? 2048 + 4 * (2 + qd) : 12 * 1024;
  const int ys = qd < 2 ? 3072 : 4;  // per pair
  uint32_t cdw[16], cdn[16];          // [pair][X_a, X_b, Y_a, Y_b]
  auto load_codes = [&](int sb) {
    const uint8_t* b = cb + (size_t)sb * kPtq1UnitBytes;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      cdn[4 * p] = *reinterpret_cast<const uint32_t*>(b + xa0 + 3072 * p);
      cdn[4 * p + 1] = *reinterpret_cast<const uint32_t*>(b + xb0 + 3072 * p);
      cdn[4 * p + 2] = *reinterpret_cast<const uint32_t*>(b + ya0 + ys * p);
      cdn[4 * p + 3] = *reinterpret_cast<const uint32_t*>(b + yb0 + ys * p);
    }
  };

  double total[4] = {0.0, 0.0, 0.0, 0.0};
  load_q(0);
  load_side(0);
  load_codes(0);
  for (int sb = 0; sb < G8; ++sb) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this superblock's q, codes and side inputs have landed
    __syncthreads();                          // ... for every wave; the last superblock's reads are done
    store_side();
    build_b();
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) cdw[k] = cdn[k];
    const int sbn = min(sb + 1, G8 - 1);  // the last superblock re-reads itself: no branch, exact waits
    load_q(sbn);
    load_side(sbn);
    load_codes(sbn);

    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const int npairs = min(4, (G - sb * 8) / 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p >= npairs) break;  // the last superblock of a row may hold fewer groups (uniform)
      v4i cacc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * p + h;
        const uint32_t xd = cdw[4 * p + h], yd = cdw[4 * p + 2 + h];
        uint32_t t[10];
        trits5(xd, t);
        trits5(yd, t + 5);
        const v4i a0 = {(int)t[0], (int)t[1], (int)t[2], (int)t[3]};
        const v4i a1 = {(int)t[4], (int)t[5], (int)t[6], (int)t[7]};
        const v4i a2 = {(int)t[8], (int)t[9], 0, 0};
        const v4u b0 = st.bimg[g][0][r][qd], b1 = st.bimg[g][1][r][qd], b2 = st.bimg[g][2][r][qd];
        v4i cz = {0, 0, 0, 0};
        cz = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, v4i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w}, cz, 0, 0, 0);
        cz = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, v4i{(int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w}, cz, 0, 0, 0);
        cz = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, v4i{(int)b2.x, (int)b2.y, (int)b2.z, (int)b2.w}, cz, 0, 0, 0);
        cacc[h] = cz;
      }
      // epilogue: lane holds C[row 4 qd + i][token r] of both groups
      const int qa = st.qs[2 * p][r], qb = st.qs[2 * p + 1][r];
      const double dxp = st.dxs[p][r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rt = 16 * wave + 4 * qd + i;  // row within the tile
        const int I0 = cacc[0][i] - qa, I1 = cacc[1][i] - qb;
        if (IDOTS) {
          const int row = tile * 64 + rt, tk = tok0 + r;
          if (row < rows && tk < tokens) {
            const size_t o = ((size_t)tk * rows + row) * G + sb * 8 + 2 * p;
            idots[o] = I0;
            idots[o + 1] = I1;
          }
        } else {
          const double inner = __builtin_fma(st.dw[2 * p + 1][rt], (double)I1, st.dw[2 * p][rt] * (double)I0);
          acc[i] = __builtin_fma(dxp, inner, acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) total[i] = sb == 0 ? acc[i] : total[i] + acc[i];
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // no load outstanding at exit
  if (IDOTS) return;
  const int tk = tok0 + r;
  if (tk >= tokens) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile * 64 + 16 * wave + 4 * qd + i;
    if (row < rows) y[(size_t)tk * rows + row] = (float)total[i];
  }
}

}  // namespace

hipError_t launch_gemm_ptq1_mfma(const uint8_t* w, const Dims& dm, int64_t tokens, const int8_t* q, const float* dx,
                                 const int16_t* bsums, float* y, int32_t* idots, hipStream_t s) {
  const v4u* codes = reinterpret_cast<const v4u*>(w);
  const v4u* scales = reinterpret_cast<const v4u*>(w + kPtq1ScaleOffset);  // the first unit's scales
  // The token blocks go in grid.y, whose extent is kept below 2^16: longer
  // prompts are launched in chunks of 2^15 token blocks, each with its
  // tokens' activations and outputs.
  constexpr int64_t kChunk = int64_t(kTok) << 15;
  const int64_t K = dm.cols, R = dm.rows, G = dm.G;
  for (int64_t t0 = 0; t0 < tokens; t0 += kChunk) {
    const int64_t nt = std::min(kChunk, tokens - t0);
    const int8_t* qc = q + t0 * K;
    const float* dxc = dx ? dx + t0 * (K / 256) : nullptr;
    const int16_t* bc = bsums + t0 * (K / 16);
    const dim3 grid((unsigned)dm.ntiles, (unsigned)((nt + kTok - 1) / kTok)), block(256);
    if (idots)
      hipLaunchKernelGGL((gemm_ptq1_kernel<true>), grid, block, 0, s, codes, scales, qc, dxc, bc, nullptr,
                         idots + t0 * R * G, (int)R, (int)G, (int)dm.G8, (int)nt);
    else
      hipLaunchKernelGGL((gemm_ptq1_kernel<false>), grid, block, 0, s, codes, scales, qc, dxc, bc, y + t0 * R,
                         nullptr, (int)R, (int)G, (int)dm.G8, (int)nt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
