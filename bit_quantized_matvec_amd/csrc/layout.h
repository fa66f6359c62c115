// layout.h -- device layouts written by the repack and read by the kernels.
//
// Internal to libtq.  The layouts are chosen for gfx950 (wave64, dwordx4
// loads, v_dot4_i32_i8 and v_mfma_i32_16x16x64_i8), not copied from the
// pages' 4-row NEON block; the principle kept from "the layout" section of
// page 1 is that extracting one operand costs one mask (plus one shift).
//
// pq2_0 repacked
//   Rows are grouped in tiles of 64 (padded with zero weights and zero
//   scales).  Columns are grouped in superchunks of 256 (two 128-groups).
//   One 4352-byte unit per (tile, sc), units tile-major: the codes (4096 B)
//   then the scale pairs (256 B), so that a superchunk is one contiguous read.
//   codes: uint4 [qd 0..3][row 0..63] of the unit; within the 16 bytes, dword c
//     (0..3), byte j (0..3), 2-bit field s (bits 2s..2s+1) holds w, as a 2-bit
//     two's-complement number (-1 -> 3, 0 -> 0, +1 -> 1), of column
//         256*sc + 64*c + 16*qd + 4*s + j.
//     Dwords c = 0,1 belong to group 2*sc, c = 2,3 to group 2*sc+1.
//     A wave with one row per lane reads qd = 0..3 as four fully coalesced
//     1 KiB loads; `(dword << (6 - 2s)) & 0xC0C0C0C0` gives 64*w for four
//     consecutive columns, the int8 operand of one dot4 against one
//     activation dword.  For the MFMA path, lane (row, qd) holds dword c,
//     whose four fields cover columns 64c + 16qd + [0, 16): a 16x16x64 MFMA
//     takes chunk c of 16 rows and its B operand is 16 contiguous bytes of q.
//   scales: uint32 [row 0..63] after the unit's codes: the fp16 scales of groups 2 sc (low
//     half) and 2 sc + 1 (high half) of the row.  A wave with one row per lane
//     reads a superchunk's scales as one 256-byte request; the MFMA path reads
//     the pairs of four consecutive rows as one 16-byte load.
//
// ptq1_0 repacked (1.75 bits per weight kept, bytes only reordered)
//   One 14336-byte unit per (tile, sb), sb = superblock of 8 groups, units
//   tile-major: the codes (13312 B) then the scales (1024 B).
//   codes: uint4 [L 0..12][row 0..63] of the unit.
//     The 52 dwords D = 4L + c of a row's superblock hold the 8 x 26 code
//     bytes: D = 6*gi + m (gi < 8, m < 6) holds bytes 4m..4m+3 of group gi;
//     D = 48 + p (p < 4) holds bytes 24, 25 of group 2p, then bytes 24, 25 of
//     group 2p+1.  Bytes are copied unchanged (padding trits included).
//   scales: fp16 [row 0..63][8] after the unit's codes: the scale of group g
//     of a row is entry g % 8 of the unit of superblock g / 8 (groups padded
//     to a multiple of 8 with 0).
#pragma once
#include <stdint.h>

namespace tq {

constexpr int kRowTile = 64;
constexpr int kGroup = 128;
constexpr int kSuper = 256;  // pq2_0 superchunk columns
constexpr int kPtqSuperGroups = 8;
constexpr int kPtqLoads = 13;  // uint4 per row per ptq1_0 superblock

struct Dims {
  int64_t rows, cols;
  int64_t ntiles;  // ceil(rows / 64)
  int64_t G;       // cols / 128
  int64_t G8;      // ceil(G / 8)
  int64_t nsc;     // cols / 256
};

inline Dims dims(int64_t rows, int64_t cols) {
  Dims d;
  d.rows = rows;
  d.cols = cols;
  d.ntiles = (rows + kRowTile - 1) / kRowTile;
  d.G = cols / kGroup;
  d.G8 = (d.G + 7) / 8;
  d.nsc = cols / kSuper;
  return d;
}

// pq2_0 is stored as one unit per (row tile, superchunk), tile-major: the
// unit's 4096 bytes of codes (uint4 [qd][row]) and then its 256 bytes of
// scale pairs (uint32 [row]), so that a superchunk is one contiguous read.
constexpr int64_t kPq2UnitBytes = 4352;
constexpr int64_t kPq2ScaleOffset = 4096;  // bytes from a unit's start to its scale pairs

// ptq1_0 likewise: one unit per (row tile, 8-group superblock): its 13
// code loads (uint4 [L][row], 13312 bytes), then its fp16 scales
// ([row][8], 1024 bytes).
constexpr int64_t kPtq1UnitBytes = 14336;
constexpr int64_t kPtq1ScaleOffset = 13312;

// Byte sizes of the repacked buffers (the code and scale shares of the
// units).
inline int64_t pq2_code_bytes(const Dims& d) { return d.ntiles * d.nsc * 4 * 64 * 16; }
inline int64_t ptq1_code_bytes(const Dims& d) { return d.ntiles * d.G8 * kPtqLoads * 64 * 16; }
inline int64_t pq2_scale_bytes(const Dims& d) { return d.ntiles * d.nsc * 64 * 4; }
inline int64_t ptq1_scale_bytes(const Dims& d) { return d.ntiles * d.G8 * 64 * 8 * 2; }

}  // namespace tq
