"""Seeded synthetic inputs for the packed-ternary matvec / matmul workloads.

Test infrastructure shared by the CPU oracle and the GPU path.  This module
holds no arithmetic of the method itself: it only draws random numbers and
lays them out in the canonical storage formats, so that both sides consume
byte-identical inputs.

Canonical formats (the storage of the files the pages describe):

* pq2_0 block, 34 bytes per 128 weights of one row: little-endian fp16 scale
  ``d`` followed by ``qs[32]``.  Weight ``k`` of the block is the 2-bit code
  ``u = w + 1`` in byte ``k >> 2``, bits ``2*(k & 3)`` and up (low bits first,
  the order of the pages' packer in "the layout" section of
  "how i made a 27b ternary model 3.8x faster...").  Blocks are row-major by
  (row, group).
* ptq1_0 block, 28 bytes per 128 weights: fp16 ``d`` then ``qs[26]``; weight
  ``k`` is trit ``k % 5`` of byte ``k // 5`` (5 trits per byte, "the detour
  that lost").  Trits 3 and 4 of byte 25 are padding.
* activations: fp32 ``[tokens][cols]``.

Distributions follow the workload list: codes uniform over {0, 1, 2}; fp16
scales uniform in [0.01, 0.05] (rounded to fp16); activations N(0, 1) fp32;
ptq1_0 bytes uniform in [0, 242].
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20261202

# Workload ids used in seeds.
TINY, DECODE, PREFILL, STEP64, PTQ1, PTQ1_PREFILL = 1, 2, 3, 4, 5, 6

# The 81 bytes whose four 2-bit fields all lie in {0, 1, 2}.  Drawing a byte
# uniformly from this list draws its four codes independently and uniformly.
VALID_PQ2_BYTES = np.array(
    [b for b in range(256) if all(((b >> (2 * s)) & 3) != 3 for s in range(4))],
    dtype=np.uint8,
)
assert VALID_PQ2_BYTES.size == 81

PQ2_BLOCK = 34
PTQ1_BLOCK = 28
GROUP = 128

# Matrix shapes of one synthetic 64-layer decode step (rows, cols).
STEP64_SHAPES = (
    ("gate", 17408, 5120),
    ("up", 17408, 5120),
    ("down", 5120, 17408),
    ("qkv", 7168, 5120),
    ("out", 5120, 6144),
)


def rng(workload: int, layer: int = 0, matrix: int = 0, extra: int = 0) -> np.random.Generator:
    """PCG64 generator seeded from (base, workload, layer, matrix, extra)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, workload, layer, matrix, extra])))


def pq2_codes(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Packed code bytes, shape [rows, cols/128, 32], uniform valid codes."""
    idx = g.integers(0, 81, size=(rows, cols // GROUP, 32), dtype=np.uint8)
    return VALID_PQ2_BYTES[idx]


def scales_f16(g: np.random.Generator, rows: int, cols: int, lo: float = 0.01, hi: float = 0.05) -> np.ndarray:
    """fp16 scales [rows, cols/128], uniform in [lo, hi] then rounded to fp16."""
    return g.uniform(lo, hi, size=(rows, cols // GROUP)).astype(np.float16)


def assemble_pq2(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Lay out [rows, G, 32] code bytes + [rows, G] fp16 scales as pq2_0 blocks."""
    rows, G, _ = codes.shape
    blk = np.empty((rows, G, PQ2_BLOCK), dtype=np.uint8)
    blk[:, :, 0:2] = np.ascontiguousarray(scales.astype("<f2")).view(np.uint8).reshape(rows, G, 2)
    blk[:, :, 2:] = codes
    return blk


def assemble_ptq1(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Lay out [rows, G, 26] trit bytes + [rows, G] fp16 scales as ptq1_0 blocks."""
    rows, G, _ = codes.shape
    blk = np.empty((rows, G, PTQ1_BLOCK), dtype=np.uint8)
    blk[:, :, 0:2] = np.ascontiguousarray(scales.astype("<f2")).view(np.uint8).reshape(rows, G, 2)
    blk[:, :, 2:] = codes
    return blk


def pq2_matrix(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """A canonical pq2_0 matrix [rows, cols/128, 34] (codes drawn first, then scales)."""
    codes = pq2_codes(g, rows, cols)
    sc = scales_f16(g, rows, cols)
    return assemble_pq2(codes, sc)


def ptq1_matrix(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """A canonical ptq1_0 matrix [rows, cols/128, 28]: bytes uniform in [0, 242], then scales."""
    codes = g.integers(0, 243, size=(rows, cols // GROUP, 26), dtype=np.uint8)
    sc = scales_f16(g, rows, cols)
    return assemble_ptq1(codes, sc)


def activations(g: np.random.Generator, tokens: int, cols: int) -> np.ndarray:
    """fp32 activations [tokens, cols], N(0, 1)."""
    return g.standard_normal(size=(tokens, cols), dtype=np.float32)


def workload(name: str):
    """(fmt, rows, cols, tokens, seed-id) of a named workload."""
    table = {
        "tiny_256x1024": ("pq2_0", 256, 1024, 1, TINY),
        "decode_32768x8192": ("pq2_0", 32768, 8192, 1, DECODE),
        "prefill_17408x5120_t4": ("pq2_0", 17408, 5120, 4, PREFILL),
        "prefill_17408x5120_t64": ("pq2_0", 17408, 5120, 64, PREFILL),
        "ptq1_32768x8192": ("ptq1_0", 32768, 8192, 1, PTQ1),
        "ptq1_prefill_17408x5120_t4": ("ptq1_0", 17408, 5120, 4, PTQ1_PREFILL),
        "ptq1_prefill_17408x5120_t64": ("ptq1_0", 17408, 5120, 64, PTQ1_PREFILL),
    }
    return table[name]


def make(name: str, tokens: int | None = None):
    """Generate (canonical weights, fp32 activations) for a named workload."""
    fmt, rows, cols, t, wid = workload(name)
    if tokens is not None:
        t = tokens
    g = rng(wid)
    w = pq2_matrix(g, rows, cols) if fmt == "pq2_0" else ptq1_matrix(g, rows, cols)
    x = activations(g, t, cols)
    return fmt, w, x
