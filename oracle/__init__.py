"""CPU oracle for the packed-ternary x q8_K products (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never does, and this package never imports
the product library.  The arithmetic lives in ``tq_oracle.c`` (plain C, built
with gcc); this module only marshals numpy arrays and splits rows over threads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

FMT = {"pq2_0": 1, "ptq1_0": 2}
BLOCK_BYTES = {"pq2_0": 34, "ptq1_0": 28}


def build(force: bool = True) -> str:
    """Compile tq_oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def load(path: str):
    """Load a compiled oracle library and declare its signatures."""
    L = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.tqo_half_to_float.argtypes = [ctypes.c_uint16]
    L.tqo_half_to_float.restype = ctypes.c_float
    L.tqo_decode_rows.argtypes = [i32, p, i64, i64, i64, p, p]
    L.tqo_decode_rows.restype = i64
    L.tqo_quantize_rows.argtypes = [p, i64, i64, i64, p, p, p]
    L.tqo_quantize_rows.restype = None
    L.tqo_group_dots.argtypes = [i32, p, i64, i64, p, i64, i64, p]
    L.tqo_group_dots.restype = i32
    L.tqo_matmul.argtypes = [i32, p, i64, i64, p, p, i64, i64, p, p, i64]
    L.tqo_matmul.restype = i32
    return L


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load(LIB)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _chunks(n: int, threads: int):
    threads = max(1, min(threads, n))
    step = -(-n // threads)
    return [(s, min(n, s + step)) for s in range(0, n, step)]


def half_to_float(h: int) -> float:
    return lib().tqo_half_to_float(int(h))


def decode(fmt: str, W: np.ndarray):
    """Canonical blocks [rows, G, bytes] -> (w int8 [rows, cols], d fp32 [rows, G], invalid-code count)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    rows, G, bb = W.shape
    assert bb == BLOCK_BYTES[fmt]
    cols = G * 128
    w = np.empty((rows, cols), dtype=np.int8)
    d = np.empty((rows, G), dtype=np.float32)
    bad = lib().tqo_decode_rows(FMT[fmt], _ptr(W), cols, 0, rows, _ptr(w), _ptr(d))
    return w, d, int(bad)


def quantize_q8k(x: np.ndarray, threads: int = 1):
    """fp32 [tokens, cols] -> (q int8 [T, cols], d fp32 [T, cols/256], bsums int16 [T, cols/16])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, K = x.shape
    assert K % 256 == 0
    q = np.empty((T, K), dtype=np.int8)
    d = np.empty((T, K // 256), dtype=np.float32)
    bs = np.empty((T, K // 16), dtype=np.int16)
    L = lib()

    def run(rng):
        L.tqo_quantize_rows(_ptr(x), K, rng[0], rng[1], _ptr(q), _ptr(d), _ptr(bs))

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, _chunks(T, threads)))
    return q, d, bs


def group_dots(fmt: str, W: np.ndarray, q: np.ndarray, rows=None, threads: int = 1) -> np.ndarray:
    """Exact int32 group dots I[t, r, g] for the selected rows (default all)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    R, G, _ = W.shape
    T, K = q.shape
    assert K == G * 128
    r0, r1 = (0, R) if rows is None else rows
    nr = r1 - r0
    out = np.empty((T, nr, G), dtype=np.int32)
    L = lib()
    parts = _chunks(nr, threads)
    bufs = [np.empty((T, b - a, G), dtype=np.int32) for a, b in parts]

    def run(i):
        a, b = parts[i]
        rc = L.tqo_group_dots(FMT[fmt], _ptr(W), K, T, _ptr(q), r0 + a, r0 + b, _ptr(bufs[i]))
        if rc:
            raise OverflowError("group dot does not fit int32")

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, range(len(parts))))
    for (a, b), buf in zip(parts, bufs):
        out[:, a:b, :] = buf
    return out


def matmul(fmt: str, W: np.ndarray, q: np.ndarray, dx: np.ndarray, rows=None, threads: int = 1, with_mag: bool = False):
    """y[t, r] (fp32) for rows r in [r0, r1) (default all); optionally sum_g |term| (fp64)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    dx = np.ascontiguousarray(dx, dtype=np.float32)
    R, G, _ = W.shape
    T, K = q.shape
    assert K == G * 128 and dx.shape == (T, K // 256)
    r0, r1 = (0, R) if rows is None else rows
    nr = r1 - r0
    y = np.empty((T, nr), dtype=np.float32)
    mag = np.empty((T, nr), dtype=np.float64) if with_mag else None
    L = lib()

    def run(rng):
        # The C routine writes y[t * stride + (r - first row)]: point it at column a.
        a, b = rng
        L.tqo_matmul(FMT[fmt], _ptr(W), K, T, _ptr(q), _ptr(dx), r0 + a, r0 + b,
                     ctypes.c_void_p(y.ctypes.data + 4 * a),
                     ctypes.c_void_p(mag.ctypes.data + 8 * a) if with_mag else None, nr)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, _chunks(nr, threads)))
    return (y, mag) if with_mag else y


def matmul_rows(fmt: str, W: np.ndarray, q: np.ndarray, dx: np.ndarray, row_ids, with_mag: bool = False):
    """y[t, i] for an arbitrary list of rows (sampled parity at full size)."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    T = q.shape[0]
    y = np.empty((T, row_ids.size), dtype=np.float32)
    mag = np.empty((T, row_ids.size), dtype=np.float64)
    for i, r in enumerate(row_ids):
        yi, mi = matmul(fmt, W, q, dx, rows=(int(r), int(r) + 1), with_mag=True)
        y[:, i] = yi[:, 0]
        mag[:, i] = mi[:, 0]
    return (y, mag) if with_mag else y


def group_dots_rows(fmt: str, W: np.ndarray, q: np.ndarray, row_ids) -> np.ndarray:
    """I[t, i, g] for an arbitrary list of rows."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    T = q.shape[0]
    G = W.shape[1]
    out = np.empty((T, row_ids.size, G), dtype=np.int32)
    for i, r in enumerate(row_ids):
        out[:, i, :] = group_dots(fmt, W, q, rows=(int(r), int(r) + 1))[:, 0, :]
    return out
