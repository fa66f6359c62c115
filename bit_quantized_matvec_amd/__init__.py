"""Python binding of libtq: packed-ternary weights x q8_K activations on MI355X.

Argument marshalling only.  Every step of the path (repack, q8_K quantization,
matrix-vector and small-batch matrix products) runs in the HIP kernels of
``libtq.so`` behind the C ABI declared in ``include/tq.h``; PyTorch provides
device memory and the current stream.  There is no CPU fallback: if the
library is not built, importing this package fails.

    import bit_quantized_matvec_amd as tq
    W = tq.repack(w_canonical_cuda, "pq2_0", rows, cols)
    q, d, bs = tq.quantize_q8k(x_cuda)          # x: float32 [tokens, cols]
    y = tq.gemv("pq2_0", W, rows, cols, q, d, bs)
"""
from __future__ import annotations

import ctypes
import os

import torch  # load torch's HIP runtime first: libtq binds to the same libamdhip64

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python bit_quantized_matvec_amd/build.py` first")

_lib = ctypes.CDLL(LIB_PATH)

_p, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGS = {
    "tq_check_shape": ([_i32, _i64, _i64, _i64], _i32),
    "tq_canonical_bytes": ([_i32, _i64, _i64], _i64),
    "tq_repacked_bytes": ([_i32, _i64, _i64], _i64),
    "tq_repack": ([_i32, _p, _p, _i64, _i64, _p, _p], _i32),
    "tq_unrepack": ([_i32, _p, _p, _i64, _i64, _p], _i32),
    "tq_quantize_q8k": ([_p, _i64, _i64, _p, _p, _p, _p], _i32),
    "tq_workspace_bytes": ([_i32, _i64, _i64, _i64], _i64),
    "tq_workspace_clear": ([_p, _i64, _p], _i32),
    "tq_gemv": ([_i32, _p, _i64, _i64, _p, _p, _p, _p, _p, _p], _i32),
    "tq_gemv_f32": ([_i32, _p, _i64, _i64, _p, _p, _p, _p], _i32),
    "tq_gemv_f32_batch": ([_i32, _i32, _p, _p, _i64, _p, _p, _p, _p], _i32),
    "tq_gemv_f32_scratch": ([_i32, _p, _i64, _i64, _p, _p, _p], _i32),
    "tq_gemm": ([_i32, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p], _i32),
    "tq_group_dots": ([_i32, _p, _i64, _i64, _i64, _p, _p, _p, _p], _i32),
    "tq_status_str": ([_i32], ctypes.c_char_p),
    "tq_last_hip_error": ([], _i32),
    "tq_version": ([], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTS = tuple(_SIGS)
FORMATS = {"pq2_0": 1, "ptq1_0": 2}
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_FORMAT, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3, -4, -5, -6


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.tq_status_str(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {_lib.tq_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def lib():
    """The loaded C library (ctypes), for callers that want the raw ABI."""
    return _lib


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt]
    return int(fmt)


def _check(status: int, where: str) -> None:
    if status != OK:
        raise TQError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, numel=None, at_least=False, device=None):
    """Raise ValueError unless `t` is a contiguous GPU tensor of `dtype` holding
    `numel` elements (or at least that many with `at_least`), on `device` if
    given.  Every tensor handed to the C ABI goes through this check first: the
    kernels trust the sizes the host validated, so an undersized or host buffer
    must never reach them."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor of dtype {dtype} "
                         f"(got {t.dtype}, device {t.device}, contiguous={t.is_contiguous()})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the weights on {device}")
    if numel is not None:
        n = t.numel()
        if (n < numel) if at_least else (n != numel):
            want = f"at least {numel}" if at_least else f"{numel}"
            raise ValueError(f"{name} holds {n} elements, needs {want}")
    return t


def _need_w(w, fmt, rows: int, cols: int, name="w"):
    """A repacked weight buffer of exactly tq_repacked_bytes for the shape."""
    n = repacked_bytes(fmt, rows, cols)
    if n <= 0:
        _check(check_shape(fmt, rows, cols) or ERR_SHAPE, name)
    return _need(w, torch.uint8, name, n)


def _need_q8k(q, d, bsums, tokens: int, cols: int, device, need_bsums: bool):
    """q8_K activations of `tokens` tokens: q int8 [T*cols], d fp32 [T*cols/256],
    bsums int16 [T*cols/16] (required for ptq1_0, checked whenever given)."""
    _need(q, torch.int8, "q", tokens * cols, device=device)
    _need(d, torch.float32, "d", tokens * (cols // 256), device=device)
    if bsums is not None or need_bsums:
        if bsums is None:
            raise ValueError("bsums is required for ptq1_0")
        _need(bsums, torch.int16, "bsums", tokens * (cols // 16), device=device)


def _need_ws(ws, fmt, rows: int, cols: int, tokens: int, device):
    if ws is not None:
        _need(ws, torch.uint8, "ws", max(16, workspace_bytes(fmt, rows, cols, tokens)), at_least=True, device=device)


def check_shape(fmt, rows: int, cols: int, tokens: int = 1) -> int:
    return _lib.tq_check_shape(_fmt(fmt), rows, cols, tokens)


def canonical_bytes(fmt, rows: int, cols: int) -> int:
    return _lib.tq_canonical_bytes(_fmt(fmt), rows, cols)


def repacked_bytes(fmt, rows: int, cols: int) -> int:
    return _lib.tq_repacked_bytes(_fmt(fmt), rows, cols)


def _shape(fmt, rows: int, cols: int, tokens: int = 1, where: str = "") -> None:
    """Raise TQError for a shape the selector rejects (before any size arithmetic)."""
    _check(check_shape(fmt, rows, cols, tokens), where or "shape")


def repack(w_canonical: torch.Tensor, fmt, rows: int, cols: int, check_codes: bool = True, out=None) -> torch.Tensor:
    """Canonical weights (uint8 CUDA tensor) -> repacked device layout (uint8).

    With ``check_codes`` (pq2_0) the call waits for the repack and raises if any
    2-bit code is 3, which pq2_0 does not use (load time only)."""
    _shape(fmt, rows, cols, 1, "tq_repack")
    _need(w_canonical, torch.uint8, "w_canonical", canonical_bytes(fmt, rows, cols))
    dev = w_canonical.device
    if out is None:
        out = torch.empty(repacked_bytes(fmt, rows, cols), dtype=torch.uint8, device=dev)
    _need_w(out, fmt, rows, cols, "out")
    flag = torch.zeros(1, dtype=torch.int32, device=dev) if check_codes else None
    _check(_lib.tq_repack(_fmt(fmt), _ptr(w_canonical), _ptr(out), rows, cols, _ptr(flag), _stream()), "tq_repack")
    if check_codes and _fmt(fmt) == FORMATS["pq2_0"] and int(flag.item()) != 0:
        raise ValueError("pq2_0 matrix holds code 3, which is not a pq2_0 value")
    return out


def unrepack(w_repacked: torch.Tensor, fmt, rows: int, cols: int) -> torch.Tensor:
    _shape(fmt, rows, cols, 1, "tq_unrepack")
    _need_w(w_repacked, fmt, rows, cols, "w_repacked")
    out = torch.empty(canonical_bytes(fmt, rows, cols), dtype=torch.uint8, device=w_repacked.device)
    _check(_lib.tq_unrepack(_fmt(fmt), _ptr(w_repacked), _ptr(out), rows, cols, _stream()), "tq_unrepack")
    return out


def quantize_q8k(x: torch.Tensor, out=None):
    """float32 [tokens, cols] -> (q int8 [T, cols], d float32 [T, cols/256], bsums int16 [T, cols/16])."""
    _need(x, torch.float32, "x")
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dim() != 2:
        raise ValueError("x must be [cols] or [tokens, cols]")
    T, K = x.shape
    _shape("pq2_0", 1, K, T, "tq_quantize_q8k")
    if out is None:
        q = torch.empty((T, K), dtype=torch.int8, device=x.device)
        d = torch.empty((T, K // 256), dtype=torch.float32, device=x.device)
        bs = torch.empty((T, K // 16), dtype=torch.int16, device=x.device)
    else:
        q, d, bs = out
        _need_q8k(q, d, bs, T, K, x.device, True)
    _check(_lib.tq_quantize_q8k(_ptr(x), T, K, _ptr(q), _ptr(d), _ptr(bs), _stream()), "tq_quantize_q8k")
    return q, d, bs


def workspace_bytes(fmt, rows: int, cols: int, tokens: int = 1) -> int:
    return _lib.tq_workspace_bytes(_fmt(fmt), rows, cols, tokens)


def workspace(fmt, rows: int, cols: int, tokens: int = 1, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for tq_gemv / tq_gemm of this shape (reusable)."""
    return torch.zeros(max(16, workspace_bytes(fmt, rows, cols, tokens)), dtype=torch.uint8, device=device)


def workspace_clear(ws: torch.Tensor) -> torch.Tensor:
    """Zero a workspace with a kernel on the current stream (no memset node, so
    it may be captured in a graph): restores a workspace whose state is not
    known, e.g. one shared by calls that overlapped."""
    _need(ws, torch.uint8, "ws")
    _check(_lib.tq_workspace_clear(_ptr(ws), ws.numel(), _stream()), "tq_workspace_clear")
    return ws


def _tokens(q) -> int:
    return q.shape[0] if q.dim() == 2 else 1


def gemv(fmt, w: torch.Tensor, rows: int, cols: int, q, d, bsums=None, out=None, ws=None) -> torch.Tensor:
    """y[rows] = W x for one q8_K token (q [cols] or [1, cols]); ws: optional workspace."""
    _shape(fmt, rows, cols, 1, "tq_gemv")
    _need_w(w, fmt, rows, cols)
    _need_q8k(q, d, bsums, 1, cols, w.device, _fmt(fmt) == FORMATS["ptq1_0"])
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=w.device)
    _need(out, torch.float32, "out", rows, device=w.device)
    _need_ws(ws, fmt, rows, cols, 1, w.device)
    _check(_lib.tq_gemv(_fmt(fmt), _ptr(w), rows, cols, _ptr(q), _ptr(d), _ptr(bsums), _ptr(out), _ptr(ws),
                        _stream()), "tq_gemv")
    return out


def gemv_f32(fmt, w: torch.Tensor, rows: int, cols: int, x: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """y[rows] = W q8_K(x) for one fp32 token x [cols] or [1, cols], quantized
    inside the product kernel (bit-identical to quantize_q8k followed by gemv)."""
    _shape(fmt, rows, cols, 1, "tq_gemv_f32")
    _need_w(w, fmt, rows, cols)
    _need(x, torch.float32, "x", cols, device=w.device)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=w.device)
    _need(out, torch.float32, "out", rows, device=w.device)
    _need_ws(ws, fmt, rows, cols, 1, w.device)
    _check(_lib.tq_gemv_f32(_fmt(fmt), _ptr(w), rows, cols, _ptr(x), _ptr(out), _ptr(ws), _stream()), "tq_gemv_f32")
    return out


def gemv_f32_scratch(fmt, w: torch.Tensor, rows: int, cols: int, x: torch.Tensor, out=None) -> torch.Tensor:
    """gemv_f32 with the column split's workspace in the library's static
    device scratch (no workspace argument, nothing allocated by the call
    itself when `out` is given).  Calls that overlap on one GPU race."""
    _shape(fmt, rows, cols, 1, "tq_gemv_f32_scratch")
    _need_w(w, fmt, rows, cols)
    _need(x, torch.float32, "x", cols, device=w.device)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=w.device)
    _need(out, torch.float32, "out", rows, device=w.device)
    _check(_lib.tq_gemv_f32_scratch(_fmt(fmt), _ptr(w), rows, cols, _ptr(x), _ptr(out), _stream()),
           "tq_gemv_f32_scratch")
    return out


def gemv_f32_batch(fmt, ws_list, rows, cols: int, xs, outs=None, ws=None):
    """Independent gemv_f32 products sharing `cols`, in one launch: problem m
    multiplies ws_list[m] (rows[m] x cols) by xs[m]; returns the outputs."""
    n = len(ws_list)
    if not (len(rows) == len(xs) == n) or (outs is not None and len(outs) != n):
        raise TQError(ERR_SHAPE, "gemv_f32_batch: list lengths differ")
    if not 1 <= n <= 4:
        raise TQError(ERR_SHAPE, "gemv_f32_batch: 1 to 4 problems")
    dev = ws_list[0].device if isinstance(ws_list[0], torch.Tensor) else None
    for m in range(n):
        _shape(fmt, rows[m], cols, 1, "tq_gemv_f32_batch")
        _need_w(ws_list[m], fmt, rows[m], cols, f"w[{m}]")
        _need(xs[m], torch.float32, f"x[{m}]", cols, device=dev)
    if outs is None:
        outs = [torch.empty(r, dtype=torch.float32, device=dev) for r in rows]
    for m in range(n):
        _need(outs[m], torch.float32, f"out[{m}]", rows[m], device=dev)
    if ws is not None:
        tiled = sum(-(-r // 64) * 64 for r in rows)
        _need_ws(ws, fmt, tiled, cols, 1, dev)
    P = ctypes.c_void_p * n
    wp = P(*[t.data_ptr() for t in ws_list])
    xp = P(*[t.data_ptr() for t in xs])
    yp = P(*[t.data_ptr() for t in outs])
    rp = (ctypes.c_int64 * n)(*rows)
    _check(_lib.tq_gemv_f32_batch(_fmt(fmt), n, wp, rp, cols, xp, yp, _ptr(ws), _stream()), "tq_gemv_f32_batch")
    return outs


def gemm(fmt, w: torch.Tensor, rows: int, cols: int, q, d, bsums=None, out=None, ws=None) -> torch.Tensor:
    """y[tokens, rows] for q8_K activations q [tokens, cols]; ws: optional workspace."""
    T = _tokens(q)
    _shape(fmt, rows, cols, T, "tq_gemm")
    _need_w(w, fmt, rows, cols)
    _need_q8k(q, d, bsums, T, cols, w.device, _fmt(fmt) == FORMATS["ptq1_0"])
    if out is None:
        out = torch.empty((T, rows), dtype=torch.float32, device=w.device)
    _need(out, torch.float32, "out", T * rows, device=w.device)
    _need_ws(ws, fmt, rows, cols, T, w.device)
    _check(_lib.tq_gemm(_fmt(fmt), _ptr(w), rows, cols, T, _ptr(q), _ptr(d), _ptr(bsums), _ptr(out), _ptr(ws),
                        _stream()), "tq_gemm")
    return out


def group_dots(fmt, w: torch.Tensor, rows: int, cols: int, q, bsums=None) -> torch.Tensor:
    """Exact int32 group dots [tokens, rows, cols/128] from the product kernels."""
    T = _tokens(q)
    _shape(fmt, rows, cols, T, "tq_group_dots")
    _need_w(w, fmt, rows, cols)
    _need(q, torch.int8, "q", T * cols, device=w.device)
    if bsums is not None or _fmt(fmt) == FORMATS["ptq1_0"]:
        if bsums is None:
            raise ValueError("bsums is required for ptq1_0")
        _need(bsums, torch.int16, "bsums", T * (cols // 16), device=w.device)
    out = torch.empty((T, rows, cols // 128), dtype=torch.int32, device=w.device)
    _check(_lib.tq_group_dots(_fmt(fmt), _ptr(w), rows, cols, T, _ptr(q), _ptr(bsums), _ptr(out), _stream()),
           "tq_group_dots")
    return out


class TernaryMatrix:
    """A repacked weight matrix resident on the GPU, with its shape and format."""

    def __init__(self, w_canonical: torch.Tensor, fmt: str, rows: int, cols: int):
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.data = repack(w_canonical, fmt, rows, cols)
        self.ws = workspace(fmt, rows, cols, device=w_canonical.device)

    def matvec(self, q, d, bsums=None, out=None):
        return gemv(self.fmt, self.data, self.rows, self.cols, q, d, bsums, out, self.ws)

    def matmul(self, q, d, bsums=None, out=None):
        return gemm(self.fmt, self.data, self.rows, self.cols, q, d, bsums, out, self.ws)

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        """fp32 activations [tokens, cols] -> fp32 [tokens, rows] (quantize, then product)."""
        q, d, bs = quantize_q8k(x)
        return self.matmul(q, d, bs)
