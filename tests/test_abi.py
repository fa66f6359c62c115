"""The C-ABI library loads, exports every declared symbol, and validates its
arguments on the host.  No kernel is launched here: every call below fails
validation before any HIP work (so these run on a CPU-only machine)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    import bit_quantized_matvec_amd as m

    return m


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(tq):
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(tq.lib(), n), n
    assert set(names) == set(tq.EXPORTS)
    assert tq.lib().tq_version() >= 100


def test_sizes(tq):
    # 34 and 28 bytes per 128 weights; repacked = canonical when rows % 64 == 0 and, for ptq1_0, groups % 8 == 0
    assert tq.canonical_bytes("pq2_0", 32768, 8192) == 71303168
    assert tq.repacked_bytes("pq2_0", 32768, 8192) == 71303168
    assert tq.canonical_bytes("ptq1_0", 32768, 8192) == 58720256
    assert tq.repacked_bytes("ptq1_0", 32768, 8192) == 58720256
    assert tq.canonical_bytes("pq2_0", 17408, 5120) == 23674880
    assert tq.repacked_bytes("pq2_0", 17408, 5120) == 23674880
    # padding of the row tile (rows -> multiple of 64) and of ptq1_0 groups (-> multiple of 8)
    assert tq.repacked_bytes("pq2_0", 1, 256) == 64 * 256 / 4 + 64 * 4  # codes + one scale pair per row and superchunk
    assert tq.repacked_bytes("ptq1_0", 65, 256) == 2 * 8 * 64 * 28
    assert tq.canonical_bytes("pq2_0", 0, 256) == 0
    assert tq.repacked_bytes(7, 64, 256) == 0


@pytest.mark.parametrize(
    "fmt,rows,cols,tokens,expect",
    [
        (1, 64, 256, 1, 0),
        (2, 5, 768, 3, 0),
        (1, 0, 256, 1, -2),
        (1, 64, 128, 1, -2),
        (1, 64, 384, 1, -2),
        (1, 64, 0, 1, -2),
        (1, 64, 256, 0, -2),
        (1, -3, 256, 1, -2),
        (1, 1 << 27, 256, 1, -2),
        (2, 64, 32768 + 256, 1, -2),
        (2, 64, 32768, 1, 0),
        (1, 64, 65536 + 256, 1, 0),
        (0, 64, 256, 1, -4),
        (3, 64, 256, 1, -4),
    ],
)
def test_selector(tq, fmt, rows, cols, tokens, expect):
    assert tq.check_shape(fmt, rows, cols, tokens) == expect


def test_validation_errors_touch_nothing(tq):
    L = tq.lib()
    P = ctypes.c_void_p
    good = P(0x100000)  # never dereferenced: each call below fails validation first
    odd = P(0x100001)
    # null pointers
    assert L.tq_gemv(1, None, 64, 256, good, good, None, good, None, None) == tq.ERR_NULL
    assert L.tq_gemv(1, good, 64, 256, good, None, None, good, None, None) == tq.ERR_NULL
    assert L.tq_gemv(2, good, 64, 256, good, good, None, good, None, None) == tq.ERR_NULL  # ptq1_0 needs bsums
    assert L.tq_gemm(1, good, 64, 256, 4, None, good, None, good, None, None) == tq.ERR_NULL
    assert L.tq_quantize_q8k(None, 1, 256, good, good, good, None) == tq.ERR_NULL
    assert L.tq_repack(1, None, good, 64, 256, None, None) == tq.ERR_NULL
    assert L.tq_group_dots(1, good, 64, 256, 1, good, None, None, None) == tq.ERR_NULL
    # alignment
    assert L.tq_gemv(1, odd, 64, 256, good, good, None, good, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv(1, good, 64, 256, odd, good, None, good, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv(1, good, 64, 256, good, odd, None, good, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv(1, good, 64, 256, good, good, None, P(0x100002), None, None) == tq.ERR_ALIGN
    assert L.tq_gemv(2, good, 64, 256, good, good, odd, good, None, None) == tq.ERR_ALIGN
    assert L.tq_quantize_q8k(P(0x100004), 1, 256, good, good, good, None) == tq.ERR_ALIGN
    assert L.tq_repack(1, good, P(0x100008), 64, 256, None, None) == tq.ERR_ALIGN
    # shapes and formats
    assert L.tq_gemv(1, good, 64, 200, good, good, None, good, None, None) == tq.ERR_SHAPE
    assert L.tq_gemm(1, good, 64, 256, 0, good, good, None, good, None, None) == tq.ERR_SHAPE
    assert L.tq_quantize_q8k(good, 1, 100, good, good, good, None) == tq.ERR_SHAPE
    assert L.tq_gemv(9, good, 64, 256, good, good, None, good, None, None) == tq.ERR_FORMAT
    assert L.tq_unrepack(9, good, good, 64, 256, None) == tq.ERR_FORMAT
    assert L.tq_gemv(1, good, 64, 256, good, good, None, good, P(0x100008), None) == tq.ERR_ALIGN  # workspace
    assert L.tq_workspace_bytes(1, 64, 200, 1) == 0 and L.tq_workspace_bytes(1, 640, 8192, 1) > 0
    assert L.tq_workspace_clear(None, 64, None) == tq.ERR_NULL
    assert L.tq_workspace_clear(P(0x100008), 64, None) == tq.ERR_ALIGN
    assert L.tq_workspace_clear(good, -1, None) == tq.ERR_SHAPE
    assert L.tq_workspace_clear(None, 0, None) == tq.OK  # nothing to clear, nothing launched
    assert L.tq_last_hip_error() == 0


def _fused_fits(rows, cols, ws):
    """The on-chip rule of tq_gemv_f32 as its declaration states it."""
    n, tiles = cols // 256, -(-rows // 64)
    s = 1
    if ws and tiles < 384:
        most = min(16, max(1, n // 4))
        while s < most and (-(-n // s) > 12 or tiles * s < 224):
            s += 1
    return -(-n // s) <= 126


def test_fused_gemv_validation(tq):
    L = tq.lib()
    P = ctypes.c_void_p
    good, odd = P(0x100000), P(0x100004)
    assert L.tq_gemv_f32(1, None, 64, 256, good, good, None, None) == tq.ERR_NULL
    assert L.tq_gemv_f32(1, good, 64, 256, None, good, None, None) == tq.ERR_NULL
    assert L.tq_gemv_f32(1, good, 64, 256, good, None, None, None) == tq.ERR_NULL
    assert L.tq_gemv_f32(1, P(0x100008), 64, 256, good, good, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv_f32(1, good, 64, 256, odd, good, None, None) == tq.ERR_ALIGN  # x needs 16 bytes
    assert L.tq_gemv_f32(1, good, 64, 256, good, P(0x100002), None, None) == tq.ERR_ALIGN
    assert L.tq_gemv_f32(1, good, 64, 256, good, good, P(0x100008), None) == tq.ERR_ALIGN
    assert L.tq_gemv_f32(1, good, 64, 200, good, good, None, None) == tq.ERR_SHAPE
    assert L.tq_gemv_f32(9, good, 64, 256, good, good, None, None) == tq.ERR_FORMAT
    assert L.tq_gemv_f32(2, good, 64, 256, None, good, None, None) == tq.ERR_UNSUPPORTED  # ptq1_0
    # the on-chip limit, both sides of it; it is checked before the pointers,
    # so the null x below is reached only by shapes that fit
    for rows, cols, ws in [(64, 32256, None), (64, 32512, None), (24576, 65536, good),
                           (24512, 65536, good), (64, 65536, good), (64, 262144, good), (64, 1 << 20, good)]:
        want = tq.ERR_NULL if _fused_fits(rows, cols, ws) else tq.ERR_UNSUPPORTED
        assert L.tq_gemv_f32(1, good, rows, cols, None, good, ws, None) == want, (rows, cols)
    assert not _fused_fits(64, 32512, None) and _fused_fits(64, 65536, P(1)) and not _fused_fits(24576, 65536, P(1))
    assert L.tq_last_hip_error() == 0


def test_fused_batch_validation(tq):
    L = tq.lib()
    P = ctypes.c_void_p
    good, odd = P(0x100000), P(0x100004)
    A = lambda *v: (ctypes.c_void_p * len(v))(*v)
    R = lambda *v: (ctypes.c_int64 * len(v))(*v)
    w2, x2, y2, r2 = A(good, good), A(good, good), A(good, good), R(64, 128)
    assert L.tq_gemv_f32_batch(1, 0, w2, r2, 256, x2, y2, None, None) == tq.ERR_SHAPE
    assert L.tq_gemv_f32_batch(1, 5, w2, r2, 256, x2, y2, None, None) == tq.ERR_SHAPE
    assert L.tq_gemv_f32_batch(9, 2, w2, r2, 256, x2, y2, None, None) == tq.ERR_FORMAT
    assert L.tq_gemv_f32_batch(1, 2, None, r2, 256, x2, y2, None, None) == tq.ERR_NULL
    assert L.tq_gemv_f32_batch(1, 2, w2, None, 256, x2, y2, None, None) == tq.ERR_NULL
    assert L.tq_gemv_f32_batch(1, 2, w2, R(64, 0), 256, x2, y2, None, None) == tq.ERR_SHAPE
    assert L.tq_gemv_f32_batch(1, 2, w2, r2, 200, x2, y2, None, None) == tq.ERR_SHAPE
    assert L.tq_gemv_f32_batch(2, 2, w2, r2, 256, x2, y2, None, None) == tq.ERR_UNSUPPORTED  # ptq1_0
    # the on-chip rule on the total row tiles, before the per-problem pointers
    assert L.tq_gemv_f32_batch(1, 2, A(None, None), R(64, 64), 32512, x2, y2, None, None) == tq.ERR_UNSUPPORTED
    assert L.tq_gemv_f32_batch(1, 2, A(good, None), R(64, 64), 256, x2, y2, None, None) == tq.ERR_NULL
    assert L.tq_gemv_f32_batch(1, 2, w2, r2, 256, A(good, odd), y2, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv_f32_batch(1, 2, A(good, P(0x100008)), r2, 256, x2, y2, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv_f32_batch(1, 2, w2, r2, 256, x2, y2, P(0x100008), None) == tq.ERR_ALIGN
    assert L.tq_last_hip_error() == 0


def test_status_strings(tq):
    L = tq.lib()
    for s in (0, -1, -2, -3, -4, -5, -6, -99):
        assert len(L.tq_status_str(s)) > 0
    with pytest.raises(tq.TQError) as e:
        tq._check(tq.ERR_SHAPE, "x")
    assert e.value.status == tq.ERR_SHAPE


def test_no_cpu_fallback_in_binding():
    """The binding never imports the oracle and has no CPU compute path."""
    src = open(os.path.join(ROOT, "bit_quantized_matvec_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no CPU fallback", "")
    for f in os.listdir(os.path.join(ROOT, "bit_quantized_matvec_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "bit_quantized_matvec_amd", "csrc", f)).read().lower()


def test_probe_library_validates_on_host(tq):
    """The measurement library beside the product (libtq_probe.so: the read
    ceiling, the decode-pattern read and the clock) loads and refuses bad
    arguments before any HIP work (hipErrorInvalidValue = 1)."""
    path = os.path.join(ROOT, "bit_quantized_matvec_amd", "libtq_probe.so")
    if not os.path.exists(path):
        pytest.skip("libtq_probe.so is not built")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.tqp_read.argtypes = [P, I64, I, I, I, P, P]
    lib.tqp_read_units.argtypes = [P, I, I, P, P]
    lib.tqp_clock.argtypes = [P, I, I, P, I64, P]
    fake = ctypes.c_void_p(16)
    assert lib.tqp_read(None, 1024, 8, 64, 1, fake, None) == 1
    assert lib.tqp_read(fake, 1000, 8, 64, 1, fake, None) == 1  # not a multiple of 16
    assert lib.tqp_read(fake, 1024, 8, 48, 1, fake, None) == 1  # threads not a multiple of 64
    assert lib.tqp_read_units(None, 512, 32, fake, None) == 1
    assert lib.tqp_read_units(fake, 512, 12, fake, None) == 1   # runs of 3: not a multiple of 8 units
    assert lib.tqp_read_units(fake, 0, 32, fake, None) == 1
    assert lib.tqp_clock(None, 8, 10, None, 0, None) == 1
