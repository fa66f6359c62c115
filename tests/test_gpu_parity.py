"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer results (q8_K fields, group dots, repacked bytes) must be bit-exact.
Float outputs must satisfy, per output element (tolerance from the workload
definition, 1e-5 relative per row):
    |y_gpu - y_ref| <= 1e-5 * |y_ref|,   or, if y_ref == 0,
    |y_gpu|         <= 1e-5 * sum_g |term_g|.
Both sides evaluate the float epilogue in fp64 with exact terms, so in practice
the outputs agree to the last bit; the tests also report how many do.
"""
import os
import sys

import numpy as np
import pytest

import tq_inputs as TI

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def tq():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_matvec_amd as m

    return m


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close_rows(y, ref, mag, rtol=1e-5, what=""):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(y - ref)
    bound = np.where(ref != 0, rtol * np.abs(ref), rtol * mag)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outputs outside tolerance; worst rel {np.max(err / np.maximum(np.abs(ref), 1e-300))}"
    return int(np.sum(y == ref))


def counters_clear(tq, ws, tiles):
    """True when the arrival counters of the first `tiles` tiles are zero: each
    tile's workspace block (the size of a one-tile workspace) starts with it."""
    import torch

    per = tq.workspace_bytes("pq2_0", 64, 256)
    idx = torch.arange(tiles, device=ws.device) * per
    words = torch.stack([ws[idx + k] for k in range(4)])
    return int(torch.count_nonzero(words)) == 0


def gpu_pipeline(tq, fmt, W, x):
    """Repack, quantize and multiply on the GPU; returns numpy results."""
    R, G, _ = W.shape
    K = G * 128
    T = x.shape[0]
    Wd = tq.repack(dev(W.reshape(-1)), fmt, R, K)
    q, d, bs = tq.quantize_q8k(dev(x))
    y = tq.gemm(fmt, Wd, R, K, q, d, bs) if T > 1 else tq.gemv(fmt, Wd, R, K, q, d, bs).view(1, R)
    I = tq.group_dots(fmt, Wd, R, K, q, bs)
    return Wd, host(q), host(d), host(bs), host(y).reshape(T, R), host(I)


# --------------------------------------------------------------------------- q8_K


def quant_cases():
    g = TI.rng(77, 1)
    yield "normal", TI.activations(g, 5, 8192)
    yield "heavy_tails", (g.standard_t(2, size=(3, 2048)) * 10).astype(np.float32)
    yield "subnormal", (g.standard_normal((2, 1024)) * 1e-40).astype(np.float32)
    yield "tiny", (g.standard_normal((1, 512)) * 1e-44).astype(np.float32)
    yield "huge", (g.uniform(-1, 1, size=(1, 512)) * 3e38).astype(np.float32)
    x = np.zeros((2, 768), np.float32)
    x[1, 300] = -2.5
    x[1, 512:] = 7.0
    yield "zeros_and_constants", x
    rows = [l.split() for l in open(os.path.join(os.path.dirname(__file__), "golden", "q8k_ties.txt")) if l.strip() and not l.startswith("#")]
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = 254
    for i, (xv, _) in enumerate(rows[1:], start=1):
        x[0, i] = float(xv)
    yield "ties", x
    yield "odd_tokens", TI.activations(g, 7, 256)
    # values within a few ulps of half-integer multiples of the block scale
    # (the quantizer's reciprocal fast path must hand these to the exact path)
    x = np.zeros((6, 256), np.float32)
    for t in range(6):
        amax = np.float32(g.uniform(0.5, 300.0))
        d = np.float32(amax / np.float32(127.0))
        k = g.integers(-126, 126, size=255).astype(np.float32)
        near = ((k + np.float32(0.5)) * d).astype(np.float32)
        steps = g.integers(-3, 4, size=255)
        x[t, 0] = amax
        x[t, 1:] = np.nextafter(near, np.where(steps > 0, np.inf, -np.inf).astype(np.float32)).astype(np.float32)
        x[t, 1:] = np.where(steps == 0, near, x[t, 1:])
    yield "near_half_integers", x


@pytest.mark.parametrize("case", [c for c, _ in quant_cases()])
def test_quantize_q8k_bit_exact(tq, orc, case):
    x = dict(quant_cases())[case]
    say("quantize", case, x.shape)
    q, d, bs = tq.quantize_q8k(dev(x))
    qo, do, bso = orc.quantize_q8k(x)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(d).view(np.uint32), do.view(np.uint32))
    assert np.array_equal(host(bs), bso)


# ------------------------------------------------------------------------- repack


@pytest.mark.parametrize("fmt,R,K", [("pq2_0", 1, 256), ("pq2_0", 65, 768), ("pq2_0", 200, 2560),
                                     ("ptq1_0", 1, 256), ("ptq1_0", 65, 768), ("ptq1_0", 130, 2304)])
def test_repack_roundtrip(tq, fmt, R, K):
    say("repack", fmt, R, K)
    g = TI.rng(77, 2, R, K)
    W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else g.integers(0, 256, size=(R, K // 128, 28), dtype=np.uint8)
    Wd = tq.repack(dev(W.reshape(-1)), fmt, R, K)
    assert Wd.numel() == tq.repacked_bytes(fmt, R, K)
    back = tq.unrepack(Wd, fmt, R, K)
    assert np.array_equal(host(back), W.reshape(-1))


def test_repack_flags_code_3(tq):
    g = TI.rng(77, 3)
    W = TI.pq2_matrix(g, 70, 512)
    tq.repack(dev(W.reshape(-1)), "pq2_0", 70, 512)  # valid: no error
    W[69, 3, 2 + 17] |= 0x30  # field 2 of one byte -> code 3
    with pytest.raises(ValueError):
        tq.repack(dev(W.reshape(-1)), "pq2_0", 70, 512)


def integer_activations(g, T, K):
    """Integer activations in [-127, 127] with |x| = 127 at a random place of
    every 256-block, so that q8_K reproduces them exactly (d = 1, q = x): the
    pages' integer-oracle inputs, with amax forced in every block, not just
    the first (page 1, "what didn't work": the first run failed for that)."""
    x = g.integers(-127, 128, size=(T, K)).astype(np.float32)
    for t in range(T):
        for b in range(K // 256):
            x[t, 256 * b + int(g.integers(0, 256))] = 127.0 if g.integers(0, 2) else -127.0
    return x


def check_integer_case(tq, orc, fmt, W, x, what):
    """q8_K of x is x itself; the integer group dots equal a plain int64 numpy
    product of the decoded weights and x; y is within R15 of the fp64 sum of
    d_w * I (d_x = 1)."""
    R, G, _ = W.shape
    K = G * 128
    T = x.shape[0]
    Wd, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
    assert np.array_equal(q, x.astype(np.int8)) and np.all(d == 1.0), what
    assert np.array_equal(bs, x.reshape(T, K // 16, 16).sum(axis=2).astype(np.int16)), what
    w, dw, _ = orc.decode(fmt, W)
    Iref = np.einsum("rgk,tgk->trg", w.astype(np.int64).reshape(R, G, 128), x.astype(np.int64).reshape(T, G, 128))
    assert np.array_equal(I, Iref), what
    terms = dw.astype(np.float64)[None, :, :] * Iref
    yref = terms.sum(axis=2)
    assert_close_rows(y, yref, np.abs(terms).sum(axis=2), what=what)


@pytest.mark.parametrize("fmt", ["pq2_0", "ptq1_0"])
def test_integer_grid(tq, orc, fmt):
    """The pages' integer-oracle grid (page 1, "did i break the model?": batch
    widths 1-5, 7, 8; rows 4, 8, 12; inner sizes 256, 512, 1024), 63 shapes per
    format, plus extremes: every activation +-127 against all-+1 and all--1
    weights (|I| = 128 * 127, the largest group dot) and all-zero weights."""
    g = TI.rng(77, 19, 1 if fmt == "pq2_0" else 2)
    n = 0
    for T in (1, 2, 3, 4, 5, 7, 8):
        for R in (4, 8, 12):
            for K in (256, 512, 1024):
                W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
                check_integer_case(tq, orc, fmt, W, integer_activations(g, T, K), f"{fmt} T={T} R={R} K={K}")
                n += 1
    R, K, T = 12, 1024, 5
    sc = TI.scales_f16(g, R, K)
    ones = 0xAA if fmt == "pq2_0" else 255  # every weight +1 (code 2 / trits 2,2,2,2,2)
    negs = 0x00  # every weight -1 (code 0 / trits 0)
    for byte, sign in ((ones, 1.0), (negs, 1.0), (ones, -1.0), (negs, -1.0)):
        codes = np.full((R, K // 128, 32 if fmt == "pq2_0" else 26), byte, np.uint8)
        W = TI.assemble_pq2(codes, sc) if fmt == "pq2_0" else TI.assemble_ptq1(codes, sc)
        x = np.full((T, K), 127.0 * sign, np.float32)
        check_integer_case(tq, orc, fmt, W, x, f"{fmt} extreme byte={byte} sign={sign}")
        n += 1
    zero = 0x55 if fmt == "pq2_0" else 0x80  # every weight 0 (code 1 / trits 1: 128 * 3^j = 128 mod 256)
    codes = np.full((R, K // 128, 32 if fmt == "pq2_0" else 26), zero, np.uint8)
    W = TI.assemble_pq2(codes, sc) if fmt == "pq2_0" else TI.assemble_ptq1(codes, sc)
    w, _, _ = orc.decode(fmt, W)
    assert not w.any()
    check_integer_case(tq, orc, fmt, W, integer_activations(g, T, K), f"{fmt} zero weights")
    say(f"integer grid {fmt}: {n + 1} cases")


def test_one_hot_probes(tq, orc):
    """A single non-zero weight times a one-hot activation locates every
    (row, column) mapping of the repacked layout, for both formats."""
    R, K = 67, 512
    g = TI.rng(77, 4)
    for fmt in ("pq2_0", "ptq1_0"):
        cols = g.choice(K, size=24, replace=False)
        rows = g.integers(0, R, size=24)
        for r, c in zip(rows, cols):
            if fmt == "pq2_0":
                codes = np.full((R, K // 128, 32), 0x55, np.uint8)  # w = 0
                k = c % 128
                codes[r, c // 128, k >> 2] = (0x55 & ~(3 << (2 * (k & 3)))) | (2 << (2 * (k & 3)))  # w = +1
                W = TI.assemble_pq2(codes, np.ones((R, K // 128), np.float16))
            else:
                zero = -(-256 * 121 // 243)  # encodes n = 121 = 11111 in base 3: every trit 1, every w 0
                W = TI.assemble_ptq1(np.full((R, K // 128, 26), zero, np.uint8), np.ones((R, K // 128), np.float16))
                k = c % 128
                digits = [1] * 5
                digits[k % 5] = 2  # w = +1 at trit k % 5
                n = sum(dg * 3 ** (4 - j) for j, dg in enumerate(digits))
                W[r, c // 128, 2 + k // 5] = -(-256 * n // 243)
            x = np.zeros((1, K), np.float32)
            x[0, c] = 1.0
            _, _, _, y, I, = gpu_pipeline(tq, fmt, W, x)[1:]
            yo = orc.matmul(fmt, W, *orc.quantize_q8k(x)[:2])
            assert np.array_equal(y, yo), (fmt, r, c)
            nz = np.argwhere(y[0] != 0).ravel().tolist()
            assert nz == [r], (fmt, r, c, nz)
            assert I[0, r, c // 128] == 127


# ------------------------------------------------------------------ GEMV / GEMM grid


GRID_R = [1, 4, 5, 12, 33, 64, 65, 200]
GRID_K = [256, 512, 1024, 1280, 2304, 8192]


@pytest.mark.parametrize("fmt", ["pq2_0", "ptq1_0"])
def test_gemv_grid(tq, orc, fmt):
    g = TI.rng(77, 5, 1 if fmt == "pq2_0" else 2)
    exact = total = 0
    for K in GRID_K:
        for R in GRID_R:
            say("gemv", fmt, R, K)
            W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
            x = TI.activations(g, 1, K)
            _, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
            qo, do, bso = orc.quantize_q8k(x)
            assert np.array_equal(q, qo) and np.array_equal(d, do) and np.array_equal(bs, bso)
            assert np.array_equal(I, orc.group_dots(fmt, W, qo)), (fmt, R, K)
            yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
            exact += assert_close_rows(y, yo, mag, what=f"{fmt} {R}x{K}")
            total += y.size
    say(f"gemv {fmt}: {exact}/{total} outputs bit-identical to the oracle")


GEMM_T = [2, 3, 4, 5, 7, 8, 16, 17, 33, 64, 65, 100]


@pytest.mark.parametrize("fmt", ["pq2_0", "ptq1_0"])
@pytest.mark.parametrize("R,K", [(1, 256), (33, 1280), (64, 2048), (130, 512)])
def test_gemm_grid(tq, orc, fmt, R, K):
    g = TI.rng(77, 6, R, K) if fmt == "pq2_0" else TI.rng(77, 16, R, K)
    W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
    exact = total = 0
    for T in GEMM_T:
        say("gemm", fmt, R, K, T)
        x = TI.activations(g, T, K)
        Wd, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
        qo, do, _ = orc.quantize_q8k(x)
        assert np.array_equal(q, qo) and np.array_equal(d, do)
        assert np.array_equal(I, orc.group_dots(fmt, W, qo)), (R, K, T)
        yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
        exact += assert_close_rows(y, yo, mag, what=f"gemm {fmt} {R}x{K} T={T}")
        total += y.size
        # one matrix-vector product per token gives the same outputs
        qd, dd, bd = tq.quantize_q8k(dev(x))
        for t in (0, T - 1):
            yv = host(tq.gemv(fmt, Wd, R, K, qd[t], dd[t], bd[t]))
            assert_close_rows(yv, yo[t], mag[t], what=f"gemv token {t}")
    say(f"gemm {fmt} {R}x{K}: {exact}/{total} outputs bit-identical to the oracle")


@pytest.mark.parametrize("fmt", ["pq2_0", "ptq1_0"])
@pytest.mark.parametrize("R,K", [(64, 256), (130, 1280), (200, 2048), (65, 3328), (17408, 5120)])
def test_gemm_equals_stacked_gemv(tq, fmt, R, K):
    """A prompt product of T tokens gives, bit for bit, the outputs of T
    matrix-vector products without a workspace.  pq2_0: both round each group
    pair's inner sum once and sum the superchunks in the same runs and run
    order; the column counts give runs of 1, 2, 2, 4 and 5 superchunks with
    ragged last runs, and the token counts every result-slot layout of the
    one-block kernel (1-4, 5-8 and 9-16 tokens), two and three 16-token
    groups (17, 40) and one and two 32-token groups (50, 64), the last group
    part empty.  ptq1_0: every token of a block takes the one-token
    kernel's steps (blocks of 1, 2 or 4 tokens, the last one padded).
    A workspace changes nothing (twice in a row, arrival counters at zero).
    17408x5120 is the prefill shape."""
    import torch

    g = TI.rng(77, 15, R, K)
    W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
    Wd = tq.repack(dev(W.reshape(-1)), fmt, R, K)
    for T in (1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 40, 50, 64):
        say("gemm vs gemv", fmt, R, K, T)
        x = TI.activations(g, T, K)
        q, d, bs = tq.quantize_q8k(dev(x))
        y = host(tq.gemm(fmt, Wd, R, K, q, d, bs))
        yv = np.stack([host(tq.gemv(fmt, Wd, R, K, q[t], d[t], bs[t])) for t in range(T)])
        assert np.array_equal(y, yv), (R, K, T, int(np.sum(y != yv)))
        # with a workspace
        ws = tq.workspace(fmt, R, K, T)
        for _ in range(2):
            yw = host(tq.gemm(fmt, Wd, R, K, q, d, bs, ws=ws))
            assert np.array_equal(yw, y), (R, K, T, "workspace", int(np.sum(yw != y)))
            assert counters_clear(tq, ws, -(-R // 64))
        if T <= 8 and fmt == "pq2_0":
            yf = np.stack([host(tq.gemv_f32("pq2_0", Wd, R, K, dev(x[t]))) for t in range(T)])
            assert np.array_equal(y, yf), (R, K, T, "fused")
    del Wd
    torch.cuda.empty_cache()


WS_SHAPES = [(1, 256), (5, 1024), (64, 2048), (65, 4096), (200, 8192), (1000, 1280), (3, 16384)]


@pytest.mark.parametrize("fmt", ["pq2_0", "ptq1_0"])
def test_gemv_workspace_split(tq, orc, fmt):
    """With a workspace, tiles below the split threshold spread their columns
    over several workgroups; every output still matches the oracle, the
    arrival counters are back at zero after each call, and a second call
    gives the same bits, also after a call of another shape in between that
    shares the workspace.  ptq1_0 sums in one order whatever the split, so
    its outputs equal those without a workspace."""
    import torch

    g = TI.rng(77, 12, 1 if fmt == "pq2_0" else 2)
    ws = tq.workspace(fmt, max(r for r, _ in WS_SHAPES), max(k for _, k in WS_SHAPES))
    prev = None
    for R, K in WS_SHAPES:
        say("gemv workspace", fmt, R, K)
        W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
        x = TI.activations(g, 1, K)
        Wd = tq.repack(dev(W.reshape(-1)), fmt, R, K)
        q, d, bs = tq.quantize_q8k(dev(x))
        assert tq.workspace_bytes(fmt, R, K) <= ws.numel()
        y1 = host(tq.gemv(fmt, Wd, R, K, q, d, bs, ws=ws))
        assert counters_clear(tq, ws, (R + 63) // 64), "arrival counters not returned to zero"
        if prev is not None:
            host(tq.gemv(*prev, ws=ws))
        y2 = host(tq.gemv(fmt, Wd, R, K, q, d, bs, ws=ws))
        assert np.array_equal(y1, y2)
        if fmt == "ptq1_0":
            # one summation order for every split: the same bits without a workspace
            assert np.array_equal(y1, host(tq.gemv(fmt, Wd, R, K, q, d, bs)))
        qo, do, _ = orc.quantize_q8k(x)
        yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
        assert_close_rows(y1, yo[0], mag[0], what=f"{fmt} {R}x{K} workspace")
        prev = (fmt, Wd, R, K, q, d, bs)


FUSED_CASES = [(1, 256, False), (1, 256, True), (65, 768, False), (200, 2560, True), (64, 8192, False),
               (33, 8192, True), (500, 1280, True), (7, 32256, False), (130, 65536, True)]


@pytest.mark.parametrize("R,K,use_ws", FUSED_CASES)
def test_gemv_f32_fused(tq, orc, R, K, use_ws):
    """Quantize-in-the-product entry: bit-identical to quantize_q8k + gemv with
    the same workspace, and within tolerance of the oracle."""
    import torch

    g = TI.rng(77, 13, R, K)
    W = TI.pq2_matrix(g, R, K)
    x = TI.activations(g, 1, K)
    x[0, 256:512] = 0.0  # one all-zero block (d = 0) when K allows it
    say("gemv_f32", R, K, use_ws)
    Wd = tq.repack(dev(W.reshape(-1)), "pq2_0", R, K)
    ws = tq.workspace("pq2_0", R, K) if use_ws else None
    # x at a 16-byte offset inside a larger buffer
    xbuf = torch.zeros(K + 8, dtype=torch.float32, device="cuda")
    xbuf[4:4 + K] = dev(x[0])
    xd = xbuf[4:4 + K]
    yf = host(tq.gemv_f32("pq2_0", Wd, R, K, xd, ws=ws))
    yf2 = host(tq.gemv_f32("pq2_0", Wd, R, K, xd, ws=ws))
    q, d, bs = tq.quantize_q8k(dev(x))
    yq = host(tq.gemv("pq2_0", Wd, R, K, q, d, ws=ws))
    assert np.array_equal(yf, yq) and np.array_equal(yf, yf2)
    if ws is not None:
        assert counters_clear(tq, ws, (R + 63) // 64)
    qo, do, _ = orc.quantize_q8k(x)
    yo, mag = orc.matmul("pq2_0", W, qo, do, with_mag=True)
    assert_close_rows(yf, yo[0], mag[0], what=f"gemv_f32 {R}x{K}")


def test_workspace_reuse_across_shapes(tq, orc):
    """One workspace shared by split products of different tile counts (above
    and below 64 tiles) and both formats, in an order where a call with fewer
    tiles comes between two calls with more: every call's outputs match its
    first result bit for bit and the oracle within tolerance, and all arrival
    counters are back at zero after each call."""
    import torch

    g = TI.rng(77, 18)
    shapes = [("pq2_0", 6000, 1024), ("pq2_0", 130, 512), ("ptq1_0", 5000, 2048), ("pq2_0", 4500, 2048),
              ("ptq1_0", 100, 4096)]
    cases = []
    for fmt, R, K in shapes:
        W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
        x = TI.activations(g, 1, K)
        Wd = tq.repack(dev(W.reshape(-1)), fmt, R, K)
        q, d, bs = tq.quantize_q8k(dev(x))
        qo, do, _ = orc.quantize_q8k(x)
        yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
        cases.append((fmt, R, K, Wd, q, d, bs, yo[0], mag[0]))
    tiles = max(-(-R // 64) for _, R, _ in shapes)
    ws = tq.workspace("pq2_0", tiles * 64, 256)
    first = {}
    for rnd in range(2):
        for i in [0, 1, 2, 3, 4, 0, 2, 1, 3]:
            fmt, R, K, Wd, q, d, bs, yo, mag = cases[i]
            say("workspace reuse", rnd, fmt, R, K)
            assert tq.workspace_bytes(fmt, R, K) <= ws.numel()
            y = host(tq.gemv(fmt, Wd, R, K, q, d, bs, ws=ws))
            assert counters_clear(tq, ws, tiles), (fmt, R, K)
            if i in first:
                assert np.array_equal(y, first[i]), (fmt, R, K)
            else:
                first[i] = y
                assert_close_rows(y, yo, mag, what=f"{fmt} {R}x{K} shared workspace")


@pytest.mark.parametrize("rows,K", [([200, 333], 2560), ([64, 1, 130, 65], 1024), ([7000], 768), ([6000, 6000], 512)])
def test_gemv_f32_batch(tq, orc, rows, K):
    """Independent fused products in one launch: without a workspace each
    output is bit-identical to its own tq_gemv_f32 call; with one (column
    splits when the total is below 384 tiles) within tolerance of the oracle,
    and the arrival counters are back at zero."""
    import torch

    g = TI.rng(77, 15, len(rows), K)
    Ws = [TI.pq2_matrix(g, R, K) for R in rows]
    xs = [TI.activations(g, 1, K) for _ in rows]
    say("gemv_f32_batch", rows, K)
    Wd = [tq.repack(dev(W.reshape(-1)), "pq2_0", R, K) for W, R in zip(Ws, rows)]
    xd = [dev(x[0]) for x in xs]
    ys = [host(y) for y in tq.gemv_f32_batch("pq2_0", Wd, rows, K, xd)]
    for m, R in enumerate(rows):
        assert np.array_equal(ys[m], host(tq.gemv_f32("pq2_0", Wd[m], R, K, xd[m]))), m
    R64 = sum(-(-R // 64) * 64 for R in rows)
    ws = tq.workspace("pq2_0", R64, K)
    yw = [host(y) for y in tq.gemv_f32_batch("pq2_0", Wd, rows, K, xd, ws=ws)]
    assert counters_clear(tq, ws, R64 // 64)
    for m, R in enumerate(rows):
        qo, do, _ = orc.quantize_q8k(xs[m])
        yo, mag = orc.matmul("pq2_0", Ws[m], qo, do, with_mag=True)
        assert_close_rows(ys[m], yo[0], mag[0], what=f"batch {m} {R}x{K}")
        assert_close_rows(yw[m], yo[0], mag[0], what=f"batch {m} {R}x{K} workspace")


def test_gemv_f32_rejects(tq):
    import torch

    R, K = 64, 32512
    Wd = torch.zeros(tq.repacked_bytes("pq2_0", R, K), dtype=torch.uint8, device="cuda")
    x = torch.zeros(K, dtype=torch.float32, device="cuda")
    y = torch.full((R,), 7.0, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.gemv_f32("pq2_0", Wd, R, K, x, out=y)
    assert e.value.status == tq.ERR_UNSUPPORTED and bool(torch.all(y == 7.0))


def test_degenerate_inputs(tq, orc):
    g = TI.rng(77, 7)
    R, K = 70, 1024
    W = TI.pq2_matrix(g, R, K)
    # zero activations: d = 0, q = 0, y = 0 exactly
    for T in (1, 3):
        _, q, d, bs, y, I = gpu_pipeline(tq, "pq2_0", W, np.zeros((T, K), np.float32))
        assert not q.any() and not d.any() and not bs.any() and not I.any() and np.all(y == 0)
    # zero weights (w = 0 everywhere) give exactly 0
    W0 = TI.assemble_pq2(np.full((R, K // 128, 32), 0x55, np.uint8), TI.scales_f16(g, R, K))
    _, _, _, _, y, I = gpu_pipeline(tq, "pq2_0", W0, TI.activations(g, 5, K))
    assert not I.any() and np.all(y == 0)
    # all +1 and all -1 (u = 2 in every slot position, the slot-3 sign hazard of the pages)
    Wp = TI.assemble_pq2(np.full((R, K // 128, 32), 0xAA, np.uint8), TI.scales_f16(g, R, K))
    Wm = TI.assemble_pq2(np.full((R, K // 128, 32), 0x00, np.uint8), TI.scales_f16(g, R, K))
    xe = np.full((2, K), 127.0, np.float32)
    xe[1] *= -1
    _, _, _, _, yp, Ip = gpu_pipeline(tq, "pq2_0", Wp, xe)
    _, _, _, _, ym, Im = gpu_pipeline(tq, "pq2_0", Wm, xe)
    assert np.all(Ip[0] == 128 * 127) and np.all(Ip[1] == -128 * 127) and np.array_equal(Im, -Ip)
    qo, do, _ = orc.quantize_q8k(xe)
    assert np.array_equal(yp, orc.matmul("pq2_0", Wp, qo, do))


def test_deterministic_and_stream(tq):
    import torch

    g = TI.rng(77, 8)
    R, K = 300, 4096
    W = TI.pq2_matrix(g, R, K)
    x = TI.activations(g, 9, K)
    Wd = tq.repack(dev(W.reshape(-1)), "pq2_0", R, K)
    q, d, bs = tq.quantize_q8k(dev(x))
    a = host(tq.gemm("pq2_0", Wd, R, K, q, d))
    b = host(tq.gemm("pq2_0", Wd, R, K, q, d))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = tq.gemm("pq2_0", Wd, R, K, q, d)
    s.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, c.cpu().numpy())


# ------------------------------------------------------------------ full-size workloads


def test_tiny_workload_full(tq, orc):
    fmt, W, x = TI.make("tiny_256x1024")
    say("tiny 256x1024")
    _, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
    qo, do, bso = orc.quantize_q8k(x)
    assert np.array_equal(q, qo) and np.array_equal(d, do) and np.array_equal(bs, bso)
    assert np.array_equal(I, orc.group_dots(fmt, W, qo))
    yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
    assert_close_rows(y, yo, mag, what="tiny")


@pytest.mark.parametrize("name", ["decode_32768x8192", "ptq1_32768x8192"])
def test_decode_workload_full(tq, orc, name):
    """Every output of the full-size matrix-vector product against the oracle,
    in the launch configuration of the benchmark (with a workspace), and the
    fused quantize-and-multiply entry bit-identical to it."""
    fmt, W, x = TI.make(name)
    say(name)
    R, G, _ = W.shape
    Wd, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
    ws = tq.workspace(fmt, R, G * 128)
    qd, dd, bd = tq.quantize_q8k(dev(x))
    yw = host(tq.gemv(fmt, Wd, R, G * 128, qd, dd, bd, ws=ws))
    assert np.array_equal(yw, y[0])
    if fmt == "pq2_0":
        assert np.array_equal(host(tq.gemv_f32(fmt, Wd, R, G * 128, dev(x[0]), ws=ws)), y[0])
    qo, do, bso = orc.quantize_q8k(x)
    assert np.array_equal(q, qo) and np.array_equal(d, do) and np.array_equal(bs, bso)
    assert np.array_equal(I, orc.group_dots(fmt, W, qo, threads=THREADS))
    yo, mag = orc.matmul(fmt, W, qo, do, threads=THREADS, with_mag=True)
    exact = assert_close_rows(y, yo, mag, what=name)
    say(f"{name}: {exact}/{y.size} outputs bit-identical")


@pytest.mark.parametrize("T", [4, 64])
def test_prefill_workload_sampled(tq, orc, T):
    """17408 x 5120 at 4 and 64 tokens: q8_K in full, outputs on sampled rows
    (first and last tile included) against the oracle."""
    fmt, W, x = TI.make("prefill_17408x5120_t64" if T == 64 else "prefill_17408x5120_t4")
    say("prefill", T)
    R = W.shape[0]
    _, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
    qo, do, bso = orc.quantize_q8k(x)
    assert np.array_equal(q, qo) and np.array_equal(d, do) and np.array_equal(bs, bso)
    g = TI.rng(77, 9, T)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(R - 64, R), g.integers(0, R, size=192)]))
    yo, mag = orc.matmul_rows(fmt, W, qo, do, rows, with_mag=True)
    assert_close_rows(y[:, rows], yo, mag, what=f"prefill T={T}")
    assert np.array_equal(I[:, rows[:40], :], orc.group_dots_rows(fmt, W, qo, rows[:40]))


def test_step64_shapes_sampled(tq, orc):
    """The five matrix shapes of the synthetic 64-layer decode step (one layer),
    each with its own fresh activation vector, sampled rows vs the oracle."""
    for mi, (name, R, K) in enumerate(TI.STEP64_SHAPES):
        say("step64 shape", name, R, K)
        g = TI.rng(TI.STEP64, 0, mi)
        W = TI.pq2_matrix(g, R, K)
        x = TI.activations(g, 1, K)
        Wd, q, d, bs, y, I = gpu_pipeline(tq, "pq2_0", W, x)
        qo, do, _ = orc.quantize_q8k(x)
        assert np.array_equal(q, qo) and np.array_equal(d, do)
        rows = np.unique(np.concatenate([np.arange(32), np.arange(R - 32, R), TI.rng(77, 10, mi).integers(0, R, 96)]))
        yo, mag = orc.matmul_rows("pq2_0", W, qo, do, rows, with_mag=True)
        assert_close_rows(y[0, rows], yo[0], mag[0], what=name)
        # the benchmark's launch: a workspace (column split below 384 tiles), and the fused entry
        ws = tq.workspace("pq2_0", R, K)
        yw = host(tq.gemv("pq2_0", Wd, R, K, dev(q), dev(d), ws=ws))
        assert_close_rows(yw[rows], yo[0], mag[0], what=name + " workspace")
        assert np.array_equal(host(tq.gemv_f32("pq2_0", Wd, R, K, dev(x[0]), ws=ws)), yw)
        assert np.array_equal(I[:, rows, :], orc.group_dots_rows("pq2_0", W, qo, rows))


@pytest.mark.parametrize("R,K,T", [(65, 65536, 40), (3, 65792, 40), (5, 131072, 5), (2, 131328, 3)])
def test_gemm_long_rows(tq, orc, R, K, T):
    """Prompt products on rows past the limit of the d_x copy fall back to one
    matrix-vector product per token; both sides of that limit agree with the
    oracle."""
    g = TI.rng(77, 14, R, K)
    W = TI.pq2_matrix(g, R, K)
    x = TI.activations(g, T, K)
    say("gemm long rows", R, K, T)
    Wd, q, d, bs, y, I = gpu_pipeline(tq, "pq2_0", W, x)
    qo, do, _ = orc.quantize_q8k(x)
    assert np.array_equal(I, orc.group_dots("pq2_0", W, qo))
    yo, mag = orc.matmul("pq2_0", W, qo, do, with_mag=True)
    assert_close_rows(y, yo, mag, what=f"gemm {R}x{K} T={T}")


@pytest.mark.parametrize("R,K,T", [(3, 32768, 3), (70, 16384, 5), (64, 8192, 7), (64, 8192, 9), (3, 32768, 16),
                                   (130, 1280, 8), (65, 3328, 31), (1, 256, 33),
                                   # 2-token blocks whose tables take 70 and 77 KiB of LDS (above 64 KiB)
                                   (64, 20480, 3), (64, 22528, 3)])
def test_gemm_ptq1_token_blocks(tq, orc, R, K, T):
    """ptq1_0 prompt products: below 8 tokens the vector-unit kernel, whose
    token-block tables fill the LDS budget (one token per block at the column
    limit, two at 16384 columns, a padded last block at 8192, two tokens with
    more than 64 KiB of tables at 20480 and 22528 columns); from 8 tokens
    the MFMA kernel (16 tokens per workgroup: ragged rows, ragged last token
    block, superblocks of fewer than 8 groups, the column limit)."""
    g = TI.rng(77, 17, R, K)
    W = TI.ptq1_matrix(g, R, K)
    x = TI.activations(g, T, K)
    say("gemm ptq1 token blocks", R, K, T)
    Wd, q, d, bs, y, I = gpu_pipeline(tq, "ptq1_0", W, x)
    qo, do, _ = orc.quantize_q8k(x)
    assert np.array_equal(I, orc.group_dots("ptq1_0", W, qo))
    yo, mag = orc.matmul("ptq1_0", W, qo, do, with_mag=True)
    assert_close_rows(y, yo, mag, what=f"gemm ptq1 {R}x{K} T={T}")


def test_max_columns(tq, orc):
    """The column limits of the ABI (pq2_0 2^20, ptq1_0 32768) and a wide
    pq2_0 case below it: one token, then a two-token prompt, without and with
    a workspace (column slices)."""
    g = TI.rng(77, 11)
    for fmt, K in (("pq2_0", 65536), ("pq2_0", 1 << 20), ("ptq1_0", 32768)):
        say("max cols", fmt, K)
        R = 3
        W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
        x = TI.activations(g, 2, K)
        qo, do, _ = orc.quantize_q8k(x)
        yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
        Wd, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x[:1])
        assert np.array_equal(I, orc.group_dots(fmt, W, qo[:1]))
        assert_close_rows(y, yo[:1], mag[:1], what=f"max cols {fmt} {K}")
        ws = tq.workspace(fmt, R, K)
        qd, dd, bsd = tq.quantize_q8k(dev(x))
        yw = host(tq.gemv(fmt, Wd, R, K, qd[1], dd[1], bsd[1], ws=ws))
        assert_close_rows(yw.reshape(1, R), yo[1:], mag[1:], what=f"max cols {fmt} {K} workspace")
        y2 = host(tq.gemm(fmt, Wd, R, K, qd, dd, bsd))
        assert_close_rows(y2, yo, mag, what=f"max cols {fmt} {K} prompt")


@pytest.mark.parametrize("fmt,T", [("ptq1_0", (1 << 19) + 17), ("pq2_0", 520001)])
def test_gemm_token_chunks(tq, orc, fmt, T):
    """Prompts long enough that the MFMA kernels are launched in two chunks of
    token blocks: ptq1_0 2^19 tokens then 17 more; pq2_0 (one row tile,
    2^22 workgroups per launch) 510304 tokens then 9697 more, both with a
    ragged last block."""
    R, K = 3, 256
    g = TI.rng(77, 19, R, K)
    W = TI.ptq1_matrix(g, R, K) if fmt == "ptq1_0" else TI.pq2_matrix(g, R, K)
    x = TI.activations(g, T, K)
    say("gemm token chunks", fmt, R, K, T)
    Wd, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
    qo, do, _ = orc.quantize_q8k(x)
    assert np.array_equal(q, qo)
    assert np.array_equal(I, orc.group_dots(fmt, W, qo))
    yo, mag = orc.matmul(fmt, W, qo, do, with_mag=True)
    assert_close_rows(y, yo, mag, what=f"gemm {fmt} {R}x{K} T={T}")
