"""tq_gemv_f32_scratch, the entry point that allocates nothing: called through
the raw C ABI (ctypes), its output must equal tq_gemv_f32 with a zeroed
caller workspace bit for bit (and the oracle within 1e-5 per output), on
two calls in a row -- the second with a smaller input -- and again on the
first shape, so that the shared static scratch left by one call serves the
next."""
import ctypes

import numpy as np
import pytest

import tq_inputs as TI

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_matvec_amd as m

    return m


def test_scratch_entry_matches_workspace_entry(tq, orc):
    import torch

    L = tq.lib()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream().cuda_stream)
    # 17408 x 5120: 272 row tiles, the columns split over the scratch;
    # then 640 x 8192 (10 tiles, another split); then 200 x 1024; then the first again
    shapes = [(17408, 5120), (640, 8192), (200, 1024), (17408, 5120)]
    cache = {}
    for n, (R, K) in enumerate(shapes):
        print("scratch entry", R, K, flush=True)
        if (R, K) not in cache:
            g = TI.rng(77, 60, R, K)
            W = TI.pq2_matrix(g, R, K)
            x = TI.activations(g, 1, K)
            Wd = tq.repack(torch.from_numpy(W.reshape(-1)).cuda(), "pq2_0", R, K)
            cache[(R, K)] = (W, x, Wd, torch.from_numpy(x[0].copy()).cuda())
        W, x, Wd, xd = cache[(R, K)]
        assert tq.lib().tq_workspace_bytes(1, R, K, 1) <= 384 * 16400
        y = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
        st = L.tq_gemv_f32_scratch(1, P(Wd.data_ptr()), R, K, P(xd.data_ptr()), P(y.data_ptr()), stream)
        assert st == tq.OK, tq.lib().tq_status_str(st)
        ws = tq.workspace("pq2_0", R, K)
        yw = torch.empty(R, dtype=torch.float32, device="cuda")
        st = L.tq_gemv_f32(1, P(Wd.data_ptr()), R, K, P(xd.data_ptr()), P(yw.data_ptr()), P(ws.data_ptr()), stream)
        assert st == tq.OK
        torch.cuda.synchronize()
        a, b = y.cpu().numpy(), yw.cpu().numpy()
        assert np.array_equal(a, b), f"call {n} {R}x{K}: {int(np.sum(a != b))} outputs differ"
        qo, do, _ = orc.quantize_q8k(x)
        rows = np.unique(np.concatenate([np.arange(min(R, 64)), np.arange(max(0, R - 64), R),
                                         TI.rng(77, 61, n).integers(0, R, 64)]))
        yo, mag = orc.matmul_rows("pq2_0", W, qo, do, rows, with_mag=True)
        ref = yo[0].astype(np.float64)
        bound = np.where(ref != 0, 1e-5 * np.abs(ref), 1e-5 * mag[0])
        assert np.all(np.abs(a[rows].astype(np.float64) - ref) <= bound)
    # shapes the plain entry does not take are refused the same way, touching nothing
    K = 1 << 20
    y = torch.full((64,), 3.0, dtype=torch.float32, device="cuda")
    z = torch.zeros(K, dtype=torch.float32, device="cuda")
    w = torch.zeros(tq.repacked_bytes("pq2_0", 64, K), dtype=torch.uint8, device="cuda")
    assert L.tq_gemv_f32_scratch(1, P(w.data_ptr()), 64, K, P(z.data_ptr()), P(y.data_ptr()), stream) \
        == tq.ERR_UNSUPPORTED  # 16 slices of 256 q8_K blocks: a slice does not fit on chip
    assert L.tq_gemv_f32_scratch(2, P(w.data_ptr()), 64, 256, P(z.data_ptr()), P(y.data_ptr()), stream) \
        == tq.ERR_UNSUPPORTED  # ptq1_0
    torch.cuda.synchronize()
    assert bool(torch.all(y == 3.0))
