"""Parity at the benchmark's own launches: the shapes and entry points that
bench.py times, against the CPU oracle (outputs within 1e-5 relative per
output, group dots bit-exact), on sampled rows where the oracle would take
too long for the whole matrix (first and last row tile always included)."""
import numpy as np
import pytest

import tq_inputs as TI
from test_gpu_parity import assert_close_rows, dev, gpu_pipeline, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_matvec_amd as m

    return m


def sample_rows(R, seed, n=192, edge=64):
    g = TI.rng(77, 40, seed)
    return np.unique(np.concatenate([np.arange(edge), np.arange(R - edge, R), g.integers(0, R, size=n)]))


@pytest.mark.parametrize("T", [1, 4, 64])
def test_ptq1_prefill_workload_sampled(tq, orc, T):
    """ptq1_0 17408 x 5120 at 1, 4 and 64 tokens (the benchmark's ptq1_0 prompt
    shapes; one token takes the matrix-vector kernel, 4 the vector-unit prompt
    kernel, 64 the MFMA prompt kernel): sampled rows against the oracle."""
    fmt, W, x = TI.make("ptq1_prefill_17408x5120_t64", tokens=T)
    R = W.shape[0]
    say("ptq1 prefill", T)
    _, q, d, bs, y, I = gpu_pipeline(tq, fmt, W, x)
    qo, do, bso = orc.quantize_q8k(x)
    assert np.array_equal(q, qo) and np.array_equal(d, do) and np.array_equal(bs, bso)
    rows = sample_rows(R, T)
    yo, mag = orc.matmul_rows(fmt, W, qo, do, rows, with_mag=True)
    exact = assert_close_rows(y[:, rows], yo, mag, what=f"ptq1 prefill T={T}")
    assert np.array_equal(I[:, rows[:48], :], orc.group_dots_rows(fmt, W, qo, rows[:48]))
    say(f"ptq1 prefill T={T}: {exact}/{yo.size} bit-identical")


def test_gate_up_batch_launch(tq, orc):
    """The 64-layer step's gate + up launch: tq_gemv_f32_batch over two
    17408 x 5120 matrices with one shared workspace (2 x 272 row tiles, so the
    columns are not split) and without, each problem with its own activation
    vector, against the oracle on sampled rows and against separate
    tq_gemv_f32 calls (bit-identical)."""
    import torch

    R, K = 17408, 5120
    Ws, Wds, xs = [], [], []
    for m in range(2):
        g = TI.rng(TI.STEP64, 0, m, 7)
        W = TI.pq2_matrix(g, R, K)
        Ws.append(W)
        Wds.append(tq.repack(dev(W.reshape(-1)), "pq2_0", R, K))
        xs.append(TI.activations(g, 1, K))
    xd = [dev(x[0]) for x in xs]
    pair_rows = 2 * (-(-R // 64) * 64)
    ws = torch.zeros(max(16, tq.workspace_bytes("pq2_0", pair_rows, K)), dtype=torch.uint8, device="cuda")
    for use_ws in (ws, None):
        say("gate+up batch, workspace" if use_ws is not None else "gate+up batch")
        outs = [host(o) for o in tq.gemv_f32_batch("pq2_0", Wds, [R, R], K, xd, ws=use_ws)]
        for m in range(2):
            single = host(tq.gemv_f32("pq2_0", Wds[m], R, K, xd[m]))
            assert np.array_equal(outs[m], single)
            rows = sample_rows(R, 50 + m)
            qo, do, _ = orc.quantize_q8k(xs[m])
            yo, mag = orc.matmul_rows("pq2_0", Ws[m], qo, do, rows, with_mag=True)
            assert_close_rows(outs[m][rows], yo[0], mag[0], what=f"gate/up {m}")
    # the shared workspace's counters are back to zero after the calls
    per = tq.workspace_bytes("pq2_0", 64, 256)
    idx = torch.arange(pair_rows // 64, device="cuda") * per
    assert int(torch.count_nonzero(torch.stack([ws[idx + k] for k in range(4)]))) == 0


@pytest.mark.parametrize("R,K", [(5120, 17408), (7168, 5120), (5120, 6144)])
def test_step_launches_with_workspace(tq, orc, R, K):
    """The 64-layer step's other launches (down 5120 x 17408, qkv 7168 x 5120,
    out 5120 x 6144): tq_gemv_f32 with a workspace, which splits the columns
    of these matrices (fewer than 384 row tiles), twice in a row, against
    tq_quantize_q8k + tq_gemv with the same workspace (bit-identical) and the
    oracle on sampled rows; the arrival counters are back at zero."""
    from test_gpu_parity import counters_clear

    g = TI.rng(TI.STEP64, 1, R, K)
    W = TI.pq2_matrix(g, R, K)
    x = TI.activations(g, 1, K)
    say("step launch with workspace", R, K)
    Wd = tq.repack(dev(W.reshape(-1)), "pq2_0", R, K)
    ws = tq.workspace("pq2_0", R, K)
    xd = dev(x[0])
    y1 = host(tq.gemv_f32("pq2_0", Wd, R, K, xd, ws=ws))
    assert counters_clear(tq, ws, -(-R // 64))
    y2 = host(tq.gemv_f32("pq2_0", Wd, R, K, xd, ws=ws))
    q, d, _ = tq.quantize_q8k(dev(x))
    yq = host(tq.gemv("pq2_0", Wd, R, K, q, d, ws=ws))
    assert np.array_equal(y1, y2) and np.array_equal(y1, yq)
    assert counters_clear(tq, ws, -(-R // 64))
    rows = sample_rows(R, 60)
    qo, do, _ = orc.quantize_q8k(x)
    yo, mag = orc.matmul_rows("pq2_0", W, qo, do, rows, with_mag=True)
    assert_close_rows(y1[rows], yo[0], mag[0], what=f"step launch {R}x{K}")


@pytest.mark.parametrize("R,K", [(28672, 3072), (28672, 2048)])
def test_gemv_f32_full_grid_one_slot(tq, orc, R, K):
    """A full grid (448 row tiles) with runs of 3 and 2 superchunks: the fused
    product keeps one ring slot there and quantizes its run in batches of 4
    and 2 blocks.  Bit-identical to tq_quantize_q8k + tq_gemv, and the oracle
    on sampled rows."""
    g = TI.rng(77, 41, R, K)
    W = TI.pq2_matrix(g, R, K)
    x = TI.activations(g, 1, K)
    say("full grid, one ring slot", R, K)
    Wd = tq.repack(dev(W.reshape(-1)), "pq2_0", R, K)
    y = host(tq.gemv_f32("pq2_0", Wd, R, K, dev(x[0])))
    q, d, _ = tq.quantize_q8k(dev(x))
    assert np.array_equal(y, host(tq.gemv("pq2_0", Wd, R, K, q, d)))
    rows = sample_rows(R, 61)
    qo, do, _ = orc.quantize_q8k(x)
    yo, mag = orc.matmul_rows("pq2_0", W, qo, do, rows, with_mag=True)
    assert_close_rows(y[rows], yo[0], mag[0], what=f"full grid {R}x{K}")
