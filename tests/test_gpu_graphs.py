"""Graph capture of the product entry points, as the benchmark replays them:
every replay must give the eager results bit for bit, also when other calls
share the workspace between replays (a split product leaves its arrival
counters at zero, and the library records no memset node)."""
import numpy as np
import pytest

import tq_inputs as TI
from test_gpu_parity import dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_matvec_amd as m

    return m


def _matrix(tq, fmt, R, K, seed):
    g = TI.rng(91, seed, R, K)
    W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
    return tq.repack(dev(W.reshape(-1)), fmt, R, K)


def test_graph_replays_match_eager(tq):
    import torch

    # shapes: split with a workspace (few tiles), unsplit, ptq1_0 split,
    # two problems in one batched launch, prompt products of both formats
    R1, K1 = 2048, 4096   # 32 tiles: the workspace splits the columns
    R2, K2 = 1024, 8192
    Rp, Kp = 1024, 4096
    Rg, Kg = 1000, 2048
    W1 = _matrix(tq, "pq2_0", R1, K1, 1)
    W2 = _matrix(tq, "pq2_0", R2, K2, 2)
    Wp = _matrix(tq, "ptq1_0", Rp, Kp, 3)
    Wb = [_matrix(tq, "pq2_0", R1, K1, 4), _matrix(tq, "pq2_0", R1, K1, 5)]
    Wg = _matrix(tq, "pq2_0", Rg, Kg, 6)
    Wgp = _matrix(tq, "ptq1_0", Rg, Kg, 7)
    g = TI.rng(91, 99)
    x1 = dev(TI.activations(g, 1, K1)[0])
    x2 = dev(TI.activations(g, 1, K2)[0])
    xp = dev(TI.activations(g, 1, Kp)[0])
    xb = [dev(TI.activations(g, 1, K1)[0]) for _ in range(2)]
    xg = {T: dev(TI.activations(g, T, Kg)) for T in (4, 40)}
    qg = {T: tq.quantize_q8k(xg[T]) for T in xg}
    ws = torch.zeros(max(tq.workspace_bytes("pq2_0", 2 * R1, K1), tq.workspace_bytes("ptq1_0", Rp, Kp)),
                     dtype=torch.uint8, device="cuda")

    # preallocated outputs, written by the eager calls and by every replay
    o = {k: torch.empty(n, dtype=torch.float32, device="cuda")
         for k, n in [("split", R1), ("plain", R2), ("ptq1", Rp), ("two_kernel", R1), ("scratch", R1)]}
    o["b0"] = torch.empty(R1, dtype=torch.float32, device="cuda")
    o["b1"] = torch.empty(R1, dtype=torch.float32, device="cuda")
    for T in xg:
        o[f"gemm{T}"] = torch.empty((T, Rg), dtype=torch.float32, device="cuda")
        o[f"gemmp{T}"] = torch.empty((T, Rg), dtype=torch.float32, device="cuda")
    q1 = (torch.empty((1, K1), dtype=torch.int8, device="cuda"), torch.empty((1, K1 // 256), device="cuda"),
          torch.empty((1, K1 // 16), dtype=torch.int16, device="cuda"))
    qp = tq.quantize_q8k(xp.view(1, -1))

    def calls():
        tq.gemv_f32("pq2_0", W1, R1, K1, x1, out=o["split"], ws=ws)
        tq.gemv_f32("pq2_0", W2, R2, K2, x2, out=o["plain"])
        tq.gemv("ptq1_0", Wp, Rp, Kp, qp[0][0], qp[1][0], qp[2][0], out=o["ptq1"], ws=ws)
        tq.quantize_q8k(x1.view(1, -1), out=q1)
        tq.gemv("pq2_0", W1, R1, K1, q1[0][0], q1[1][0], q1[2][0], out=o["two_kernel"], ws=ws)
        tq.gemv_f32_batch("pq2_0", Wb, [R1, R1], K1, xb, outs=[o["b0"], o["b1"]], ws=ws)
        tq.gemv_f32_scratch("pq2_0", W1, R1, K1, x1, out=o["scratch"])
        for T in xg:
            q, d, bs = qg[T]
            tq.gemm("pq2_0", Wg, Rg, Kg, q, d, bs, out=o[f"gemm{T}"])
            tq.gemm("ptq1_0", Wgp, Rg, Kg, q, d, bs, out=o[f"gemmp{T}"])

    calls()
    torch.cuda.synchronize()
    ref = {k: host(v) for k, v in o.items()}
    assert np.array_equal(ref["split"], ref["two_kernel"])
    assert np.array_equal(ref["split"], ref["scratch"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    noise_x = dev(TI.activations(g, 1, K1)[0])
    for rep in range(3):
        for v in o.values():
            v.fill_(float("nan"))
        # other calls through the same workspace between replays
        tq.gemv_f32("pq2_0", Wb[rep % 2], R1, K1, noise_x, ws=ws)
        tq.gemv("ptq1_0", Wp, Rp, Kp, qp[0][0], qp[1][0], qp[2][0], ws=ws)
        torch.cuda.synchronize()
        say("graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in o.items():
            assert np.array_equal(host(v), ref[k]), (rep, k)
