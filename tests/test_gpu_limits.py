"""Launch limits and workspace recovery on the GPU.

* Launches whose item count exceeds one grid pass: the repack kernels loop
  over their items with a grid stride (at most 2^20 workgroups of 256, i.e.
  2^28 work-items per launch) and the quantizer over its q8_K blocks (at most
  2^22 blocks per pass).  A matrix of more than 2^32 weights and an activation
  batch of more than 2^30 values take a second pass; the items of that pass
  are checked byte for byte (repack round trip) and against the oracle.
* tq_workspace_clear: a workspace whose counters were left non-zero makes the
  split product wrong (the contract stated in include/tq.h); clearing it with
  the kernel restores exact results, also when the clear is captured in a
  graph and replayed several times.
"""
import numpy as np
import pytest

import tq_inputs as TI
from test_gpu_parity import assert_close_rows, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_matvec_amd as m

    return m


def test_repack_past_one_grid_pass(tq):
    """pq2_0 131136 x 32768 (4.3e9 weights, 2.7e8 code dwords > 2^28 work-items
    of one pass) and ptq1_0 of the same shape: repack then unrepack round-trips
    byte for byte on the device."""
    import torch

    R, K = (1 << 17) + 64, 32768
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    for fmt in ("pq2_0", "ptq1_0"):
        say("repack past one pass", fmt, R, K)
        n = tq.canonical_bytes(fmt, R, K)
        if fmt == "pq2_0":
            table = torch.from_numpy(TI.VALID_PQ2_BYTES.astype(np.uint8)).cuda()
            canon = table[torch.randint(0, 81, (n,), device="cuda", generator=gen, dtype=torch.int32)]
        else:
            canon = torch.randint(0, 256, (n,), device="cuda", generator=gen, dtype=torch.int32).to(torch.uint8)
        Wd = tq.repack(canon, fmt, R, K, check_codes=(fmt == "pq2_0"))
        back = tq.unrepack(Wd, fmt, R, K)
        torch.cuda.synchronize()
        assert torch.equal(back, canon)
        del canon, Wd, back
        torch.cuda.empty_cache()


def test_quantize_past_one_grid_pass(tq, orc):
    """4097 tokens x 262144 columns (1.07e9 values, 4.2e6 q8_K blocks > the
    2^22 blocks of one pass): the first token and the last two, which fall in
    the second pass, bit-exact against the oracle."""
    import torch

    T, K = 4097, 1 << 18
    say("quantize past one pass", T, K)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(78)
    x = torch.randn((T, K), device="cuda", generator=gen)
    q, d, bs = tq.quantize_q8k(x)
    torch.cuda.synchronize()
    for t in (0, T - 2, T - 1):
        xt = x[t:t + 1].cpu().numpy()
        qo, do, bso = orc.quantize_q8k(xt)
        assert np.array_equal(q[t:t + 1].cpu().numpy(), qo)
        assert np.array_equal(d[t:t + 1].cpu().numpy(), do)
        assert np.array_equal(bs[t:t + 1].cpu().numpy(), bso)
    del x, q, d, bs
    torch.cuda.empty_cache()


def test_workspace_clear_recovers(tq, orc):
    """A workspace with garbage counters gives a wrong split product; after
    tq_workspace_clear (eager, then captured in a graph and replayed three
    times, with eager work between the replays) the product is exact again."""
    import torch

    R, K = 640, 8192  # 10 row tiles: the workspace splits the columns
    g = TI.rng(77, 41)
    W = TI.pq2_matrix(g, R, K)
    x = TI.activations(g, 1, K)
    Wd = tq.repack(dev(W.reshape(-1)), "pq2_0", R, K)
    q, d, bs = tq.quantize_q8k(dev(x))
    qo, do, _ = orc.quantize_q8k(x)
    yo, mag = orc.matmul("pq2_0", W, qo, do, with_mag=True)
    ref = host(tq.gemv("pq2_0", Wd, R, K, q, d, bs))
    assert_close_rows(ref.reshape(1, R), yo, mag, what="no workspace")
    ws = tq.workspace("pq2_0", R, K)
    assert np.array_equal(host(tq.gemv("pq2_0", Wd, R, K, q, d, bs, ws=ws)), ref)
    # garbage in every byte (counters included): the contract is broken
    ws.fill_(0x5A)
    y = torch.full((R,), 12345.0, device="cuda")
    tq.gemv("pq2_0", Wd, R, K, q, d, bs, out=y, ws=ws)
    assert not np.array_equal(host(y), ref)
    # eager clear
    tq.workspace_clear(ws)
    assert int(torch.count_nonzero(ws)) == 0
    assert np.array_equal(host(tq.gemv("pq2_0", Wd, R, K, q, d, bs, ws=ws)), ref)
    # the clear captured in a graph (no memset node), replayed three times
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            tq.workspace_clear(ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, rep
        assert np.array_equal(host(tq.gemv("pq2_0", Wd, R, K, q, d, bs, ws=ws)), ref), rep
    # odd sizes: the tail bytes past the last 16-byte word are cleared too
    buf = torch.full((1000,), 7, dtype=torch.uint8, device="cuda")
    tq.workspace_clear(buf[:999])
    b = host(buf)
    assert not b[:999].any() and b[999] == 7
