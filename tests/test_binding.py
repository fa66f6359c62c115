"""The Python binding checks every tensor before it reaches the C ABI: device,
dtype, contiguity and element count.  The kernels trust the sizes the host
validated, so a host tensor or an undersized buffer must raise here instead of
being read or written out of bounds on the GPU.  No kernel is launched (every
call below fails validation), so these run on a CPU-only machine: a tensor
subclass that reports itself as a GPU tensor stands in for device memory."""
import pytest
import torch


@pytest.fixture(scope="module")
def tq():
    import bit_quantized_matvec_amd as m

    return m


class FakeGpu(torch.Tensor):
    """Host memory that claims to be on the GPU: reaches the size checks."""

    @property
    def is_cuda(self):
        return True


def fake(n, dtype):
    return torch.zeros(n, dtype=dtype).as_subclass(FakeGpu)


R, K = 128, 512


def operands(tq, fmt="pq2_0", T=1):
    w = fake(tq.repacked_bytes(fmt, R, K), torch.uint8)
    q = fake(T * K, torch.int8)
    d = fake(T * K // 256, torch.float32)
    bs = fake(T * K // 16, torch.int16)
    return w, q, d, bs


def test_host_tensors_rejected(tq):
    w, q, d, bs = operands(tq)
    with pytest.raises(ValueError, match="CUDA"):
        tq.gemv("pq2_0", w, R, K, torch.zeros(K, dtype=torch.int8), d, bs, out=fake(R, torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        tq.gemv("pq2_0", w, R, K, q, d, bs, out=torch.zeros(R, dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        tq.gemv_f32("pq2_0", w, R, K, torch.zeros(K, dtype=torch.float32), out=fake(R, torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        tq.quantize_q8k(torch.zeros((1, K), dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        tq.repack(torch.zeros(tq.canonical_bytes("pq2_0", R, K), dtype=torch.uint8), "pq2_0", R, K)
    with pytest.raises(ValueError, match="CUDA"):
        tq.gemv("pq2_0", w, R, K, q, d, bs, out=fake(R, torch.float32), ws=torch.zeros(1 << 20, dtype=torch.uint8))


def test_undersized_buffers_rejected(tq):
    w, q, d, bs = operands(tq)
    y = fake(R, torch.float32)
    with pytest.raises(ValueError, match="out holds"):
        tq.gemv("pq2_0", w, R, K, q, d, bs, out=fake(R - 1, torch.float32))
    with pytest.raises(ValueError, match="ws holds"):
        tq.gemv("pq2_0", w, R, K, q, d, bs, out=y, ws=fake(tq.workspace_bytes("pq2_0", R, K) - 16, torch.uint8))
    with pytest.raises(ValueError, match="q holds"):
        tq.gemv("pq2_0", w, R, K, fake(K - 16, torch.int8), d, bs, out=y)
    with pytest.raises(ValueError, match="d holds"):
        tq.gemv("pq2_0", w, R, K, q, fake(1, torch.float32), bs, out=y)
    with pytest.raises(ValueError, match="bsums holds"):
        tq.gemv("pq2_0", w, R, K, q, d, fake(3, torch.int16), out=y)
    with pytest.raises(ValueError, match="w holds"):
        tq.gemv("pq2_0", fake(tq.repacked_bytes("pq2_0", R, K) - 1, torch.uint8), R, K, q, d, bs, out=y)
    with pytest.raises(ValueError, match="x holds"):
        tq.gemv_f32("pq2_0", w, R, K, fake(K - 4, torch.float32), out=y)
    with pytest.raises(ValueError, match="ws holds"):
        tq.gemv_f32("pq2_0", w, R, K, fake(K, torch.float32), out=y, ws=fake(8, torch.uint8))
    # prompt product: out must hold tokens x rows
    T = 4
    w, q4, d4, bs4 = operands(tq, T=T)
    q4 = q4.view(T, K)
    with pytest.raises(ValueError, match="out holds"):
        tq.gemm("pq2_0", w, R, K, q4, d4, bs4, out=fake(T * R - 1, torch.float32))
    with pytest.raises(ValueError, match="d holds"):
        tq.gemm("pq2_0", w, R, K, q4, d, bs4, out=fake(T * R, torch.float32))
    # the quantizer's outputs
    x = fake(T * K, torch.float32).view(T, K)
    with pytest.raises(ValueError, match="bsums holds"):
        tq.quantize_q8k(x, out=(fake(T * K, torch.int8), fake(T * K // 256, torch.float32), fake(K // 16, torch.int16)))
    # repack output
    with pytest.raises(ValueError, match="out holds"):
        tq.repack(fake(tq.canonical_bytes("pq2_0", R, K), torch.uint8), "pq2_0", R, K, out=fake(100, torch.uint8))


def test_ptq1_needs_bsums_and_batch_checks(tq):
    w, q, d, bs = operands(tq, "ptq1_0")
    y = fake(R, torch.float32)
    with pytest.raises(ValueError, match="bsums is required"):
        tq.gemv("ptq1_0", w, R, K, q, d, None, out=y)
    with pytest.raises(ValueError, match="bsums is required"):
        tq.group_dots("ptq1_0", w, R, K, q, None)
    wp = fake(tq.repacked_bytes("pq2_0", R, K), torch.uint8)
    xs = [fake(K, torch.float32), fake(K, torch.float32)]
    with pytest.raises(ValueError, match=r"out\[1\] holds"):
        tq.gemv_f32_batch("pq2_0", [wp, wp], [R, R], K, xs, outs=[fake(R, torch.float32), fake(R - 1, torch.float32)])
    with pytest.raises(ValueError, match=r"x\[0\] holds"):
        tq.gemv_f32_batch("pq2_0", [wp, wp], [R, R], K, [fake(K - 4, torch.float32), xs[1]],
                          outs=[fake(R, torch.float32), fake(R, torch.float32)])
    with pytest.raises(ValueError, match="ws holds"):
        tq.gemv_f32_batch("pq2_0", [wp, wp], [R, R], K, xs, outs=[fake(R, torch.float32), fake(R, torch.float32)],
                          ws=fake(tq.workspace_bytes("pq2_0", R, K), torch.uint8))


def test_wrong_dtype_and_shape(tq):
    w, q, d, bs = operands(tq)
    y = fake(R, torch.float32)
    with pytest.raises(ValueError, match="dtype"):
        tq.gemv("pq2_0", w, R, K, fake(K, torch.uint8), d, bs, out=y)
    with pytest.raises(ValueError, match="dtype"):
        tq.gemv("pq2_0", w, R, K, q, d, bs, out=fake(R, torch.float64))
    with pytest.raises(tq.TQError) as e:
        tq.gemv("pq2_0", w, R, 200, q, d, bs, out=y)
    assert e.value.status == tq.ERR_SHAPE
    with pytest.raises(ValueError, match="torch tensor"):
        tq.gemv("pq2_0", w, R, K, None, d, bs, out=y)
