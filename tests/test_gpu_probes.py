"""GPU checks of the measurement helpers the benchmark relies on: the shader-clock probe reads
a plausible clock from the counters, and the bandwidth probe's copy copies every byte."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    h = tmm.Gemm(0)
    yield h
    h.close()


def test_clock_probe_reads_a_plausible_clock(g):
    import torch
    import tiled_matrix_multiply_amd as tmm
    khz = tmm.gemm_wall_clock_khz(g.handle)
    assert khz > 0
    buf = torch.zeros(4 * 64, dtype=torch.int64, device="cuda:0")
    assert tmm.gemm_probe_clock(g.handle, None, buf.data_ptr(), 64, 30) == tmm.GEMM_OK
    torch.cuda.synchronize()
    v = buf.cpu().numpy().reshape(-1, 4).astype(np.float64)
    ticks = v[:, 3] - v[:, 1]
    assert (ticks >= 30 * khz / 1000 - 1).all(), ticks      # the spin lasted its span
    mhz = (v[:, 2] - v[:, 0]) / ticks * khz / 1000.0
    print(f"[probe] shader clock {mhz.mean():.0f} MHz (min {mhz.min():.0f}, max {mhz.max():.0f})")
    assert ((mhz > 100) & (mhz < 3000)).all(), mhz
    # arguments out of range are refused before any launch
    assert tmm.gemm_probe_clock(g.handle, None, buf.data_ptr(), 0, 30) == tmm.GEMM_ERR_INVALID_VALUE
    assert tmm.gemm_probe_clock(g.handle, None, None, 4, 30) == tmm.GEMM_ERR_INVALID_VALUE


def test_bandwidth_probe_copies_every_byte(g):
    import torch
    import tiled_matrix_multiply_amd as tmm
    n = (1 << 22) + 16 * 37          # bytes: not a multiple of the grid's stride
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    assert tmm.gemm_probe_bandwidth(g.handle, None, src.data_ptr(), dst.data_ptr(), n,
                                    sink.data_ptr()) == tmm.GEMM_OK
    assert tmm.gemm_probe_bandwidth(g.handle, None, src.data_ptr(), None, n,
                                    sink.data_ptr()) == tmm.GEMM_OK
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert tmm.gemm_probe_bandwidth(g.handle, None, src.data_ptr(), None, n - 8,
                                    sink.data_ptr()) == tmm.GEMM_ERR_INVALID_VALUE
    assert tmm.gemm_probe_bandwidth(g.handle, None, src.data_ptr(), src.data_ptr(), n,
                                    sink.data_ptr()) == tmm.GEMM_ERR_ALIAS
