"""GPU parity of stream-K (GEMM_KERNEL_MFMA_256_SK): the K tiles of all 256 x 256 output tiles
shared out evenly over a persistent grid of one workgroup per compute unit, each walking its run
one output tile (segment) at a time, the parts of a split tile added by the last to arrive, in
the order of their K ranges.  Called through gemm_run_ws_kernel, against the float64 oracle.

The parts are summed in a fixed order whichever part arrives last, so repeated runs must agree
bit for bit; every call must leave the workspace's counters at zero.
"""
import itertools
import zlib

import numpy as np
import pytest

import oracle
import workloads as W

import gemm_harness as H

pytestmark = pytest.mark.gpu

STREAM_K = 10  # GEMM_KERNEL_MFMA_256_SK
SLOT = 256 * 256 * 4


@pytest.fixture(scope="module")
def g():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    h = tmm.Gemm(0)
    yield h
    h.close()


def _cu_count():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _workspace(g, M, N):
    import torch
    import tiled_matrix_multiply_amd as tmm
    nbytes = tmm.gemm_kernel_workspace_bytes(g.handle, STREAM_K, M, N)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    assert ws.data_ptr() % 256 == 0
    return ws, nbytes


def _counters(ws, M, N):
    """The [arrive, done] counter pairs of an M x N output's tiles."""
    tiles = (-(-M // 256)) * (-(-N // 256))
    off = 2 * _cu_count() * SLOT // 4
    return ws[off:off + 2 * tiles].cpu().numpy()


def _parts(M, N, K):
    """Largest number of segments any output tile is cut into, from the run formula."""
    T, KT = (-(-M // 256)) * (-(-N // 256)), -(-K // 64)
    I = T * KT
    G = min(_cu_count(), I)
    owner = lambda x: ((x + 1) * G - 1) // I
    return max(owner(t * KT + KT - 1) - owner(t * KT) + 1 for t in range(T))


def _report(name, res):
    print(f"[streamk] {name}: {res}", flush=True)


def test_workspace_size(g):
    import tiled_matrix_multiply_amd as tmm
    cu = _cu_count()
    for M, N in [(1, 1), (256, 256), (257, 256), (3072, 3072), (4352, 1000)]:
        tiles = (-(-M // 256)) * (-(-N // 256))
        assert tmm.gemm_kernel_workspace_bytes(g.handle, STREAM_K, M, N) == \
            2 * cu * SLOT + -(-8 * tiles // 256) * 256
    assert tmm.gemm_kernel_workspace_bytes(g.handle, tmm.GEMM_KERNEL_MFMA_256x128_SK2, 512, 512) == \
        tmm.split_k_workspace_bytes(512, 512)
    assert tmm.gemm_kernel_workspace_bytes(g.handle, tmm.GEMM_KERNEL_MFMA_256, 512, 512) == 0
    assert tmm.gemm_kernel_workspace_bytes(g.handle, STREAM_K, -1, 5) == tmm.GEMM_ERR_INVALID_VALUE


@pytest.mark.parametrize("dtype,ta,tb", list(itertools.product(["f16", "bf16"], [False, True],
                                                                  [False, True])))
def test_integer_inputs_bit_exact(g, dtype, ta, tb):
    """Integer inputs in [-4, 4], exact in any order of accumulation: every layout, ragged M, N
    and K, beta and bias.  12 output tiles of 16 K tiles make fewer K tiles (192) than compute
    units, so each segment is one K tile and every tile is cut into 16 parts."""
    M, N, K = 700, 900, 1000
    assert _parts(M, N, K) == 16
    seed = zlib.crc32(f"streamk/{dtype}/{ta}/{tb}".encode()) & 0xFFFF
    p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, seed=seed,
                       dist_a=("int", (-4, 4)), dist_b=("int", (-4, 4)), fp8_scaled=False,
                       alpha=2.0, beta=-1.0, dist_c=("int", (-8, 8)), epilogue=W.EPI_BIAS)
    p.bias = np.round(p.bias * 30).astype(np.float32)
    ws, nbytes = _workspace(g, M, N)
    got, _, pad_ok = H.run_padded(g, p, kernel=STREAM_K, workspace=ws, workspace_bytes=nbytes)
    Cref, _ = oracle.gemm(p)
    expect = oracle.decode(p.c_type, W.encode(Cref, p.c_type))
    bad = np.argwhere(got != expect)
    assert pad_ok
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[0]}"
    assert (_counters(ws, M, N) == 0).all()


@pytest.mark.parametrize("dtype,M,N,K,ta,tb", [
    ("bf16", 3072, 3072, 1024, False, True),   # 144 tiles: parts of 2 and 3
    ("f16", 1000, 1300, 3000, True, False),    # 24 tiles of 47 K tiles: about 11 parts each
    ("bf16", 4352, 4352, 520, False, False),   # 289 tiles, more than compute units; ragged K
    ("bf16", 2304, 2560, 2048, True, True),    # 90 tiles
    ("f16", 100, 100, 20000, False, True),     # one tile cut into 256 parts
    ("bf16", 520, 1000, 1, True, False),       # K = 1: one K tile per output tile, none split
    ("f16", 4352, 1000, 64, False, False),     # 68 tiles of one K tile each
    ("bf16", 4352, 4352, 130, True, True),     # 289 tiles of 3 K tiles: runs span whole tiles
])
def test_gated_every_entry(g, dtype, M, N, K, ta, tb):
    """Random operands with beta, bias and GELU: every entry of the result meets the oracle's
    gate, and the counters are back at zero."""
    p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, alpha=0.75, beta=0.5,
                       seed=M + N + K, dist_a=("normal", 1.0), dist_b=("normal", K ** -0.5),
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    ws, nbytes = _workspace(g, M, N)
    got, _, pad_ok = H.run_padded(g, p, kernel=STREAM_K, workspace=ws, workspace_bytes=nbytes)
    res = H.gate_full(p, got)
    _report(f"{dtype} {M}x{N}x{K} ({_parts(M, N, K)} parts at most)", res)
    assert pad_ok and res.ok, res
    assert (_counters(ws, M, N) == 0).all()


def test_reproducible_and_shared_workspace(g):
    """Five runs of a problem whose tiles are cut into up to 11 parts give the same bits; a
    smaller call on the same workspace in between changes nothing; the result also meets the
    gate and agrees with the plain 256 x 256 tile within it."""
    # leading dimensions that are whole 16-byte multiples, as the matrix-core kernels need
    p = W.make_problem(1000, 1304, 3000, a_type="bf16", seed=77, dist_a=("normal", 1.0),
                       dist_b=("normal", 3000 ** -0.5), epilogue=W.EPI_BIAS | W.EPI_GELU)
    small = W.make_problem(300, 520, 704, a_type="bf16", seed=78, dist_a=("normal", 1.0),
                           dist_b=("normal", 704 ** -0.5), epilogue=W.EPI_BIAS)
    ws, nbytes = _workspace(g, p.M, p.N)
    d, ds = H.Device(p), H.Device(small)
    outs = []
    for i in range(5):
        d.reset_c()
        raw, got = H.run(g, p, kernel=STREAM_K, dev=d, workspace=ws, workspace_bytes=nbytes)
        outs.append(raw)
        if i == 2:
            _, got_small = H.run(g, small, kernel=STREAM_K, dev=ds, workspace=ws,
                                 workspace_bytes=nbytes)
            assert H.gate_full(small, got_small).ok
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    res = H.gate_full(p, got)
    _report("bf16 1000x1304x3000 five runs", res)
    assert res.ok
    d.reset_c()
    _, plain = H.run(g, p, kernel=4, dev=d)
    assert H.gate_full(p, plain).ok
    assert (_counters(ws, p.M, p.N) == 0).all()


def test_k_zero_runs_the_epilogue(g):
    """K = 0: the product is empty and the call runs as the plain 256 x 256 tile
    (C = beta C + bias, then GELU)."""
    p = W.make_problem(300, 400, 0, a_type="f16", seed=5, alpha=1.0, beta=0.5,
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    ws, nbytes = _workspace(g, p.M, p.N)
    got, _, pad_ok = H.run_padded(g, p, kernel=STREAM_K, workspace=ws, workspace_bytes=nbytes)
    assert pad_ok and H.gate_full(p, got).ok


def test_validation(g):
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(512, 512, 512, a_type="f16", seed=3)
    d = H.Device(p)
    ws, nbytes = _workspace(g, p.M, p.N)
    args = (p.M, p.N, p.K, 0, 0, 1.0, d.A.data_ptr(), p.lda, 1.0, d.B.data_ptr(), p.ldb, 1.0, 0.0,
            d.C.data_ptr(), p.ldc, tmm.GEMM_F16, tmm.GEMM_F16, tmm.GEMM_F16, 0, None)
    assert tmm.gemm_run_ws_kernel(g.handle, STREAM_K, None, *args, ws.data_ptr(), nbytes - 256) == tmm.GEMM_ERR_INVALID_VALUE
    assert tmm.gemm_run_ws_kernel(g.handle, STREAM_K, None, *args, None, 0) == tmm.GEMM_ERR_INVALID_VALUE
    # the static scratch array is far smaller than a stream-K workspace
    assert tmm.gemm_run_noalloc(g.handle, STREAM_K, None, *args) == tmm.GEMM_ERR_TOO_LARGE
    # fp32 is not a type of the stream-K kernel
    p32 = W.make_problem(512, 512, 512, a_type="f32", seed=3)
    d32 = H.Device(p32)
    a32 = (512, 512, 512, 0, 0, 1.0, d32.A.data_ptr(), 512, 1.0, d32.B.data_ptr(), 512, 1.0, 0.0,
           d32.C.data_ptr(), 512, tmm.GEMM_F32, tmm.GEMM_F32, tmm.GEMM_F32, 0, None)
    assert tmm.gemm_run_ws_kernel(g.handle, STREAM_K, None, *a32, ws.data_ptr(), nbytes) == tmm.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (_counters(ws, p.M, p.N) == 0).all()
