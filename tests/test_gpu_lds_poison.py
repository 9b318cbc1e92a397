"""LDS race check of the staged K loop.  libgemm_lds_poison.so is libgemm.so with the matrix-core
kernels of the main families built to overwrite every LDS stage with all-ones words (a NaN in
each floating-point type staged) before the stage is refilled, and every stage before the
first copies.  A fragment read that ran ahead of its tile's copies, or that still read a stage
after its refill began, would then see the poison instead of data that may happen to be right.
Both libraries run the same calls on the same inputs; the outputs must agree bit for bit, and
hold no NaN.

Covered: the 32, 64, 128, 256 and 256 x 128 tiles (with their in-workgroup K splits and the
256 tile's copying waves), the split across two workgroups, stream-K, per-tensor and
block-scaled E4M3, E2M1 and E2M3 and quantized B (the prefill kernel, whose B stages are
written by the waves), in several layouts, with ragged M, N and K, beta and bias + GELU.
"""
import contextlib
import ctypes
import os

import numpy as np
import pytest

import workloads as W
import gemm_harness as H
from oracle import decode
from gemm_harness import from_device, to_device

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def _using(tmm, lib):
    """Route the binding's calls to `lib` (the binding looks its library up at call time)."""
    saved = tmm._lib
    tmm._lib = lib
    try:
        yield
    finally:
        tmm._lib = saved


@pytest.fixture(scope="module")
def libs():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    path = os.path.join(os.path.dirname(tmm.LIB_PATH), "libgemm_lds_poison.so")
    assert os.path.exists(path), f"{path} is missing: build the library first"
    dbg = ctypes.CDLL(path)
    for name in tmm.EXPORTS:
        src, dst = getattr(tmm.library(), name), getattr(dbg, name)
        dst.argtypes, dst.restype = src.argtypes, src.restype
    g = tmm.Gemm(0)
    with _using(tmm, dbg):
        gd = tmm.Gemm(0)
    yield tmm, g, dbg, gd
    with _using(tmm, dbg):
        gd.close()
    g.close()


def _workspace(tmm, g, kernel, M, N):
    import torch
    n = tmm.gemm_kernel_workspace_bytes(g.handle, kernel, M, N)
    if n <= 0:
        return None, 0
    return torch.zeros(-(-n // 4), dtype=torch.int32, device="cuda:0"), n


def _both(libs, p, kernel):
    """Decoded outputs (exact, float64) of the library and of its race-check build for one
    problem, with leading dimensions padded to the matrix-core kernels' 16-byte rows."""
    tmm, g, dbg, gd = libs
    out = []
    for lib, h in ((tmm.library(), g), (dbg, gd)):
        with _using(tmm, lib):
            ws, nbytes = _workspace(tmm, h, kernel, p.M, p.N)
            got, _, pad_ok = H.run_padded(h, p, kernel=kernel, workspace=ws,
                                          workspace_bytes=nbytes)
        assert pad_ok
        out.append(got)
    return out


def _check(name, got, got_dbg):
    same = np.array_equal(got.view(np.uint64), got_dbg.view(np.uint64))
    print(f"[poison] {name}: {got.size} outputs, bit-identical={same}", flush=True)
    assert not np.isnan(got).any(), f"{name}: the library's output holds NaN"
    assert not np.isnan(got_dbg).any(), f"{name}: the race-check build read a poisoned stage"
    bad = np.argwhere(got.view(np.uint64) != got_dbg.view(np.uint64))
    assert bad.size == 0, f"{name}: {bad.shape[0]} outputs differ, first at {bad[0]}"


LAYOUTS = [(False, False), (True, True)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kernel", [7, 2, 3, 4, 8])  # 32, 64, 128, 256, 256 x 128
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_sixteen_bit_tiles(libs, dtype, kernel, ta, tb):
    # K = 1000: 16 K tiles of 64, the last partial (zero-filled and fixed up)
    p = W.make_problem(520, 700, 1000, a_type=dtype, trans_a=ta, trans_b=tb, alpha=0.75,
                       beta=0.5, seed=kernel * 4 + 2 * ta + tb, dist_a=("normal", 1.0),
                       dist_b=("normal", 1000 ** -0.5), epilogue=W.EPI_BIAS | W.EPI_GELU)
    _check(f"{dtype} kernel {kernel} ta={ta} tb={tb}", *_both(libs, p, kernel))


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False)])
def test_256_tile_other_layouts(libs, ta, tb):
    p = W.make_problem(1000, 777, 1333, a_type="bf16", trans_a=ta, trans_b=tb, seed=11,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0), epilogue=W.EPI_BIAS)
    _check(f"bf16 256 tile ta={ta} tb={tb}", *_both(libs, p, 4))


@pytest.mark.parametrize("kernel,M,N,K", [
    (9, 520, 520, 1000),     # two workgroups per 256 x 128 tile
    (10, 700, 900, 1000),    # stream-K: 12 tiles of 16 K tiles, each cut into 16 parts
    (10, 1000, 1304, 3000),  # stream-K: parts of about 11 K tiles
])
def test_split_kernels(libs, kernel, M, N, K):
    p = W.make_problem(M, N, K, a_type="bf16", alpha=1.25, beta=-0.5, seed=M + K,
                       dist_a=("normal", 1.0), dist_b=("normal", K ** -0.5),
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    _check(f"bf16 kernel {kernel} {M}x{N}x{K}", *_both(libs, p, kernel))


@pytest.mark.parametrize("kernel", [7, 2, 3, 4])
@pytest.mark.parametrize("ta", [False, True])
def test_fp32_tiles(libs, kernel, ta):
    p = W.make_problem(300, 260, 333, a_type="f32", trans_a=ta, alpha=1.5, beta=-0.5,
                       seed=kernel + 10 * ta)
    _check(f"f32 kernel {kernel} ta={ta}", *_both(libs, p, kernel))


@pytest.mark.parametrize("kernel", [2, 3, 4])
@pytest.mark.parametrize("mx", [False, True])
def test_fp8_tiles(libs, kernel, mx):
    # K = 1056: eight and a quarter K tiles of 128 (the MX blocks of 32 all whole)
    p = W.make_problem(520, 700, 1056, a_type="e4m3", c_type="bf16", seed=30 + kernel, mx=mx,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0), epilogue=W.EPI_BIAS)
    _check(f"e4m3 kernel {kernel} mx={mx}", *_both(libs, p, kernel))


@pytest.mark.parametrize("kernel", [2, 3, 4])
@pytest.mark.parametrize("a_type", ["e2m1", "e2m3"])
@pytest.mark.parametrize("mx", [False, True])
def test_four_and_six_bit_tiles(libs, kernel, a_type, mx):
    """Packed 4- and 6-bit operands (both stored K-contiguous, as the matrix-core kernels take
    them).  The 6-bit tiles fill 96 bytes of each 128-byte LDS row; on the 256 tile only those
    are copied, so the other 32 keep the poison, which no fragment read may touch."""
    # 4 bits: K = 1056, whole blocks of 32 and a partial last K tile of 256 elements; 6 bits:
    # K = 1152, the matrix-core kernels take only whole 128-element K tiles
    K = 1056 if a_type == "e2m1" else 1152
    p = W.make_problem(520, 700, K, a_type=a_type, c_type="bf16", trans_b=True, mx=mx,
                       seed=40 + kernel + 10 * mx, dist_a=("normal", 1.0), dist_b=("normal", 1.0),
                       epilogue=W.EPI_BIAS)
    _check(f"{a_type} kernel {kernel} mx={mx}", *_both(libs, p, kernel))


@pytest.mark.parametrize("M,N,K", [(512, 700, 1024), (1000, 1300, 2048)])
def test_quantized_prefill(libs, M, N, K):
    import torch
    tmm, g, dbg, gd = libs
    q = W.make_qproblem(M, N, K, bits=4, group=64, x_type="bf16", seed=M,
                        epilogue=W.EPI_BIAS | W.EPI_GELU)
    out = []
    for lib, h in ((tmm.library(), g), (dbg, gd)):
        X, Wq = to_device(q.X), to_device(q.Wq)
        S, O, C = to_device(q.scales), to_device(q.offsets), to_device(q.C)
        bias = to_device(q.bias) if q.bias is not None else None
        with _using(tmm, lib):
            tmm.run_q(h.handle, X, Wq, S, O, C, M=M, N=N, K=K, bits=4, group=64, x_type="bf16",
                      alpha=q.alpha, beta=q.beta, epilogue=q.epilogue, bias=bias,
                      kernel=tmm.GEMM_KERNEL_QMFMA)
        torch.cuda.synchronize()
        out.append(decode("bf16", from_device(C, "bf16")))
    _check(f"q4 prefill {M}x{N}x{K}", *out)
