"""GPU parity of the group-quantized product C = epi(alpha X W^T + beta C + bias) (affine codes,
w = s*q + o per group of G k) against the oracle, through the C ABI: the matrix-vector kernel of
decode, the matrix-core kernel of prefill and the scalar kernel, at sizes the oracle finishes in
seconds and at the decode workload's full size."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import gate
from gemm_harness import from_device, to_device

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


def qrun(g, q, kernel=0, **kw):
    """Run a QProblem on the GPU; returns decoded float64 C."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    X, Wq = to_device(q.X), to_device(q.Wq)
    S, O = to_device(q.scales), to_device(q.offsets)
    C = to_device(q.C)
    bias = to_device(q.bias) if q.bias is not None else None
    tmm.run_q(g.handle, X, Wq, S, O, C, M=q.M, N=q.N, K=q.K, bits=q.bits, group=q.group,
              x_type=q.x_type, alpha=q.alpha, beta=q.beta, epilogue=q.epilogue, bias=bias,
              kernel=kernel, **kw)
    torch.cuda.synchronize()
    return oracle.decode(q.x_type, from_device(C, q.x_type))


def qgate(q, got):
    Cref, D = oracle.qgemm(q)
    cin = oracle.decode(q.x_type, q.C) if q.beta != 0 else None
    tol = gate.tolerance(q.K, q.x_type, 1, bool(q.epilogue & W.EPI_GELU))
    return gate.check(got, Cref, D, tol, q.x_type, q.beta, cin)


def kernels():
    import tiled_matrix_multiply_amd as tmm
    return tmm


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 128), (8, 16), (8, 64)])
@pytest.mark.parametrize("x_type", ["bf16", "f16"])
def test_qgemv_parity(g, M, bits, G, x_type):
    import tiled_matrix_multiply_amd as tmm
    # N = 301 leaves the last workgroup partly empty; K spans several 64-chunk batches per lane
    q = W.make_qproblem(M, 301, 2048 + 2 * G, bits=bits, group=G, x_type=x_type, seed=M + bits,
                        epilogue=W.EPI_BIAS | W.EPI_GELU)
    r = qgate(q, qrun(g, q, kernel=tmm.GEMM_KERNEL_QGEMV))
    print(r)
    assert r.ok, r


@pytest.mark.parametrize("M,N,K,bits,G", [
    (1, 77, 4352, 4, 64),   # 136 chunks: two units per row block, the second mostly masked
    (1, 77, 4288, 4, 64),   # 67 groups (odd): per-lane scales and offsets, two units
    (2, 50, 2112, 4, 64),   # 33 groups (odd), one unit
    (1, 40, 8320, 4, 32),   # 260 groups: per-lane scales and offsets, three units
    (1, 33, 8192, 8, 64),   # 8-bit: four units
    (4, 77, 8192, 4, 64),   # 68 KiB of staged activations: more than 64 KiB of dynamic LDS
    (3, 50, 6144, 4, 64),   # three rows (the four-row kernel, one masked)
])
def test_qgemv_unit_shapes(g, M, N, K, bits, G):
    """Row blocks that take several units of chunks, ragged last units, and both forms of the
    scale and offset loads, with beta and the full epilogue."""
    import tiled_matrix_multiply_amd as tmm
    q = W.make_qproblem(M, N, K, bits=bits, group=G, x_type="bf16", seed=K + M, beta=0.5,
                        alpha=0.75, epilogue=W.EPI_BIAS | W.EPI_GELU)
    r = qgate(q, qrun(g, q, kernel=tmm.GEMM_KERNEL_QGEMV))
    print(r)
    assert r.ok, r


@pytest.mark.parametrize("bits,G", [(4, 8), (4, 64), (8, 3)])
def test_qsimt_parity_any_shape(g, bits, G):
    import tiled_matrix_multiply_amd as tmm
    q = W.make_qproblem(37, 29, 24 * G, bits=bits, group=G, x_type="bf16", seed=9, beta=-0.5,
                        alpha=1.25, epilogue=W.EPI_BIAS)
    r = qgate(q, qrun(g, q, kernel=tmm.GEMM_KERNEL_SIMT))
    print(r)
    assert r.ok, r


def test_q_auto_choices(g):
    # kernel choice touches no memory: well-separated, 16-byte aligned fake addresses
    kw = dict(bits=4, group=64, X=0x10000000, Wq=0x20000000, scales=0x30000000,
              offsets=0x40000000, C=0x50000000)
    assert g.select_kernel_q(1, 64, 256, **kw) == "qgemv"
    assert g.select_kernel_q(4, 64, 256, **kw) == "qgemv"
    # four rows of K = 8192 stage 68 KiB of activations (over 64 KiB, within the 80 KiB the
    # kernel takes); K = 10240 needs 85 KiB: the matrix-core kernel
    assert g.select_kernel_q(4, 64, 8192, **kw) == "qgemv"
    assert g.select_kernel_q(4, 64, 10240, **kw) == "qmfma"
    # group 8 is not a whole number of 16-byte chunks: the scalar kernel
    assert g.select_kernel_q(1, 64, 256, **dict(kw, group=8)) == "simt"
    # a code row stride that is not a multiple of 16 bytes
    assert g.select_kernel_q(1, 64, 256, **dict(kw, ldw=136)) == "simt"
    # misaligned codes
    assert g.select_kernel_q(1, 64, 256, **dict(kw, Wq=0x20000008)) == "simt"


def test_q_epilogue_variants(g):
    import tiled_matrix_multiply_amd as tmm
    for epi in (0, W.EPI_BIAS, W.EPI_GELU, W.EPI_BIAS | W.EPI_GELU):
        for beta in (0.0, 0.75):
            q = W.make_qproblem(2, 200, 1024, bits=4, group=64, seed=epi + 10, beta=beta,
                                alpha=-1.5, epilogue=epi)
            for k in (tmm.GEMM_KERNEL_QGEMV, tmm.GEMM_KERNEL_SIMT):
                r = qgate(q, qrun(g, q, kernel=k))
                assert r.ok, (epi, beta, k, r)


def test_q_beta_zero_does_not_read_c(g):
    q = W.make_qproblem(1, 96, 512, bits=4, group=64, seed=3)
    q.C = np.full(q.C.shape, 0x7FC0, dtype=np.uint16)  # bf16 NaN in C_in, never read
    got = qrun(g, q)
    q.C = np.zeros_like(q.C)
    r = qgate(q, got)
    assert r.ok, r


def test_q_degenerate_sizes(g):
    import tiled_matrix_multiply_amd as tmm
    # K = 0: C = epi(beta C + bias)
    q = W.make_qproblem(3, 17, 0, bits=4, group=64, seed=2, beta=0.5, epilogue=W.EPI_BIAS)
    for k in (tmm.GEMM_KERNEL_AUTO, tmm.GEMM_KERNEL_SIMT, tmm.GEMM_KERNEL_QGEMV):
        r = qgate(q, qrun(g, q, kernel=k))
        assert r.ok, (k, r)
    # M = 0 / N = 0: no-ops that return OK
    q = W.make_qproblem(1, 8, 128, bits=4, group=64, seed=2)
    X, Wq, S, O, C = (to_device(a) for a in (q.X, q.Wq, q.scales, q.offsets, q.C))
    st = tmm.gemm_run_q(g.handle, None, 0, 8, 128, 1.0, X.data_ptr(), 128, Wq.data_ptr(), 64, 4,
                        64, S.data_ptr(), O.data_ptr(), 2, 0.0, C.data_ptr(), 8,
                        tmm.GEMM_BF16, 0, None)
    assert st == tmm.GEMM_OK


def test_q_decode_full_size(g):
    """The decode workload at full size (1 x 28672 x 8192, 4-bit, groups of 64), every output
    against the oracle."""
    q = W.q4_decode()
    r = qgate(q, qrun(g, q))
    print(r)
    assert r.ok, r


@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 128), (8, 32), (8, 64)])
@pytest.mark.parametrize("x_type", ["bf16", "f16"])
def test_qmfma_parity(g, bits, G, x_type):
    """Matrix-core kernel: ragged M and N (not multiples of any tile), K spanning many K tiles.
    The weights pass through the 16-bit type once dequantised: at most 2^-9 (bf16) or 2^-12
    (f16) of each product, inside the u_out term of the gate."""
    import tiled_matrix_multiply_amd as tmm
    q = W.make_qproblem(300, 520, 1024, bits=bits, group=G, x_type=x_type, seed=G + bits,
                        epilogue=W.EPI_BIAS | W.EPI_GELU)
    r = qgate(q, qrun(g, q, kernel=tmm.GEMM_KERNEL_QMFMA))
    print(r)
    assert r.ok, r


def test_qmfma_epilogue_variants(g):
    import tiled_matrix_multiply_amd as tmm
    for epi in (0, W.EPI_BIAS | W.EPI_GELU):
        for beta in (0.0, -0.5):
            q = W.make_qproblem(264, 392, 512, bits=4, group=64, seed=epi + 20, beta=beta,
                                alpha=0.75, epilogue=epi)
            r = qgate(q, qrun(g, q, kernel=tmm.GEMM_KERNEL_QMFMA))
            assert r.ok, (epi, beta, r)


def test_qmfma_is_auto_for_many_rows(g):
    kw = dict(bits=4, group=64, X=0x10000000, Wq=0x20000000, scales=0x30000000,
              offsets=0x40000000, C=0x50000000)
    assert g.select_kernel_q(512, 4096, 4096, **kw) == "qmfma"
    assert g.select_kernel_q(5, 4096, 4096, **kw) == "qmfma"
    # K not a whole number of 64-element tiles: the scalar kernel
    assert g.select_kernel_q(512, 4096, 4064, **dict(kw, group=32)) == "simt"


def test_q_prefill_full_size(g):
    """The prefill workload at full size (4096^3, 4-bit, groups of 64), every output entry
    against the oracle."""
    q = W.q4_prefill()
    r = qgate(q, qrun(g, q))
    print(r)
    assert r.ok, r


@pytest.mark.parametrize("epilogue", [False, True])
def test_q_prefill_equals_the_bf16_gemm_of_its_weights(g, epilogue):
    """The prefill kernel dequantises each weight as it stages B (w = s q + o in one fp32 fused
    multiply-add, rounded once to bf16) and multiplies on the 256 x 256 tile like the plain bf16
    kernel.  Given those weights, dequantised on the host and stored N x K, the plain kernel on
    the same tile must return the same bits.  On the host the exact s q + o (float64) is rounded
    to fp32, as the fused multiply-add rounds it, and then to bf16.  4096^3, where the prefill
    kernel takes the 256 tile."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    if epilogue:
        q = W.make_qproblem(4096, 4096, 4096, bits=4, group=64, alpha=0.75, beta=0.5, seed=17,
                            epilogue=W.EPI_BIAS | W.EPI_GELU)
    else:
        q = W.q4_prefill()
    codes = np.empty((q.N, q.K), dtype=np.float64)
    codes[:, 0::2] = q.Wq & 15
    codes[:, 1::2] = q.Wq >> 4
    s = np.repeat(oracle.decode("bf16", q.scales), q.group, axis=1)
    o = np.repeat(oracle.decode("bf16", q.offsets), q.group, axis=1)
    w = (s * codes + o).astype(np.float32)
    wb = W.encode(w.astype(np.float64), "bf16")
    fused = qrun(g, q, kernel=tmm.GEMM_KERNEL_QMFMA)
    X, Wd, C = to_device(q.X), to_device(wb), to_device(q.C)
    bias = to_device(q.bias) if q.bias is not None else None
    tmm.run(g.handle, X, Wd, C, M=q.M, N=q.N, K=q.K, trans_b=True, alpha=q.alpha, beta=q.beta,
            a_type="bf16", epilogue=q.epilogue, bias=bias, kernel=tmm.GEMM_KERNEL_MFMA_256)
    torch.cuda.synchronize()
    plain = oracle.decode("bf16", from_device(C, "bf16"))
    same = fused.view(np.uint64) == plain.view(np.uint64)
    print(f"[quant] prefill vs bf16 GEMM of its weights (epilogue={epilogue}): "
          f"{same.mean():.6f} of {same.size} outputs bit-identical", flush=True)
    assert same.all(), f"{(~same).sum()} outputs differ, first at {np.argwhere(~same)[0]}"
