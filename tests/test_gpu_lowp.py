"""GPU parity for the 8-, 6- and 4-bit paths beyond E4M3 with per-tensor scales: OCP E5M2, mixed
E4M3 x E5M2, packed fp4 (E2M1), packed 6-bit E2M3 / E3M2, and the OCP microscaling (MX)
block-scaled formats, all through the C ABI against the float64 oracle.  Bars as in test_gpu_parity: bit-exact where the
arithmetic is exact, the normalised-error gate K*2^-23 + u_out elsewhere."""
import itertools
import zlib

import numpy as np
import pytest

import oracle
import workloads as W

import gemm_harness as H

pytestmark = pytest.mark.gpu

KERNELS = {"simt": 1, "mfma64": 2, "mfma128": 3, "mfma256": 4}
PAIRS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e2m1", "e2m1")]


@pytest.fixture(scope="module")
def g():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    h = tmm.Gemm(0)
    yield h
    h.close()


def _report(name, res):
    print(f"[lowp] {name}: {res}", flush=True)


def _layouts(a_type):
    """(trans_a, trans_b) pairs a type is tested in: packed fp4 matrix-core runs need A stored
    M x K and B stored N x K."""
    if a_type == "e2m1":
        return [(False, True)]
    return list(itertools.product([False, True], [False, True]))


# ----------------------------------------------------------------------- format probes --

@pytest.mark.parametrize("kernel", list(KERNELS))
def test_e5m2_and_e2m1_are_ocp(g, kernel):
    """Codes that name the formats: E5M2 0x7B = 57344, 0x01 = 2^-16, 0x80 = -0; E2M1 nibble
    0x7 = 6, 0x1 = 0.5, 0xF = -6, packed low nibble first."""
    M, N, K = 32, 32, 64
    A = np.zeros((M, K), np.uint8)
    A[0, 0], A[1, 0], A[2, 0], A[3, 1] = 0x7B, 0x01, 0x80, 0x3C
    B = np.zeros((K, N), np.uint8)
    B[0, :] = 0x3C     # 1.0
    B[1, :] = 0x40     # 2.0
    p = W.Problem("e5m2_probe", M, N, K, False, False, 1.0, 0.0, "e5m2", "e5m2", "bf16", 0, A, B,
                  np.zeros((M, N), np.uint16), None)
    _, got = H.run(g, p, KERNELS[kernel])
    assert got[0, 0] == 57344.0 and got[1, 0] == 2.0 ** -16 and got[2, 0] == 0.0
    assert got[3, 0] == 2.0
    assert np.array_equal(got, oracle.gemm(p)[0])
    codes = np.zeros((M, K), np.uint8)
    codes[0, 0], codes[1, 0], codes[2, 0], codes[3, 1] = 0x7, 0x1, 0xF, 0x3   # 6, .5, -6, 1.5
    bc = np.zeros((N, K), np.uint8)
    bc[:, 0], bc[:, 1] = 0x2, 0x4                                             # 1.0, 2.0
    q = W.Problem("e2m1_probe", M, N, K, False, True, 1.0, 0.0, "e2m1", "e2m1", "bf16", 0,
                  W.pack_e2m1(codes), W.pack_e2m1(bc), np.zeros((M, N), np.uint16), None)
    _, got = H.run(g, q, KERNELS[kernel])
    assert got[0, 0] == 6.0 and got[1, 0] == 0.5 and got[2, 0] == -6.0 and got[3, 0] == 3.0
    assert np.array_equal(got, oracle.gemm(q)[0])


# ------------------------------------------------------------------ bit-exact integers --

@pytest.mark.parametrize("pair,kernel,layout",
                         [(pr, k, lo) for pr in PAIRS for k in KERNELS for lo in _layouts(pr[0])])
def test_integer_inputs_bit_exact(g, pair, kernel, layout):
    """Integers in [-4, 4] are exact in E4M3, E5M2 and E2M1: any fp32 accumulation order gives
    the exact sum, so the output must equal it rounded once to bf16."""
    at, bt = pair
    ta, tb = layout
    M, N, K = 200, 264, 320
    seed = zlib.crc32(f"{at}/{bt}/{kernel}/{ta}/{tb}".encode()) & 0xFFFF
    with_epi = (seed % 2) == 0
    p = W.make_problem(M, N, K, a_type=at, b_type=bt, trans_a=ta, trans_b=tb, seed=seed,
                       dist_a=("int", (-4, 4)), dist_b=("int", (-4, 4)), fp8_scaled=False,
                       alpha=2.0 if with_epi else 1.0, beta=-1.0 if with_epi else 0.0,
                       dist_c=("int", (-8, 8)), epilogue=W.EPI_BIAS if with_epi else 0)
    if p.bias is not None:
        p.bias = np.round(p.bias * 30).astype(np.float32)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
    Cref, _ = oracle.gemm(p)
    expect = oracle.decode("bf16", W.encode(Cref, "bf16"))
    bad = np.argwhere(got != expect)
    assert pad_ok
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[0]}"


# ------------------------------------------------------------------------ MX formats --

MX_CASES = [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e2m1", "e2m1")]


@pytest.mark.parametrize("pair,kernel,layout",
                         [(pr, k, lo) for pr in MX_CASES for k in KERNELS for lo in _layouts(pr[0])])
def test_mx_gate(g, pair, kernel, layout):
    """Block-scaled random operands, K = 352 (11 blocks: a partial last K tile for every tile
    size), ragged M and N, padded rows, and scale rows padded with NaN scales that must never
    be used (every kernel masks blocks past K)."""
    at, bt = pair
    ta, tb = layout
    M, N, K = 200, 264, 352
    seed = zlib.crc32(f"mx/{at}/{bt}/{kernel}/{ta}/{tb}".encode()) & 0xFFFF
    p = W.make_problem(M, N, K, a_type=at, b_type=bt, trans_a=ta, trans_b=tb, seed=seed, mx=True,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0), alpha=0.75,
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
    res = H.gate_full(p, got)
    _report(f"mx {at}x{bt} {kernel} ta={ta} tb={tb}", res)
    assert pad_ok and res.ok, res


def test_mx_scale_of_each_block_and_row(g):
    """All elements 1.0 and a different power-of-two scale for every (row, block) and
    (column, block): C[i, j] = 32 * sum_kb 2^(sa[i,kb]-127) 2^(sb[j,kb]-127), exact in bf16.
    A scale applied to the wrong block, row or column changes the result."""
    M, N, K = 96, 160, 64
    one = 0x38  # E4M3 1.0
    A = np.full((M, K), one, np.uint8)
    B = np.full((K, N), one, np.uint8)
    i, kb = np.meshgrid(np.arange(M), np.arange(2), indexing="ij")
    sa = (127 + (i + 3 * kb) % 5 - 2).astype(np.uint8)
    j, kb = np.meshgrid(np.arange(N), np.arange(2), indexing="ij")
    sb = (127 + (2 * j + kb) % 3 - 1).astype(np.uint8)
    p = W.Problem("mx_scales", M, N, K, False, False, 1.0, 0.0, "e4m3", "e4m3", "bf16", 0, A, B,
                  np.zeros((M, N), np.uint16), None, sa_blk=sa, sb_blk=sb)
    Cref, _ = oracle.gemm(p)
    for kernel in KERNELS:
        got, _, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
        assert pad_ok and np.array_equal(got, Cref), kernel


@pytest.mark.parametrize("name", ["e5m2_4096", "mxfp8_4096", "mxfp4_4096", "mxfp6_4096"])
def test_full_size(g, name):
    """The 4096^3 low-precision workloads, every output entry against the oracle."""
    p = getattr(W, name)()
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report(name, res)
    assert res.ok, res


def test_fp4_other_layouts_use_simt(g):
    """Packed fp4 stored M-contiguous or N-contiguous is served by the scalar kernel; forcing a
    matrix-core family there is refused."""
    import tiled_matrix_multiply_amd as tmm
    M, N, K = 64, 96, 128
    p = W.make_problem(M, N, K, a_type="e2m1", trans_a=False, trans_b=False, seed=11, mx=False,
                       dist_a=("int", (-3, 3)), dist_b=("int", (-3, 3)), fp8_scaled=False)
    d = H.Device(p)
    assert tmm.select_kernel(g.handle, M, N, K, a_type="e2m1", A=d.A, B=d.B, C=d.C) == "simt"
    with pytest.raises(tmm.GemmError) as e:
        H.run(g, p, KERNELS["mfma64"], d)
    assert e.value.status == tmm.GEMM_ERR_UNSUPPORTED
    _, got = H.run(g, p, 0, d)
    assert np.array_equal(got, oracle.gemm(p)[0])


# ---------------------------------------------------------------------- 6-bit formats --

FP6_PAIRS = [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e3m2", "e2m3")]


@pytest.mark.parametrize("kernel", list(KERNELS))
def test_fp6_codes_are_ocp(g, kernel):
    """Codes that name the 6-bit formats, through every kernel family: E2M3 0x1F = 7.5,
    0x01 = 1/8, 0x21 = -1/8, 0x08 = 1, 0x10 = 2; E3M2 0x1F = 28, 0x01 = 1/16, 0x0C = 1,
    0x10 = 2; packed four per three bytes, element i at bits 6i (k = 5 straddles a byte)."""
    M, N, K = 32, 32, 128
    cases = (("e2m3", 0x08, 0x10, [7.5, 0.125, -0.125]),
             ("e3m2", 0x0C, 0x10, [28.0, 0.0625, -0.0625]))
    for t, one, two, expect in cases:
        A = np.zeros((M, K), np.uint8)
        A[0, 0], A[1, 0], A[2, 0] = 0x1F, 0x01, 0x21
        A[3, 5] = one
        B = np.zeros((N, K), np.uint8)  # stored N x K
        B[:, 0] = one
        B[:, 5] = two
        p = W.Problem(f"{t}_probe", M, N, K, False, True, 1.0, 0.0, t, t, "bf16", 0,
                      W.pack_fp6(A), W.pack_fp6(B), np.zeros((M, N), np.uint16), None)
        _, got = H.run(g, p, KERNELS[kernel])
        assert list(got[:3, 0]) == expect and (got[:3] == got[:3, :1]).all(), (t, got[:4, :4])
        assert (got[3] == 2.0).all() and (got[4:] == 0).all(), t


@pytest.mark.parametrize("pair,kernel", [(pr, k) for pr in FP6_PAIRS for k in KERNELS])
def test_mx_fp6_gate(g, pair, kernel):
    """Block-scaled 6-bit operands (A stored M x K, B stored N x K), K = 384 (three 128-element
    K tiles), ragged M and N, padded rows (poisoned) and scale rows padded with NaN scales,
    alpha, beta and the full epilogue."""
    at, bt = pair
    M, N, K = 200, 264, 384
    seed = zlib.crc32(f"mx6/{at}/{bt}/{kernel}".encode()) & 0xFFFF
    p = W.make_problem(M, N, K, a_type=at, b_type=bt, trans_a=False, trans_b=True, seed=seed,
                       mx=True, dist_a=("normal", 1.0), dist_b=("normal", 1.0), alpha=0.75,
                       beta=-0.5, epilogue=W.EPI_BIAS | W.EPI_GELU)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
    res = H.gate_full(p, got)
    _report(f"mx {at}x{bt} {kernel}", res)
    assert pad_ok and res.ok, res


@pytest.mark.parametrize("pair,kernel", [(pr, k) for pr in FP6_PAIRS[:3] for k in KERNELS])
def test_fp6_per_tensor_gate(g, pair, kernel):
    """Per-tensor scaled 6-bit operands (scale max|x| -> the format's largest value)."""
    at, bt = pair
    M, N, K = 130, 96, 256
    seed = zlib.crc32(f"fp6/{at}/{bt}/{kernel}".encode()) & 0xFFFF
    p = W.make_problem(M, N, K, a_type=at, b_type=bt, trans_a=False, trans_b=True, seed=seed,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0), alpha=1.25)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
    res = H.gate_full(p, got)
    _report(f"fp6 {at}x{bt} {kernel}", res)
    assert pad_ok and res.ok, res


def test_fp6_partial_k_tile_uses_simt(g):
    """K not a whole number of 128-element tiles (352 = 11 blocks): the scalar kernel serves it,
    and forcing a matrix-core family is refused."""
    import tiled_matrix_multiply_amd as tmm
    M, N, K = 64, 96, 352
    p = W.make_problem(M, N, K, a_type="e2m3", trans_b=True, seed=12, mx=True,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0))
    d = H.Device(p)
    assert tmm.select_kernel(g.handle, M, N, K, trans_b=True, a_type="e2m3", A=d.A, B=d.B,
                             C=d.C) == "simt"
    with pytest.raises(tmm.GemmError) as e:
        H.run(g, p, KERNELS["mfma64"], d)
    assert e.value.status == tmm.GEMM_ERR_UNSUPPORTED
    _, got = H.run(g, p, 0, d)
    res = H.gate_full(p, got)
    assert res.ok, res
