"""GPU parity: the HIP kernels, called through the C ABI, against the float64 oracle.

Bars: bit-exact where the arithmetic is exact (integer-valued inputs, identity/permutation
operands, the fp8 format probe); otherwise the normalised-error gate
max |C - Cref| / (sum_k |a b| + |beta C_in|) <= K * 2^-23 + u_out, checked on every output entry,
the full 2048^3 and 4096^3 workloads included (the float64 oracle runs 4096^3 in seconds on the
host's cores); the headline workload is also checked on sampled entries each recomputed on its
own (a second path through the oracle).  The 16-bit GELU is checked in relative terms over the
whole line, its negative tail included.
"""
import itertools
import zlib

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import gate

import gemm_harness as H

pytestmark = pytest.mark.gpu

KERNELS = {"simt": 1, "mfma64": 2, "mfma128": 3, "mfma256": 4, "mfma32": 7}
WIDE = ("f32", "f16", "bf16")  # the types the 32 x 32 kernel takes


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
    print(f"[parity] {name}: {res}", flush=True)


# ------------------------------------------------------------------ fp8 format probe --

@pytest.mark.parametrize("kernel", ["mfma64", "mfma128", "mfma256", "simt"])
def test_fp8_is_ocp_e4m3(g, kernel):
    """Bytes whose meaning differs between OCP E4M3 and the older FNUZ variant:
    0x7E = 448 (FNUZ: 224), 0x01 = 2^-9 (FNUZ: 2^-10), 0x80 = -0 (FNUZ: NaN)."""
    M, N, K = 32, 32, 64
    A = np.zeros((M, K), np.uint8)
    A[0, 0], A[1, 0], A[2, 0], A[3, 1], A[4, 5] = 0x7E, 0x01, 0x80, 0x08, 0xFE
    B = np.zeros((K, N), np.uint8)
    B[0, :] = 0x38     # 1.0
    B[1, :] = 0x40     # 2.0
    B[5, :] = 0xB8     # -1.0
    p = W.Problem("fp8_probe", M, N, K, False, False, 1.0, 0.0, "e4m3", "e4m3", "bf16", 0, A, B,
                  np.zeros((M, N), np.uint16), None)
    raw, got = H.run(g, p, KERNELS[kernel])
    Cref, _ = oracle.gemm(p)
    assert got[0, 0] == 448.0 and got[1, 0] == 2.0 ** -9 and got[3, 0] == 2.0 ** -5
    assert got[4, 0] == 448.0 and not np.isnan(got).any()
    assert np.array_equal(got, Cref)


# ------------------------------------------------------------- bit-exact integer runs --

def _rne(x: np.ndarray, c_type: str) -> np.ndarray:
    """Round exact values to the output format (the single final rounding)."""
    return W.encode(x, c_type)


@pytest.mark.parametrize("dtype,kernel,ta,tb",
                         [c for c in itertools.product(["f32", "f16", "bf16", "e4m3"], KERNELS,
                                                       [False, True], [False, True])
                          if c[1] != "mfma32" or c[0] in WIDE])
def test_integer_inputs_bit_exact(g, dtype, kernel, ta, tb):
    """Integer inputs in [-4, 4]: every partial sum is an integer below 2^24, so any fp32
    accumulation order is exact and the result must equal the exact value rounded once."""
    M, N, K = 200, 264, 300
    seed = zlib.crc32(f"{dtype}/{kernel}/{ta}/{tb}".encode()) & 0xFFFF
    with_epi = (seed % 2) == 0
    p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, seed=seed,
                       dist_a=("int", (-4, 4)), dist_b=("int", (-4, 4)), fp8_scaled=False,
                       alpha=2.0 if with_epi else 1.0, beta=-1.0 if with_epi else 0.0,
                       dist_c=("int", (-8, 8)), epilogue=W.EPI_BIAS if with_epi else 0)
    if p.bias is not None:
        p.bias = np.round(p.bias * 30).astype(np.float32)   # small integers
    # leading dimensions padded to 16-byte multiples so that every kernel family accepts them
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
    Cref, _ = oracle.gemm(p)
    expect = oracle.decode(p.c_type, _rne(Cref, p.c_type))
    bad = np.argwhere(got != expect)
    assert pad_ok
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[0]}: got {got[tuple(bad[0])]} want {expect[tuple(bad[0])]}"


@pytest.mark.parametrize("dtype,K,ta,tb",
                         [(d, k, ta, tb) for d in ("f16", "bf16") for k in (1, 40, 64, 100, 128, 150, 192, 264)
                          for ta, tb in ((False, False), (True, True))] +
                         [(d, 150, ta, tb) for d in ("f16", "bf16") for ta, tb in ((False, True), (True, False))])
def test_short_k_256_tile_bit_exact(g, dtype, K, ta, tb):
    """The 256 x 256 tile over 1 .. 5 K tiles of 64: the K loop's first, second and last tiles
    take the special cases (tile 1 partly copied ahead, copies past the end of K, a partial
    last tile rewritten before its barrier).  Integer inputs: exact in any summation order."""
    M, N = 300, 264
    seed = zlib.crc32(f"short/{dtype}/{K}/{ta}/{tb}".encode()) & 0xFFFF
    p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, seed=seed,
                       dist_a=("int", (-4, 4)), dist_b=("int", (-4, 4)), fp8_scaled=False,
                       alpha=1.0, beta=-1.0, dist_c=("int", (-8, 8)), epilogue=W.EPI_BIAS)
    p.bias = np.round(p.bias * 30).astype(np.float32)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS["mfma256"])
    Cref, _ = oracle.gemm(p)
    expect = oracle.decode(p.c_type, _rne(Cref, p.c_type))
    bad = np.argwhere(got != expect)
    assert pad_ok
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[0]}: got {got[tuple(bad[0])]} want {expect[tuple(bad[0])]}"


def test_mfma32_refuses_8_bit_inputs(g):
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(64, 64, 128, a_type="e4m3", seed=5)
    with pytest.raises(tmm.GemmError) as e:
        H.run(g, p, KERNELS["mfma32"])
    assert e.value.status == tmm.GEMM_ERR_UNSUPPORTED


def test_identity_and_permutation_bit_exact(g):
    rng = np.random.default_rng(3)
    n = 320
    for dtype in ["f32", "bf16", "e4m3", "f16"]:
        b = rng.standard_normal((n, n))
        P = np.zeros((n, n))
        P[np.arange(n), rng.permutation(n)] = 1.0
        p = W.Problem("perm", n, n, n, False, False, 1.0, 0.0, dtype, dtype, W.OUT_TYPE[dtype],
                      0, W.encode(P, dtype, 1.0), W.encode(b, dtype, 1.0),
                      np.zeros((n, n), W.STORAGE[W.OUT_TYPE[dtype]]), None)
        raw, got = H.run(g, p)
        Cref, _ = oracle.gemm(p)
        # C = P B selects rows of B exactly; bf16/fp16/f32 outputs hold B's values exactly
        # except fp8 inputs, whose values bf16 also holds exactly.
        assert np.array_equal(got, Cref), dtype


# ------------------------------------------------------------------- named workloads --

def test_fp32_256(g):
    p = W.fp32_256()
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report("fp32 256^3", res)
    assert res.ok


@pytest.mark.parametrize("trans_a", [False, True])
def test_fp32_1000_ragged(g, trans_a):
    p = W.fp32_1000_ragged(trans_a)
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report(f"fp32 1000^3 alpha=1.5 beta=-0.5 {'TN' if trans_a else 'NN'}", res)
    assert res.ok


def test_fp32_1000_nn_vs_tn_report(g):
    """Same logical A stored two ways; reported, not gated (accumulation order may differ)."""
    _, nn = H.run(g, W.fp32_1000_ragged(False))
    _, tn = H.run(g, W.fp32_1000_ragged(True))
    print(f"[parity] fp32 1000 NN vs TN bitwise equal fraction: {np.mean(nn == tn):.4f}")


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096])
def test_fp16_square(g, n):
    p = W.fp16_square(n)
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report(f"fp16 {n}^3", res)
    assert res.ok


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096])
def test_bf16_bias_gelu_fused(g, n):
    p = W.bf16_bias_gelu(n)
    _, got = H.run(g, p)
    res = H.gate_full(p, got, cache=True)
    _report(f"bf16+bias+GELU fused {n}^3", res)
    assert res.ok
    if n == 4096:
        # the headline workload: sampled entries too, each recomputed on its own by the oracle
        res = H.gate_sampled(p, got)
        _report(f"bf16+bias+GELU fused {n}^3 (sampled, per-entry oracle)", res)
        assert res.ok


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096])
def test_bf16_bias_gelu_unfused(g, n):
    """GEMM without epilogue, then the separate bias+GELU pass; two roundings to bf16."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.bf16_bias_gelu(n)
    d = H.Device(p)
    H.run(g, p, dev=d, epilogue=0)
    g.bias_gelu(d.C, d.bias, M=p.M, N=p.N, c_type="bf16")
    torch.cuda.synchronize()
    got = oracle.decode("bf16", H.from_device(d.C, "bf16"))
    res = H.gate_full(p, got, roundings=2, cache=True)
    _report(f"bf16 GEMM then bias+GELU (unfused) {n}^3", res)
    assert res.ok


@pytest.mark.parametrize("c_type", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,N,ldc", [(37, 24, 24), (37, 24, 40), (5, 13, 13), (1, 8, 8),
                                     (300001, 8, 8), (9, 2056, 2056)])
@pytest.mark.parametrize("epi", [W.EPI_BIAS | W.EPI_GELU, W.EPI_GELU, W.EPI_BIAS])
def test_unfused_bias_gelu_pass(g, c_type, M, N, ldc, epi):
    """The separate elementwise pass on its own: C = GELU(C + bias) in place, on vector-path
    shapes (N and ldc multiples of 8, rows past the 65535 x 4 the launch covers in one pass)
    and scalar-path shapes, against the oracle's erf-GELU of the same stored values.  Inputs
    ~ N(0, 3^2), so the negative tail down to about -14 is exercised.  The bound is relative:
    one rounding to the output type plus the GELU's own error (EPS_GELU), or half a step among
    subnormals.  The padding of a row (ldc > N) must come back untouched."""
    import torch
    rng = np.random.default_rng(M * 7 + N * 3 + ldc + epi)
    x = rng.normal(0.0, 3.0, size=(M, ldc))
    stored = W.encode(x, c_type)
    bias = rng.normal(0.0, 0.5, size=N).astype(np.float32)
    Cd, bd = H.to_device(stored), H.to_device(bias)
    g.bias_gelu(Cd, bd, M=M, N=N, ldc=ldc, c_type=c_type, epilogue=epi)
    torch.cuda.synchronize()
    raw = H.from_device(Cd, c_type)
    assert np.array_equal(raw[:, N:], stored[:, N:])
    got = oracle.decode(c_type, raw[:, :N])
    xin = oracle.decode(c_type, stored[:, :N])
    t = xin + (bias.astype(np.float64) if epi & W.EPI_BIAS else 0.0)
    if epi & W.EPI_GELU:
        want = _gelu64(t)
        few = t.ravel()[:64]
        assert np.allclose([oracle.gelu(v) for v in few], want.ravel()[:64], rtol=1e-14, atol=0)
    else:
        want = t
    # The bias add is one fp32 rounding of t (relative 2^-24) ahead of GELU, whose relative
    # sensitivity d log(x Phi(x)) / d log x = 1 + x phi(x) / Phi(x) stays below 1 + x^2.
    eps = 0.0
    if epi & W.EPI_GELU:
        eps = EPS_GELU + ((1.0 + t * t) * 2.0 ** -24 if epi & W.EPI_BIAS else 0.0)
    elif epi & W.EPI_BIAS:
        eps = 2.0 ** -24
    bad = ~(np.abs(got - want) <= (U_OUT[c_type] + eps) * np.abs(want) + SUB[c_type])
    assert not bad.any(), f"{bad.sum()} elements, first at {np.argwhere(bad)[0]}: got {got[bad][0]} want {want[bad][0]}"


# Relative error of the library's GELU: the 16-bit outputs' erfc approximation is within 1e-5
# of x Phi(x) wherever x Phi(x) is a normal fp32 number (1.9e-6 on [-6, 3]); the fp32 outputs'
# device erfcf loses up to about 2 z^2 fp32 roundings to its argument z = -x / sqrt 2 in the
# tail (1.2e-5 at x = -14).  2^-16 = 1.5e-5 covers both.
EPS_GELU = 2.0 ** -16
U_OUT = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}   # unit roundoff
# Absolute allowance: half a subnormal step of the 16-bit outputs; for fp32 outputs 8 subnormal
# steps, since past x = -13 the device erfcf is itself an fp32 subnormal, each of its roundings
# up to half a step, and the result scales it by |x| / 2 <= 7.
SUB = {"f32": 2.0 ** -146, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def _gelu64(t):
    """x Phi(x) in float64, vectorised (the oracle's formula, 0.5 x erfc(-x / sqrt 2))."""
    from scipy.special import erfc
    return 0.5 * t * erfc(-t / np.sqrt(2.0))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kernel", ["simt", "mfma32", "mfma64", "mfma128", "mfma256"])
def test_gelu_tail_fused_k1(g, dtype, kernel):
    """The fused epilogue's GELU in relative terms over [-14, 4]: with K = 1 every accumulator
    is one exact product (a 16-bit value times a power of two), so the pre-activation is known
    exactly and the output must be x Phi(x) rounded once, to within EPS_GELU.  The shape has
    full and edge tiles for every kernel family."""
    M, N = 520, 264
    rng = np.random.default_rng(zlib.crc32(f"gelu/{dtype}/{kernel}".encode()))
    x = W.encode(rng.uniform(-7.0, 2.0, size=(M, 1)), dtype)
    scales = rng.choice([2.0, 1.0, 0.5, -0.5, 1.0, 2.0], size=(1, N))
    p = W.Problem("gelu_tail", M, N, 1, False, False, 1.0, 0.0, dtype, dtype, dtype,
                  W.EPI_GELU, x, W.encode(scales, dtype), np.zeros((M, N), W.STORAGE[dtype]),
                  None)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
    t = oracle.decode(dtype, x) * scales
    want = _gelu64(t)
    Cref, _ = oracle.gemm(p)
    assert np.allclose(Cref, want, rtol=1e-13, atol=1e-300)
    assert t.min() < -13.0 and t.max() > 3.5
    bad = ~(np.abs(got - want) <= (U_OUT[dtype] + EPS_GELU) * np.abs(want) + SUB[dtype])
    assert pad_ok
    assert not bad.any(), (f"{kname}: {bad.sum()} elements, first at {np.argwhere(bad)[0]}: "
                           f"x={t[bad][0]!r} got {got[bad][0]!r} want {want[bad][0]!r}")


@pytest.mark.parametrize("n", [512, 4096])
def test_fp8_e4m3(g, n):
    p = W.fp8_4096(n)
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report(f"fp8 E4M3 {n}^3 (sa={p.scale_a:.4g}, sb={p.scale_b:.4g})", res)
    assert res.ok


def test_bf16_twin_4096(g):
    p = W.bf16_twin_of_fp8(4096)
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report("bf16 4096^3 (fp8 twin)", res)
    assert res.ok


@pytest.mark.parametrize("M,N,K", [(1280, 1280, 1280), (1024, 2048, 2048)])
def test_k_split_beyond_one_round(g, M, N, K):
    """The 64 x 64 tile with its K loop split, on more tiles than compute units."""
    p = W.make_problem(M, N, K, a_type="bf16", seed=17, dist_a=("normal", 1.0),
                       dist_b=("normal", 1.0 / np.sqrt(K)), epilogue=W.EPI_BIAS | W.EPI_GELU)
    _, got = H.run(g, p)
    res = H.gate_full(p, got)
    _report(f"bf16+bias+GELU {M}x{N}x{K} (64 tile, K split)", res)
    assert res.ok


def test_kernel_selection(g):
    ptrs = dict(A=1 << 40, B=2 << 40, C=3 << 40)   # aligned, disjoint; never dereferenced
    assert g.select_kernel(4096, 4096, 4096, a_type="bf16", **ptrs) == "mfma256"
    assert g.select_kernel(2048, 2048, 2048, a_type="bf16", **ptrs) == "mfma128"
    # beyond two rounds of 128 x 128 workgroups the 256 x 256 tile is faster
    assert g.select_kernel(3072, 3072, 3072, a_type="bf16", **ptrs) == "mfma256"
    assert g.select_kernel(3072, 4096, 4096, a_type="bf16", **ptrs) == "mfma256"
    # 16-bit inputs whose 128 x 128 tiles need more than one round of the compute units and
    # whose 256 x 128 tiles fit in one: the 256 x 128 tile
    assert g.select_kernel(2816, 2816, 2816, a_type="bf16", **ptrs) == "mfma256x128"
    assert g.select_kernel(2048, 4096, 4096, a_type="bf16", **ptrs) == "mfma256x128"
    assert g.select_kernel(4096, 2048, 4096, a_type="f16", **ptrs) == "mfma256x128"
    assert g.select_kernel(1100, 4104, 520, a_type="bf16", **ptrs) == "mfma256x128"
    # ... but not other types, nor at one round of 128 x 128 tiles or fewer
    assert g.select_kernel(2816, 2816, 2816, a_type="f32", **ptrs) == "mfma128"
    assert g.select_kernel(2048, 4096, 4096, a_type="e4m3", **ptrs) == "mfma128"
    assert g.select_kernel(1024, 4096, 4096, a_type="bf16", **ptrs) == "mfma128"
    assert g.select_kernel(2048, 2048, 8192, a_type="bf16", **ptrs) == "mfma128"
    assert g.select_kernel(1024, 1024, 1024, a_type="f16", **ptrs) == "mfma64"
    assert g.select_kernel(1792, 1792, 1792, a_type="bf16", **ptrs) == "mfma128"
    assert g.select_kernel(1280, 1280, 1280, a_type="bf16", **ptrs) == "mfma64"
    # 64 x 64 tiles would fill a quarter of the compute units or less: 32 x 32, K split 4 ways
    assert g.select_kernel(512, 512, 512, a_type="bf16", **ptrs) == "mfma32"
    assert g.select_kernel(256, 256, 256, a_type="f32", **ptrs) == "mfma32"
    assert g.select_kernel(512, 512, 512, a_type="e4m3", **ptrs) == "mfma64"
    assert g.select_kernel(1000, 1000, 1000, a_type="f32", **ptrs) == "mfma64"
    assert g.select_kernel(1000, 1000, 1000, a_type="f32", A=(1 << 40) + 4, B=2 << 40,
                           C=3 << 40) == "simt"


# ------------------------------------------------------------------------ edge cases --

SHAPES = [(1, 1, 1), (31, 33, 17), (64, 64, 64), (65, 63, 129), (257, 255, 1), (300, 8, 4097),
          (1000, 777, 333), (130, 1030, 40)]


@pytest.mark.parametrize("dtype,kernel", [(d, k) for d in ("f32", "bf16")
                                           for k in ("mfma64", "mfma128", "mfma256")])
def test_edge_granules(g, dtype, kernel):
    """Edge tiles store whole 16-byte granules where they lie inside the matrix and the one
    granule that straddles column N element by element: N of every remainder class against the
    granule (1, 2, 3, 6 and 7 elements past a boundary of 8 for 16-bit outputs, 1 to 3 of 4 for
    fp32), ragged M, beta (masked C loads at the edge), bias and GELU; padding poisoned with NaN
    must come back intact."""
    for i, N in enumerate((257, 258, 259, 262, 263, 513)):
        M, K = 300 + 17 * i, 96 + 8 * i
        p = W.make_problem(M, N, K, a_type=dtype, alpha=0.75, beta=0.5, seed=700 + i,
                           dist_a=("normal", 1.0), dist_b=("normal", K ** -0.5),
                           epilogue=W.EPI_BIAS | W.EPI_GELU)
        got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel])
        res = H.gate_full(p, got)
        _report(f"{dtype} {M}x{N}x{K} {kname} edge granules", res)
        assert kname and pad_ok and res.ok, (N, res)


@pytest.mark.parametrize("dtype,kernel",
                         [(d, k) for d in ("f32", "f16", "bf16", "e4m3")
                          for k in ("auto", "simt", "mfma64", "mfma128", "mfma256", "mfma32")
                          if k != "mfma32" or d in WIDE])
def test_edge_shapes(g, dtype, kernel):
    """Ragged shapes with leading dimensions padded to 16-byte multiples (padding poisoned
    with NaN): every kernel family must mask its loads and stores at every edge."""
    kid = 0 if kernel == "auto" else KERNELS[kernel]
    for i, (M, N, K) in enumerate(SHAPES):
        if kernel == "simt" and M * N * K > 5e7:
            continue
        ta, tb = bool(i & 1), bool(i & 2)
        p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, alpha=0.75,
                           beta=0.5 if i % 3 == 0 else 0.0, epilogue=(i % 4), seed=40 + i,
                           dist_a=("normal", 1.0), dist_b=("normal", 1.0))
        got, kname, pad_ok = H.run_padded(g, p, kernel=kid)
        res = H.gate_full(p, got)
        tag = f"{dtype} {kernel}({kname}) {M}x{N}x{K} ta={ta} tb={tb}"
        assert res.ok, f"{tag}: {res}"
        assert pad_ok, f"{tag}: wrote outside the logical C"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "e4m3"])
def test_edge_shapes_unpadded_auto(g, dtype):
    """The same shapes stored densely: unaligned leading dimensions take the fallback."""
    for i, (M, N, K) in enumerate(SHAPES):
        ta, tb = bool(i & 1), bool(i & 2)
        p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, alpha=1.25,
                           beta=-0.5 if i % 2 else 0.0, epilogue=((i + 1) % 4), seed=60 + i,
                           dist_a=("normal", 1.0), dist_b=("normal", 1.0))
        _, got = H.run(g, p)
        res = H.gate_full(p, got)
        assert res.ok, f"{dtype} {M}x{N}x{K} ta={ta} tb={tb} aligned={H.mfma_aligned(p)}: {res}"


def test_k_zero_is_beta_c_plus_bias(g):
    for dtype in ["f32", "bf16", "e4m3"]:
        p = W.make_problem(70, 90, 0, a_type=dtype, beta=-2.0, epilogue=W.EPI_BIAS | W.EPI_GELU,
                           seed=9)
        _, got = H.run(g, p)
        res = H.gate_full(p, got)
        assert res.ok, (dtype, res)


def test_beta_zero_never_reads_c(g):
    p = W.make_problem(128, 128, 64, a_type="f32", seed=2)
    p.C = np.full((128, 128), np.nan, np.float32)
    _, got = H.run(g, p)
    assert np.isfinite(got).all()
    assert H.gate_full(p, got).ok


def test_m_zero_is_noop(g):
    import tiled_matrix_multiply_amd as tmm
    st = tmm.gemm_run(g.handle, None, 0, 5, 5, 0, 0, 1.0, None, 5, 1.0, None, 5, 1.0, 0.0, None,
                      5, 0, 0, 0, 0, None)
    assert st == tmm.GEMM_OK


@pytest.mark.parametrize("pad", ["aligned", "odd"])
def test_padded_leading_dimensions(g, pad):
    """ld > logical width: aligned padding keeps the matrix-core path, odd padding (+1) forces
    the fallback; both must give the oracle's result and leave the padding untouched."""
    ld_fn = H.aligned_ld if pad == "aligned" else (lambda w: w + 1)
    for dtype in ["f32", "bf16", "e4m3"]:
        p = W.make_problem(150, 90, 170, a_type=dtype, beta=0.5, seed=11, trans_a=True,
                           epilogue=W.EPI_BIAS)
        got, kname, pad_ok = H.run_padded(g, p, ld_fn)
        assert (kname == "simt") == (pad == "odd"), kname
        res = H.gate_full(p, got)
        assert res.ok and pad_ok, (dtype, pad, res, pad_ok)


def test_unaligned_pointer_falls_back(g):
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(96, 96, 96, a_type="f32", seed=12)
    A = H.to_device(np.concatenate([np.zeros(1, np.float32), p.A.ravel()]))[1:]
    B = H.to_device(p.B)
    C = H.to_device(p.C)
    assert g.select_kernel(96, 96, 96, a_type="f32", A=A, B=B, C=C) == "simt"
    with pytest.raises(tmm.GemmError) as e:
        tmm.run(g.handle, A, B, C, M=96, N=96, K=96, kernel=tmm.GEMM_KERNEL_MFMA_64)
    assert e.value.status == tmm.GEMM_ERR_UNSUPPORTED
    tmm.run(g.handle, A, B, C, M=96, N=96, K=96)
    torch.cuda.synchronize()
    assert H.gate_full(p, oracle.decode("f32", H.from_device(C, "f32"))).ok


def test_alias_rejected_before_launch(g):
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(64, 64, 64, a_type="f32", seed=13)
    d = H.Device(p)
    with pytest.raises(tmm.GemmError) as e:
        tmm.run(g.handle, d.A, d.B, d.A, M=64, N=64, K=64)
    assert e.value.status == tmm.GEMM_ERR_ALIAS


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_k_split_paths(g, dtype):
    """The 64 x 64 kernel splits its K loop between two groups of waves when its tiles leave no
    compute unit a second workgroup and K holds at least four tiles; both forms, ragged K."""
    for M, N, K in [(1100, 1100, 300),   # 324 tiles > 256 compute units: one group
                    (512, 520, 1000),    # 72 tiles: two groups, ragged last tile
                    (130, 200, 4500)]:   # 12 tiles, long K: two groups
        p = W.make_problem(M, N, K, a_type=dtype, alpha=1.25, beta=-0.5, seed=M + K,
                           epilogue=W.EPI_BIAS | W.EPI_GELU, dist_a=("normal", 1.0),
                           dist_b=("normal", 1.0))
        got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS["mfma64"])
        res = H.gate_full(p, got)
        assert res.ok and pad_ok, f"{dtype} {M}x{N}x{K}: {res}"


# ------------------------------------------------------------------- large extents --

@pytest.mark.parametrize("case", ["long_k", "tall", "wide", "long_rows"])
def test_large_extents(g, case):
    """Sizes far from the square workloads: K = 2^17 (the bound K * 2^-23 at its largest
    tested value, and the K split), 2^18 rows or columns (4096 tiles, one workgroup per tile
    and beyond 65535 tiles of the scalar kernel's grid.y would be), and rows of 2^21 elements
    (4 MiB: the staging copies' 32-bit offsets span 63 such rows)."""
    if case == "long_k":
        p = W.make_problem(64, 96, 1 << 17, a_type="bf16", seed=70, dist_a=("normal", 1.0),
                           dist_b=("normal", 1.0), epilogue=W.EPI_BIAS | W.EPI_GELU)
        got, kname, pad_ok = H.run_padded(g, p)
    elif case in ("tall", "wide"):
        M, N = (1 << 18, 16) if case == "tall" else (16, 1 << 18)
        p = W.make_problem(M, N, 64, a_type="f16", seed=71, dist_a=("normal", 1.0),
                           dist_b=("normal", 1.0), beta=0.5, alpha=-1.0)
        got, kname, pad_ok = H.run_padded(g, p)
    else:
        p = W.make_problem(64, 80, 96, a_type="bf16", seed=72, dist_a=("normal", 1.0),
                           dist_b=("normal", 1.0), trans_b=True)
        got, kname, pad_ok = H.run_padded(g, p, ld_fn=lambda w: w if w == p.N else 1 << 21)
    res = H.gate_full(p, got)
    print(f"[large] {case} {p.M}x{p.N}x{p.K} {kname}: {res}", flush=True)
    assert kname != "simt", kname
    assert pad_ok and res.ok, res


@pytest.mark.parametrize("trans_a", [False, True])
def test_tall_unaligned_takes_simt(g, trans_a):
    """M = 2^20 + 3 rows with an odd leading dimension: the matrix-core kernels cannot take the
    layout, so AUTO uses the scalar kernel, which must take any M (its workgroups stride over
    the tiles; there is no per-dimension grid limit)."""
    M, N, K = (1 << 20) + 3, 5, 40
    p = W.make_problem(M, N, K, a_type="f32", trans_a=trans_a, seed=73, alpha=0.5, beta=-1.0,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0), dist_c=("normal", 1.0),
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    got, kname, pad_ok = H.run_padded(g, p, ld_fn=lambda w: w + 1 if w % 2 == 0 else w + 2)
    res = H.gate_full(p, got)
    print(f"[large] tall unaligned {M}x{N}x{K} trans_a={trans_a} {kname}: {res}", flush=True)
    assert kname == "simt", kname
    assert pad_ok and res.ok, res
