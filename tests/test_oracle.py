"""Pins for the CPU oracle: facts fixed by mathematics and by the number formats, not by the
oracle's own code.  A plausible mistake anywhere in the oracle (a dropped term, a wrong sign,
a swapped index or stride, a transposed operand, a wrong decoder) fails at least one of these.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import gate

DTYPES = ["f32", "f16", "bf16", "e4m3"]


def _dyadic(rng, shape, denom=8, lim=8):
    """Values k/denom with |k| <= lim: exact in every supported input format."""
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float64) / denom


def _frac_gemm(a, b, alpha, sa, sb, beta, cin, bias, gelu):
    """Exact rational reference with fractions.Fraction (a, b are logical float64 matrices)."""
    M, K = a.shape
    N = b.shape[1]
    S = [[sum((Fraction(a[i, k]) * Fraction(b[k, j]) for k in range(K)), Fraction(0))
          for j in range(N)] for i in range(M)]
    Dd = [[sum((abs(Fraction(a[i, k]) * Fraction(b[k, j])) for k in range(K)), Fraction(0))
           for j in range(N)] for i in range(M)]
    out = np.empty((M, N))
    den = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            t = Fraction(alpha) * Fraction(sa) * Fraction(sb) * S[i][j]
            if beta != 0.0:
                t += Fraction(beta) * Fraction(cin[i, j])
            if bias is not None:
                t += Fraction(float(bias[j]))
            if gelu:
                tf = float(t)
                out[i, j] = 0.5 * tf * (1.0 + math.erf(tf / math.sqrt(2.0)))
            else:
                out[i, j] = float(t)
            den[i, j] = float(Fraction(sa) * Fraction(sb) * Dd[i][j])
    return out, den


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_exact_all_small_shapes(dtype):
    """Every (M,N,K) in {1..4}^3, random transposes, alpha/beta/bias: exact to the last bit."""
    rng = np.random.default_rng(100 + DTYPES.index(dtype))
    c_type = W.OUT_TYPE[dtype]
    for M, N, K in itertools.product(range(1, 5), repeat=3):
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        a = _dyadic(rng, (M, K))
        b = _dyadic(rng, (K, N))
        alpha = float(rng.choice([1.0, 1.5, -0.25, 2.0]))
        beta = float(rng.choice([0.0, -0.5, 0.75]))
        cin = _dyadic(rng, (M, N), denom=4)
        use_bias = bool(rng.integers(2))
        bias = (_dyadic(rng, (N,), denom=16).astype(np.float32) if use_bias else None)
        sa = sb = 1.0
        if dtype == "e4m3":
            sa, sb = float(rng.choice([0.5, 2.0, 1.0])), float(rng.choice([0.25, 4.0]))
        A = W.encode(a.T.copy() if ta else a, dtype, 1.0)
        B = W.encode(b.T.copy() if tb else b, dtype, 1.0)
        C = W.encode(cin, c_type)
        epi = W.EPI_BIAS if use_bias else 0
        Cref, D = oracle.gemm_raw(M, N, K, ta, tb, alpha, A, M if ta else K, sa, B,
                                  K if tb else N, sb, beta, C, N, dtype, dtype, c_type, epi,
                                  bias)
        exp, den = _frac_gemm(a, b, alpha, sa, sb, beta, cin, bias, gelu=False)
        assert np.array_equal(Cref, exp), (M, N, K, ta, tb, Cref, exp)
        assert np.array_equal(D, den), (M, N, K, ta, tb)


def test_brute_force_gelu_epilogue():
    rng = np.random.default_rng(7)
    for M, N, K in [(1, 1, 1), (2, 3, 4), (4, 4, 4), (3, 1, 2)]:
        a, b = _dyadic(rng, (M, K)), _dyadic(rng, (K, N))
        cin = _dyadic(rng, (M, N), denom=4)
        bias = _dyadic(rng, (N,), denom=16).astype(np.float32)
        Cref, _ = oracle.gemm_raw(M, N, K, False, False, 1.25, W.to_f32(a), K, 1.0, W.to_f32(b),
                                  N, 1.0, -0.5, W.to_f32(cin), N, "f32", "f32", "f32",
                                  W.EPI_BIAS | W.EPI_GELU, bias)
        exp, _ = _frac_gemm(a, b, 1.25, 1, 1, -0.5, cin, bias, gelu=True)
        np.testing.assert_allclose(Cref, exp, rtol=1e-15, atol=1e-300)


def test_padded_leading_dimensions():
    """lda/ldb/ldc larger than the logical sizes: the padding must never be read."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 6
    for ta, tb in itertools.product([False, True], repeat=2):
        a, b, cin = _dyadic(rng, (M, K)), _dyadic(rng, (K, N)), _dyadic(rng, (M, N))
        a_st = a.T if ta else a
        b_st = b.T if tb else b
        lda, ldb, ldc = a_st.shape[1] + 3, b_st.shape[1] + 5, N + 2
        Ab = np.full((a_st.shape[0], lda), np.nan)
        Ab[:, :a_st.shape[1]] = a_st
        Bb = np.full((b_st.shape[0], ldb), np.nan)
        Bb[:, :b_st.shape[1]] = b_st
        Cb = np.full((M, ldc), np.nan)
        Cb[:, :N] = cin
        Cref, D = oracle.gemm_raw(M, N, K, ta, tb, 1.0, W.to_f32(Ab), lda, 1.0, W.to_f32(Bb),
                                  ldb, 1.0, 0.5, W.to_f32(Cb), ldc, "f32", "f32", "f32")
        exp, den = _frac_gemm(a, b, 1.0, 1, 1, 0.5, cin, None, False)
        assert np.array_equal(Cref, exp)
        assert np.array_equal(D, den)


def test_identity_and_permutation_exact():
    rng = np.random.default_rng(11)
    n, N = 37, 29
    for dtype in DTYPES:
        b = rng.standard_normal((n, N))
        B = W.encode(b, dtype, 1.0)
        bdec = oracle.decode(dtype, B)
        eye = W.encode(np.eye(n), dtype, 1.0)
        c_type = W.OUT_TYPE[dtype]
        Cref, _ = oracle.gemm_raw(n, N, n, False, False, 1.0, eye, n, 1.0, B, N, 1.0, 0.0, None,
                                  N, dtype, dtype, c_type)
        assert np.array_equal(Cref, bdec), dtype
        perm = rng.permutation(n)
        P = np.zeros((n, n))
        P[np.arange(n), perm] = 1.0
        Cref, _ = oracle.gemm_raw(n, N, n, False, False, 1.0, W.encode(P, dtype, 1.0), n, 1.0,
                                  B, N, 1.0, 0.0, None, N, dtype, dtype, c_type)
        assert np.array_equal(Cref, bdec[perm]), dtype


def test_rank1_closed_form():
    """A = u v^T, B = v' w^T  =>  C = (v . v') u w^T, exactly with dyadic values."""
    rng = np.random.default_rng(5)
    M, N, K = 19, 23, 31
    u, v = _dyadic(rng, M, 4, 4), _dyadic(rng, K, 4, 4)
    vp, w = _dyadic(rng, K, 4, 4), _dyadic(rng, N, 4, 4)
    a, b = np.outer(u, v), np.outer(vp, w)
    for dtype in ["f32", "bf16", "e4m3"]:
        Cref, D = oracle.gemm_raw(M, N, K, False, False, 1.0, W.encode(a, dtype, 1.0), K, 1.0,
                                  W.encode(b, dtype, 1.0), N, 1.0, 0.0, None, N, dtype, dtype,
                                  W.OUT_TYPE[dtype])
        dot = float(np.dot(v, vp))
        assert np.array_equal(Cref, dot * np.outer(u, w)), dtype
        assert np.array_equal(D, float(np.dot(np.abs(v), np.abs(vp))) * np.outer(np.abs(u),
                                                                                  np.abs(w)))


def test_alpha_beta_linearity_integer_exact():
    rng = np.random.default_rng(9)
    M, N, K = 33, 17, 40
    a = rng.integers(-4, 5, (M, K)).astype(np.float64)
    b = rng.integers(-4, 5, (K, N)).astype(np.float64)
    c = rng.integers(-4, 5, (M, N)).astype(np.float64)
    A, B, C = W.to_f32(a), W.to_f32(b), W.to_f32(c)
    base, _ = oracle.gemm_raw(M, N, K, 0, 0, 1.0, A, K, 1.0, B, N, 1.0, 0.0, None, N,
                              "f32", "f32", "f32")
    two, _ = oracle.gemm_raw(M, N, K, 0, 0, 2.0, A, K, 1.0, B, N, 1.0, 0.0, None, N,
                             "f32", "f32", "f32")
    assert np.array_equal(two, 2.0 * base)
    withc, _ = oracle.gemm_raw(M, N, K, 0, 0, 1.0, A, K, 1.0, B, N, 1.0, 3.0, C, N,
                               "f32", "f32", "f32")
    assert np.array_equal(withc - base, 3.0 * c)
    # beta = 0 never reads C: NaN in C must not propagate.
    nanc = np.full((M, N), np.nan, dtype=np.float32)
    z, _ = oracle.gemm_raw(M, N, K, 0, 0, 1.0, A, K, 1.0, B, N, 1.0, 0.0, nanc, N,
                           "f32", "f32", "f32")
    assert np.array_equal(z, base)


def test_transpose_identity_bitwise():
    """A*B == (B^T A^T)^T bit for bit: same k order, storage read through the trans flags."""
    rng = np.random.default_rng(13)
    M, N, K = 21, 34, 55
    A = W.to_f32(rng.uniform(-1, 1, (M, K)))
    B = W.to_f32(rng.uniform(-1, 1, (K, N)))
    c1, d1 = oracle.gemm_raw(M, N, K, 0, 0, 1.0, A, K, 1.0, B, N, 1.0, 0.0, None, N,
                             "f32", "f32", "f32")
    # op(A') = B^T read from B's storage (transA, lda = N); op(B') = A^T from A (transB, ldb=K)
    c2, d2 = oracle.gemm_raw(N, M, K, 1, 1, 1.0, B, N, 1.0, A, K, 1.0, 0.0, None, M,
                             "f32", "f32", "f32")
    assert np.array_equal(c1, c2.T)
    assert np.array_equal(d1, d2.T)


def test_numpy_float64_matmul_cross_check():
    rng = np.random.default_rng(17)
    for (M, N, K), (ta, tb) in zip([(64, 48, 80), (33, 65, 17), (100, 1, 257)],
                                   [(0, 0), (1, 0), (1, 1)]):
        a, b, c = rng.uniform(-1, 1, (M, K)), rng.uniform(-1, 1, (K, N)), rng.uniform(-1, 1,
                                                                                       (M, N))
        A, B, C = W.to_f32(a.T.copy() if ta else a), W.to_f32(b.T.copy() if tb else b), \
            W.to_f32(c)
        Cref, D = oracle.gemm_raw(M, N, K, ta, tb, 1.5, A, M if ta else K, 1.0, B,
                                  K if tb else N, 1.0, -0.5, C, N, "f32", "f32", "f32")
        a32 = (A.T if ta else A).astype(np.float64)
        b32 = (B.T if tb else B).astype(np.float64)
        ref = 1.5 * (a32 @ b32) - 0.5 * C.astype(np.float64)
        scale = float((np.abs(a32) @ np.abs(b32)).max())
        np.testing.assert_allclose(Cref, ref, rtol=0, atol=1e-12 * scale)
        np.testing.assert_allclose(D, np.abs(a32) @ np.abs(b32), rtol=1e-13)


def test_k_zero_and_empty():
    rng = np.random.default_rng(1)
    M, N = 4, 6
    c = rng.uniform(-1, 1, (M, N))
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    Cref, D = oracle.gemm_raw(M, N, 0, 0, 0, 1.0, None, 1, 1.0, None, N, 1.0, 2.0, W.to_f32(c),
                              N, "f32", "f32", "f32", W.EPI_BIAS, bias)
    assert np.array_equal(D, np.zeros((M, N)))
    assert np.array_equal(Cref, 2.0 * W.to_f32(c).astype(np.float64) + bias.astype(np.float64))
    Cref, D = oracle.gemm_raw(0, N, 5, 0, 0, 1.0, np.zeros(1, np.float32), 5, 1.0,
                              np.zeros(5 * N, np.float32), N, 1.0, 0.0, None, N, "f32", "f32",
                              "f32")
    assert Cref.shape == (0, N)


def test_rows_and_points_agree_with_full():
    p = W.make_problem(45, 38, 70, a_type="bf16", trans_a=True, alpha=0.75, beta=0.5,
                       epilogue=W.EPI_BIAS | W.EPI_GELU, seed=21)
    Cref, D = oracle.gemm(p)
    r, d = oracle.gemm_rows(p, 10, 7)
    assert np.array_equal(r, Cref[10:17]) and np.array_equal(d, D[10:17])
    rows = np.array([0, 44, 13, 7])
    cols = np.array([37, 0, 20, 5])
    pc, pd = oracle.gemm_points(p, rows, cols)
    assert np.array_equal(pc, Cref[rows, cols]) and np.array_equal(pd, D[rows, cols])


# ---------------------------------------------------------------------------------- codecs --

def test_e4m3_decoder_spec_points():
    """Fixed points of the OCP 8-bit E4M3 definition."""
    codes = np.array([0x38, 0x7E, 0x08, 0x01, 0x80, 0x00, 0xFE, 0x07, 0x09], dtype=np.uint8)
    vals = oracle.decode("e4m3", codes)
    assert list(vals[:4]) == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9]
    assert vals[4] == 0.0 and math.copysign(1, vals[4]) == -1.0
    assert vals[5] == 0.0 and math.copysign(1, vals[5]) == 1.0
    assert vals[6] == -448.0
    assert vals[7] == 7 * 2.0 ** -9          # largest subnormal
    assert vals[8] == 9 * 2.0 ** -9          # 2^-6 * (1 + 1/8)
    nan = oracle.decode("e4m3", np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all()


def test_e4m3_exhaustive_against_torch_and_encoder():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode("e4m3", codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    # encode(decode(c)) == c for every non-NaN code; the encoder is monotone and saturating.
    back = W.to_e4m3_bits(ours[~nan])
    assert np.array_equal(back, codes[~nan])
    x = np.linspace(-500, 500, 20001)
    q = oracle.decode("e4m3", W.to_e4m3_bits(x))
    assert np.all(np.diff(q) >= 0) and q.max() == 448.0 and q.min() == -448.0
    # the encoder rounds to nearest, ties to even, like torch's cast
    y = rng_vals = np.random.default_rng(0).normal(0, 30, 5000)
    t = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(W.to_e4m3_bits(rng_vals), t.numpy())


def test_bf16_codec_ties_to_even():
    f = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F80FFFF], dtype=np.uint32)
    bits = W.to_bf16_bits(f.view(np.float32).astype(np.float64))
    assert list(bits) == [0x3F80, 0x3F82, 0x3F81, 0x3F81]


def test_bf16_and_f16_decoders_exhaustive():
    torch = pytest.importorskip("torch")
    words = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bf = oracle.decode("bf16", words)
    ref = torch.from_numpy(words.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(bf) == nan).all() and np.array_equal(bf[~nan], ref[~nan])
    h = oracle.decode("f16", words)
    ref16 = words.view(np.float16).astype(np.float64)
    nan = np.isnan(ref16)
    assert (np.isnan(h) == nan).all() and np.array_equal(h[~nan], ref16[~nan])
    assert np.array_equal(np.signbit(h[~nan]), np.signbit(ref16[~nan]))


def test_fp8_scale_recipe():
    x = np.random.default_rng(0).normal(0, 1, (64, 64))
    s = W.e4m3_scale(x)
    assert s == np.float32(np.abs(x).max() / 448.0)
    q = oracle.decode("e4m3", W.to_e4m3_bits(x / float(s)))
    assert np.abs(q).max() == 448.0
    assert W.e4m3_scale(np.zeros(4)) == 1.0


# ------------------------------------------------------------------------------------ GELU --

def test_gelu_closed_forms():
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(1.0) == pytest.approx(0.8413447460685429, rel=1e-15)   # Phi(1)
    for x in [0.1, 0.7, 1.3, 2.9, 5.0]:
        assert oracle.gelu(x) - oracle.gelu(-x) == pytest.approx(x, rel=1e-14)
        assert oracle.gelu(x) == pytest.approx(0.5 * x * (1 + math.erf(x / math.sqrt(2))),
                                               rel=1e-15)
    assert oracle.gelu(40.0) == 40.0
    assert oracle.gelu(-40.0) == 0.0
    # erf-GELU, not the tanh approximation: they differ by ~1e-4 near x = -2.
    tanh_form = 0.5 * -2.0 * (1 + math.tanh(math.sqrt(2 / math.pi) * (-2.0 - 0.044715 * 8)))
    assert abs(oracle.gelu(-2.0) - tanh_form) > 1e-5


# ------------------------------------------------------------------------------------ gate --

def test_gate_rejects_nan_and_planted_errors():
    Cref = np.array([[1.0, -2.0], [0.5, 0.0]])
    D = np.array([[3.0, 4.0], [1.0, 0.0]])
    tol = gate.tolerance(64, "bf16")
    assert gate.check(Cref.copy(), Cref, D, tol, "bf16").ok
    bad = Cref.copy()
    bad[0, 1] = np.nan
    assert not gate.check(bad, Cref, D, tol, "bf16").ok
    bad = Cref.copy()
    bad[0, 0] += 4.0 * tol * 3.0
    r = gate.check(bad, Cref, D, tol, "bf16")
    assert not r.ok and r.argmax == (0, 0)
    bad = Cref.copy()
    bad[1, 1] = 1e-30          # zero denominator: only an exact zero passes
    assert not gate.check(bad, Cref, D, tol, "bf16").ok
    assert gate.tolerance(1000, "f32", gelu=False) == pytest.approx(1000 * 2 ** -23 + 5 * 2 ** -24)
    # bias-dominated entry (tiny D): the final rounding is judged against |Cref|
    Cref = np.array([0.1])
    D = np.array([1e-6])
    one_rounding = np.array([np.float32(0.1)], dtype=np.float64)
    assert gate.check(one_rounding, Cref, D, gate.tolerance(1, "f32", gelu=False), "f32").ok
    assert not gate.check(Cref * (1 + 2 ** -18), Cref, D, gate.tolerance(1, "f32", gelu=False),
                          "f32").ok
    # rounding into the subnormal range: within half a subnormal step passes, more fails
    Cref = np.array([3e-7])
    D = np.array([3e-7])
    sub = 2.0 ** -24
    assert gate.check(np.array([round(3e-7 / sub) * sub]), Cref, D, gate.tolerance(1, "f16"),
                      "f16").ok
    assert not gate.check(np.array([3e-7 + 2 * sub]), Cref, D, gate.tolerance(1, "f16"), "f16").ok


def test_oracle_detects_planted_sign_error():
    """A transposed-operand or sign slip in a candidate result is caught by the gate."""
    p = W.make_problem(40, 24, 56, a_type="f32", seed=2, beta=-0.5, alpha=1.5)
    Cref, D = oracle.gemm(p)
    cin = p.C.astype(np.float64)
    tol = gate.tolerance(p.K, "f32")
    good = Cref.astype(np.float32).astype(np.float64)
    assert gate.check(good, Cref, D, tol, "f32", p.beta, cin).ok
    wrong_sign = Cref - 2 * p.beta * cin        # beta term with the wrong sign
    assert not gate.check(wrong_sign, Cref, D, tol, "f32", p.beta, cin).ok
    a = p.A.astype(np.float64)
    b = p.B.astype(np.float64)
    swapped = 1.5 * (a @ b[:, ::-1]) + p.beta * cin   # columns of B reversed
    assert not gate.check(swapped, Cref, D, tol, "f32", p.beta, cin).ok


def test_named_workloads_shapes():
    p = W.fp32_1000_ragged(trans_a=True)
    assert p.A.shape == (1000, 1000) and p.lda == 1000 and p.beta == -0.5
    q = W.fp32_1000_ragged(trans_a=False)
    # the same logical A, stored transposed
    assert np.array_equal(p.A, q.A.T)
    f8 = W.fp8_4096(256)
    assert f8.A.dtype == np.uint8 and f8.c_type == "bf16"
    g = W.bf16_bias_gelu(512)
    assert g.bias is not None and g.bias.dtype == np.float32 and g.epilogue == 3
