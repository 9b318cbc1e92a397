"""Pins for the oracle's group-quantized product C = epi(alpha X W^T + beta C + bias) with
w[j, k] = s[j, k // G] * q[j, k] + o[j, k // G] (the quantized matmul of "X3: Metal GEMM",
section 7, in the affine group reading stated in oracle.c).  Exact rational brute force, the
unit-scale reduction to the plain product, nibble order, group locality, an offset-only closed
form and an independent numpy dequantisation.  CPU only."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W


def _bits16(vals, x_type):
    """Storage words of exactly representable values."""
    out = W.encode(np.asarray(vals, dtype=np.float64), x_type)
    back = oracle.decode(x_type, out)
    assert np.array_equal(back, np.asarray(vals, dtype=np.float64)), "value not representable"
    return out


def _qp(M, N, K, bits, G, x_type, x, q, s, o, alpha=1.0, beta=0.0, c_in=None, epilogue=0,
        bias=None):
    """A QProblem from explicit values (x: M x K, q: N x K codes, s, o: N x K/G)."""
    C = (_bits16(c_in, x_type) if c_in is not None
         else np.zeros((M, N), dtype=W.STORAGE[x_type]))
    return W.QProblem(name="pin", M=M, N=N, K=K, bits=bits, group=G, x_type=x_type,
                      alpha=alpha, beta=beta, epilogue=epilogue, X=_bits16(x, x_type),
                      Wq=W.pack_codes(np.asarray(q, dtype=np.uint8), bits),
                      scales=_bits16(s, x_type), offsets=_bits16(o, x_type), C=C, bias=bias)


@pytest.mark.parametrize("bits,G,x_type", [(4, 2, "bf16"), (4, 4, "f16"), (8, 2, "f16"),
                                           (8, 4, "bf16")])
def test_q_brute_force_exact(bits, G, x_type):
    rng = np.random.default_rng(bits * 10 + G)
    dy = np.array([-2.0, -1.5, -1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 1.0, 1.5, 2.0])
    top = (1 << bits) - 1
    for M, N, ng in itertools.product((1, 2, 3), (1, 2, 3), (1, 2, 3)):
        K = G * ng
        x = rng.choice(dy, size=(M, K))
        q = rng.integers(0, top + 1, size=(N, K))
        s = rng.choice(dy, size=(N, ng))
        o = rng.choice(dy, size=(N, ng))
        c_in = rng.choice(dy, size=(M, N))
        p = _qp(M, N, K, bits, G, x_type, x, q, s, o, alpha=0.75, beta=-1.25, c_in=c_in)
        C, D = oracle.qgemm(p)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(x[i, k]) * (Fraction(s[j, k // G]) * int(q[j, k]) +
                                              Fraction(o[j, k // G])) for k in range(K)]
                want = Fraction(3, 4) * sum(terms) + Fraction(-5, 4) * Fraction(c_in[i, j])
                assert Fraction(C[i, j]) == want, (M, N, K, i, j)
                assert Fraction(D[i, j]) == sum(abs(t) for t in terms)


def test_q_unit_scale_reduces_to_plain_product():
    """s = 1, o = 0: the quantized product is the plain product with B = the codes, stored
    N x K (transB), through the oracle's other path: identical bits."""
    rng = np.random.default_rng(5)
    for bits, G in ((4, 32), (8, 64)):
        M, N, K = 7, 9, 192
        x = W.encode(rng.normal(size=(M, K)), "bf16")
        xv = oracle.decode("bf16", x)
        q = rng.integers(0, 1 << bits, size=(N, K))
        ng = K // G
        p = _qp(M, N, K, bits, G, "bf16", xv, q, np.ones((N, ng)), np.zeros((N, ng)),
                alpha=1.5)
        C, D = oracle.qgemm(p)
        Cp, Dp = oracle.gemm_raw(M, N, K, False, True, 1.5, x, K, 1.0,
                                 q.astype(np.float32), K, 1.0, 0.0, None, N, "bf16", "f32",
                                 "bf16")
        assert np.array_equal(C, Cp) and np.array_equal(D, Dp)


def test_q_nibble_order():
    """Byte 0x21 holds codes 1 (k even, low nibble) then 2; 0x43 holds 3 then 4."""
    K, G = 8, 8
    Wq = np.array([[0x21, 0x43, 0x65, 0x87]], dtype=np.uint8)
    x = np.eye(K)
    p = W.QProblem(name="nib", M=K, N=1, K=K, bits=4, group=G, x_type="bf16", alpha=1.0,
                   beta=0.0, epilogue=0, X=_bits16(x, "bf16"), Wq=Wq,
                   scales=_bits16([[1.0]], "bf16"), offsets=_bits16([[0.0]], "bf16"),
                   C=np.zeros((K, 1), dtype=np.uint16), bias=None)
    C, _ = oracle.qgemm(p)
    assert C[:, 0].tolist() == [1, 2, 3, 4, 5, 6, 7, 8]


def test_q_group_locality():
    """Doubling the scale of group g of row j changes only column j, by exactly
    sum_{k in g} x_k s q_k (a power-of-two change keeps every value exact)."""
    rng = np.random.default_rng(11)
    M, N, K, G = 4, 5, 96, 32
    dy = np.array([-1.0, -0.5, 0.5, 1.0, 0.25, -0.25])
    x = rng.choice(dy, size=(M, K))
    q = rng.integers(0, 16, size=(N, K))
    s = rng.choice(dy, size=(N, K // G))
    o = rng.choice(dy, size=(N, K // G))
    C0, _ = oracle.qgemm(_qp(M, N, K, 4, G, "bf16", x, q, s, o))
    j, g = 3, 1
    s2 = s.copy()
    s2[j, g] *= 2
    C1, _ = oracle.qgemm(_qp(M, N, K, 4, G, "bf16", x, q, s2, o))
    others = [c for c in range(N) if c != j]
    assert np.array_equal(C0[:, others], C1[:, others])
    ks = range(g * G, (g + 1) * G)
    for i in range(M):
        delta = sum(Fraction(x[i, k]) * Fraction(s[j, g]) * int(q[j, k]) for k in ks)
        assert Fraction(C1[i, j]) - Fraction(C0[i, j]) == delta


def test_q_offsets_only_closed_form():
    """s = 0 and one offset c everywhere: C = c * sum_k x_k, whatever the codes."""
    rng = np.random.default_rng(12)
    M, N, K, G = 6, 3, 128, 64
    x = oracle.decode("bf16", W.encode(rng.normal(size=(M, K)), "bf16"))
    q = rng.integers(0, 16, size=(N, K))
    c = 0.375
    p = _qp(M, N, K, 4, G, "bf16", x, q, np.zeros((N, 2)), np.full((N, 2), c))
    C, _ = oracle.qgemm(p)
    for i in range(M):
        assert np.all(C[i] == c * math.fsum(x[i]))


def _numpy_dequant(p):
    """Independent dequantisation: unpack codes, decode scales / offsets with numpy views."""
    Wq = p.Wq.astype(np.int64)
    if p.bits == 4:
        q = np.empty((p.N, p.K), dtype=np.int64)
        q[:, 0::2] = Wq & 15
        q[:, 1::2] = Wq >> 4
    else:
        q = Wq
    if p.x_type == "bf16":
        dec = lambda v: (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        dec = lambda v: v.view(np.float16).astype(np.float64)
    s = np.repeat(dec(p.scales), p.group, axis=1)
    o = np.repeat(dec(p.offsets), p.group, axis=1)
    return dec(p.X), s * q + o


@pytest.mark.parametrize("bits,G,x_type", [(4, 64, "bf16"), (4, 32, "f16"), (8, 128, "bf16")])
def test_q_numpy_crosscheck(bits, G, x_type):
    p = W.make_qproblem(16, 24, 512, bits=bits, group=G, x_type=x_type, seed=3, beta=0.5,
                        epilogue=W.EPI_BIAS)
    C, D = oracle.qgemm(p)
    x, w = _numpy_dequant(p)
    cin = oracle.decode(x_type, p.C)
    want = x @ w.T + 0.5 * cin + p.bias.astype(np.float64)
    assert np.allclose(C, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(D, np.abs(x) @ np.abs(w).T, rtol=1e-12)


def test_q_gelu_epilogue_matches_plain_epilogue():
    p = W.make_qproblem(3, 8, 128, bits=4, group=64, seed=4, epilogue=W.EPI_BIAS | W.EPI_GELU)
    C, _ = oracle.qgemm(p)
    p.epilogue = 0
    S, _ = oracle.qgemm(p)
    for i in range(3):
        for j in range(8):
            assert C[i, j] == oracle.gelu(S[i, j] + float(p.bias[j]))


def test_q_generator_recipe():
    p = W.make_qproblem(2, 6, 256, bits=4, group=64, seed=9)
    x, w = _numpy_dequant(p)
    rng = np.random.default_rng(9)
    rng.normal(size=(2, 256))
    draw = rng.normal(0.0, 1.0 / 16.0, size=(6, 256))
    s = np.repeat(oracle.decode("bf16", p.scales), 64, axis=1)
    # every code is the nearest level to its draw, except where bf16 rounding of the offset
    # and scale pushes the group's extremes just outside the code range
    assert np.all(np.abs(w - draw) <= 0.5 * s + 2.0 ** -7 * np.abs(draw).max())
    assert p.Wq.shape == (6, 128) and p.scales.shape == (6, 4)


def test_q_rejects_bad_arguments():
    p = W.make_qproblem(2, 3, 128, bits=4, group=64, seed=1)
    p.group = 48  # K % G != 0
    with pytest.raises(ValueError):
        oracle.qgemm(p)
    p.group = 64
    p.bits = 3
    with pytest.raises(ValueError):
        oracle.qgemm(p)
