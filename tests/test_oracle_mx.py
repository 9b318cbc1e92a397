"""Pins for the oracle's 8-bit E5M2, 4-bit E2M1, 6-bit E2M3 / E3M2 and OCP microscaling (MX)
paths: values the OCP formats define, an independent library decoder where one exists, and exact
rational brute force.  CPU only."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

# OCP E2M1: the eight magnitudes the format defines (exponent bias 1, one mantissa bit).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e5m2_spec_points():
    d = oracle.decode("e5m2", np.array([0x3C, 0x7B, 0x04, 0x01, 0x03, 0x80, 0xBC, 0x7C, 0xFC,
                                        0x7D, 0x7E, 0x7F], dtype=np.uint8))
    assert d[0] == 1.0 and d[1] == 57344.0 and d[2] == 2.0 ** -14
    assert d[3] == 2.0 ** -16 and d[4] == 3 * 2.0 ** -16
    assert d[5] == 0.0 and np.signbit(d[5]) and d[6] == -1.0
    assert d[7] == np.inf and d[8] == -np.inf and np.isnan(d[9:]).all()


def test_e5m2_exhaustive_against_torch_and_encoder():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e5m2"):
        pytest.skip("torch has no float8_e5m2")
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode("e5m2", codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).float().double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)
    finite = np.isfinite(mine)
    back = W.to_e5m2_bits(mine[finite])
    # encode(decode(c)) is the identity on finite codes (both zeros keep their sign)
    assert np.array_equal(back, codes[finite])
    # saturation and ties to even
    assert W.to_e5m2_bits(np.array([1e9, -1e9]))[0] == 0x7B
    assert W.to_e5m2_bits(np.array([1.125]))[0] == 0x3C  # halfway 1 .. 1.25 -> even mantissa 0
    assert W.to_e5m2_bits(np.array([1.375]))[0] == 0x3E  # halfway 1.25 .. 1.5 -> mantissa 2


def test_e2m1_table_packing_and_encoder():
    codes = np.arange(16, dtype=np.uint8)
    packed = W.pack_e2m1(codes.reshape(1, 16))
    assert packed.shape == (1, 8) and packed[0, 0] == 0x10 and packed[0, 7] == 0xFE
    d = oracle.decode("e2m1", packed)[0]
    expect = E2M1_TABLE + [-v for v in E2M1_TABLE]
    assert np.array_equal(d, np.array(expect)) and np.signbit(d[8])
    # encoder: nearest, ties to even code, saturation
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.3, 100.0])
    q = W.to_e2m1_codes(x)
    assert list(q) == [0, 2, 2, 4, 4, 6, 6, 7, 0x9, 7]
    assert np.array_equal(W.to_e2m1_codes(np.array(E2M1_TABLE)), np.arange(8))


# The 6-bit types of the OCP MX v1.0 specification as value grids: each binade of the format,
# from the subnormals up, with its step (a description independent of the bit fields).
#   E2M3: [0, 1) in steps of 1/8 (subnormals 0 .. 7/8), then [1, 2) by 1/8, [2, 4) by 1/4,
#         [4, 8) by 1/2 up to 7.5.
#   E3M2: [0, 1/4) by 1/16, [1/4, 1/2) by 1/16, [1/2, 1) by 1/8, [1, 2) by 1/4, [2, 4) by 1/2,
#         [4, 8) by 1, [8, 16) by 2, [16, 32) by 4 up to 28.
def _grid(parts):
    out = []
    for lo, n, step in parts:
        out += [Fraction(lo) + i * Fraction(step) for i in range(n)]
    return [float(v) for v in out]


E2M3_GRID = _grid([(0, 8, Fraction(1, 8)), (1, 8, Fraction(1, 8)), (2, 8, Fraction(1, 4)),
                   (4, 8, Fraction(1, 2))])
E3M2_GRID = _grid([(0, 4, Fraction(1, 16)), (Fraction(1, 4), 4, Fraction(1, 16)),
                   (Fraction(1, 2), 4, Fraction(1, 8)), (1, 4, Fraction(1, 4)),
                   (2, 4, Fraction(1, 2)), (4, 4, 1), (8, 4, 2), (16, 4, 4)])


@pytest.mark.parametrize("elem,grid,top", [("e2m3", E2M3_GRID, 7.5), ("e3m2", E3M2_GRID, 28.0)])
def test_fp6_tables_packing_and_encoder(elem, grid, top):
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64)
    packed = W.pack_fp6(codes)
    assert packed.shape == (1, 48)
    d = oracle.decode(elem, packed)[0]
    assert list(d[:32]) == grid and d[31] == top
    assert list(d[32:]) == [-v for v in grid] and np.signbit(d[32])
    # encode(decode(c)) is the identity on the non-negative codes; nearest with ties to the
    # even code; saturation at the largest finite value
    assert np.array_equal(W.to_fp6_codes(np.array(grid), elem), np.arange(32))
    mid = (np.array(grid[8:12]) + np.array(grid[9:13])) / 2  # halfway between codes 8..12
    assert list(W.to_fp6_codes(mid, elem)) == [8, 10, 10, 12]
    assert W.to_fp6_codes(np.array([1e6, -1e6]), elem).tolist() == [31, 63]


def test_fp6_packing_by_hand():
    """Codes 1, 2, 3, 4 packed: 1 | 2 << 6 | 3 << 12 | 4 << 18 = 0x103081, bytes 81 30 10."""
    packed = W.pack_fp6(np.array([[1, 2, 3, 4]], dtype=np.uint8))
    assert packed.tolist() == [[0x81, 0x30, 0x10]]
    assert oracle.decode("e2m3", packed).tolist() == [[0.125, 0.25, 0.375, 0.5]]
    # an element that straddles a byte boundary: code 63 in slot 1 (bits 6..11)
    p2 = W.pack_fp6(np.array([[0, 63, 0, 0]], dtype=np.uint8))
    assert p2.tolist() == [[0xC0, 0x0F, 0x00]]
    assert oracle.decode("e3m2", p2).tolist() == [[0.0, -28.0, 0.0, 0.0]]


def test_e8m0_scales():
    d = oracle.decode_e8m0(np.array([127, 128, 126, 0, 254, 255], dtype=np.uint8))
    assert d[0] == 1.0 and d[1] == 2.0 and d[2] == 0.5
    assert d[3] == 2.0 ** -127 and d[4] == 2.0 ** 127 and np.isnan(d[5])


def _rand_elems(rng, dtype, shape):
    """Random values of an element format, chosen from values the format defines, with
    magnitudes in [1/4, 8] for the 8-bit formats so that (with block scales within 2^+-8) every
    partial sum of the brute-force shapes is exact in float64."""
    if dtype == "e2m1":
        mags = np.array(E2M1_TABLE)
    elif dtype in W.FP6:
        mags = np.array(E2M3_GRID if dtype == "e2m3" else E3M2_GRID)
    else:
        mags = W._E4M3_MAG if dtype == "e4m3" else W._E5M2_MAG
        mags = mags[(mags >= 0.25) & (mags <= 8.0)]
    v = rng.choice(mags, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    return v


def _encode_elems(v, dtype):
    return W.pack_e2m1(W.to_e2m1_codes(v)) if dtype == "e2m1" else W.encode(v, dtype)


@pytest.mark.parametrize("ta,tb,elem", [(False, False, "e4m3"), (True, True, "e5m2"),
                                        (False, True, "e2m1"), (True, False, "e4m3"),
                                        (False, True, "e2m3"), (False, True, "e3m2")])
def test_mx_brute_force_exact(ta, tb, elem):
    """MX block scaling against exact rationals: op(A)[i,k] = v * 2^(sa[i,k//32]-127)."""
    rng = np.random.default_rng(7)
    for M, N, K in [(1, 1, 32), (2, 3, 64), (3, 2, 96)]:
        a = _rand_elems(rng, elem, (M, K))
        b = _rand_elems(rng, elem, (K, N))
        sa = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
        sb = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
        A = _encode_elems(a.T if ta else a, elem)
        B = _encode_elems(b.T if tb else b, elem)
        prob = W.Problem(name="t", M=M, N=N, K=K, trans_a=ta, trans_b=tb, alpha=1.0, beta=0.0,
                         a_type=elem, b_type=elem, c_type="f32", epilogue=0, A=A, B=B,
                         C=np.zeros((M, N), np.float32), bias=None, sa_blk=sa, sb_blk=sb)
        Cref, D = oracle.gemm(prob)
        for i, j in itertools.product(range(M), range(N)):
            terms = [Fraction(a[i, k]) * Fraction(2) ** (int(sa[i, k // 32]) - 127) *
                     Fraction(b[k, j]) * Fraction(2) ** (int(sb[j, k // 32]) - 127)
                     for k in range(K)]
            assert Cref[i, j] == float(sum(terms, Fraction(0)))
            assert D[i, j] == float(sum((abs(t) for t in terms), Fraction(0)))


def test_mx_unit_scales_reduce_to_plain_gemm():
    """All block scales 2^0: the MX result equals the per-tensor product on the same bytes."""
    rng = np.random.default_rng(8)
    M, N, K = 5, 7, 64
    a = _rand_elems(rng, "e4m3", (M, K))
    b = _rand_elems(rng, "e4m3", (K, N))
    A, B = W.encode(a, "e4m3"), W.encode(b, "e4m3")
    common = dict(name="t", M=M, N=N, K=K, trans_a=False, trans_b=False, alpha=1.5, beta=0.0,
                  a_type="e4m3", b_type="e4m3", c_type="bf16", epilogue=0, A=A, B=B,
                  C=np.zeros((M, N), np.uint16), bias=None)
    plain = oracle.gemm(W.Problem(**common))
    mx = oracle.gemm(W.Problem(**common, sa_blk=np.full((M, 2), 127, np.uint8),
                               sb_blk=np.full((N, 2), 127, np.uint8)))
    assert np.array_equal(plain[0], mx[0]) and np.array_equal(plain[1], mx[1])


def test_mx_block_scale_moves_only_its_block():
    """Raising one block scale of row 0 by one doubles exactly that block's contribution."""
    rng = np.random.default_rng(9)
    M, N, K = 2, 3, 64
    a = _rand_elems(rng, "e5m2", (M, K))
    b = _rand_elems(rng, "e5m2", (K, N))
    sa = np.full((M, 2), 127, np.uint8)
    sb = np.full((N, 2), 127, np.uint8)
    base = dict(name="t", M=M, N=N, K=K, trans_a=False, trans_b=False, alpha=1.0, beta=0.0,
                a_type="e5m2", b_type="e5m2", c_type="f32", epilogue=0, A=W.encode(a, "e5m2"),
                B=W.encode(b, "e5m2"), C=np.zeros((M, N), np.float32), bias=None, sb_blk=sb)
    c0, _ = oracle.gemm(W.Problem(**base, sa_blk=sa))
    sa2 = sa.copy()
    sa2[0, 1] = 128
    c1, _ = oracle.gemm(W.Problem(**base, sa_blk=sa2))
    block1 = a[0, 32:] @ b[32:, :]
    assert np.allclose(c1[0] - c0[0], block1, rtol=0, atol=1e-9 * (1 + np.abs(block1).max()))
    assert np.array_equal(c1[1], c0[1])


def test_mx_quantize_recipe():
    """Block scale = 2^(floor(log2 amax) - emax); elements within the format's rounding of
    v / scale; the block maximum lands in the format's top binade (or saturates)."""
    rng = np.random.default_rng(10)
    x = rng.normal(0, 3.0, size=(4, 96))
    x[1, 32:64] = 0.0
    for elem, eps in (("e4m3", 2.0 ** -4), ("e5m2", 2.0 ** -3), ("e2m1", 2.0 ** -2),
                      ("e2m3", 2.0 ** -4), ("e3m2", 2.0 ** -3)):
        q, s = W.mx_quantize(x, elem)
        assert s.shape == (4, 3) and s[1, 1] == 127
        scale = oracle.decode_e8m0(s)
        vals = oracle.decode(elem, q) * np.repeat(scale, 32, axis=1)
        amax = np.abs(x.reshape(4, 3, 32)).max(axis=2)
        nz = amax > 0
        assert np.array_equal(scale[nz], 2.0 ** (np.floor(np.log2(amax[nz])) - W.MX_EMAX[elem]))
        # per element: one rounding (relative eps, or half the block's smallest step) after
        # clipping |v| / scale to the format's largest finite value
        top = {"e4m3": W.E4M3_MAX, "e5m2": W.E5M2_MAX, "e2m1": W.E2M1_MAX, "e2m3": W.E2M3_MAX,
               "e3m2": W.E3M2_MAX}[elem]
        sc = np.repeat(scale, 32, axis=1)
        clipped = np.sign(x) * np.minimum(np.abs(x), top * sc)
        step = sc * {"e4m3": 2.0 ** -9, "e5m2": 2.0 ** -16, "e2m1": 0.5, "e2m3": 0.125,
                     "e3m2": 0.0625}[elem]
        assert (np.abs(vals - clipped) <= np.maximum(eps * np.abs(clipped), step / 2)).all()
        # the block maximum sits in [2^emax, 2^(emax+1)) before clipping
        hi = np.abs(x.reshape(4, 3, 32)).max(axis=2)[nz] / scale[nz]
        assert ((hi >= 2.0 ** W.MX_EMAX[elem]) & (hi < 2.0 ** (W.MX_EMAX[elem] + 1))).all()
