"""Seeded synthetic inputs for the tiled GEMM  C = alpha * op(A) * op(B) + beta * C.

This module only draws random matrices and turns float64 draws into the exact bytes that a
GEMM call consumes: fp32, fp16 or bf16 words, or OCP fp8-E4M3 bytes plus one fp32 scale per
tensor.  It holds none of the GEMM arithmetic.  Both the HIP library and the CPU oracle receive
the very same bytes from here, so input quantisation error cancels when the two are compared
(the checksum gate of "Rigel" (arXiv 2606.12765), section 3: the float64 reference is built from
the exact quantised bytes the GPU consumes).

Workloads (all square sizes come from the pages' square benchmarks; the distributions and seeds
are fixed here):
  * fp32 256^3, alpha=1, beta=0, A,B ~ U[-1,1], seed 0.
  * fp32 1000^3, alpha=1.5, beta=-0.5, A,B,C_in ~ U[-1,1], seed 1; also with A stored K x M.
  * fp16 n^3 for n in {512,1024,2048,4096}, A,B ~ N(0, 0.5^2), seed 2, fp16 output.
  * bf16 n^3 + bias + erf-GELU, A ~ N(0,1), B ~ N(0,1/K), bias ~ N(0, 0.1^2) fp32, seed 3.
  * fp8-E4M3 4096^3 with per-tensor scales (max|x| -> 448) and its bf16 twin, A,B ~ N(0,1),
    seed 4, bf16 output.
  * fp8-E5M2 4096^3 (per-tensor scale max|x| -> 57344), and the OCP microscaling (MX) formats
    MXFP8 (E4M3 elements) and MXFP4 (E2M1 elements) at 4096^3: one E8M0 scale per 32
    consecutive k of each row of op(A) and each column of op(B), A,B ~ N(0,1), seed 5.
Draw order is always: logical A (M x K, row-major), then logical B (K x N), then C_in (M x N),
then bias (N).  A transposed operand is the same logical matrix stored as its transpose.
"""
from __future__ import annotations

import dataclasses
import hashlib
import json
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16", "e4m3", "e5m2", "e2m1", "e2m3", "e3m2")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3, "e5m2": 4, "e2m1": 5, "e2m3": 6,
              "e3m2": 7}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1, "e2m1": 0.5, "e2m3": 0.75,
         "e3m2": 0.75}
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8,
           "e5m2": np.uint8, "e2m1": np.uint8, "e2m3": np.uint8, "e3m2": np.uint8}
FP8 = ("e4m3", "e5m2")
FP6 = ("e2m3", "e3m2")
PACKED = ("e2m1",) + FP6  # stored several elements per byte along the row
MX_BLOCK = 32  # elements per E8M0 block scale (OCP microscaling)

EPI_NONE = 0
EPI_BIAS = 1
EPI_GELU = 2

# Output type for each supported input type.
OUT_TYPE = {"f32": "f32", "f16": "f16", "bf16": "bf16", "e4m3": "bf16", "e5m2": "bf16",
            "e2m1": "bf16", "e2m3": "bf16", "e3m2": "bf16"}


# --------------------------------------------------------------------------------------------
# Encoders: float64 draws -> storage bytes (round to nearest, ties to even).
# --------------------------------------------------------------------------------------------

def to_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> IEEE binary32, round to nearest even (numpy's cast)."""
    return np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> IEEE binary16 bit patterns, round to nearest even (numpy's cast)."""
    return np.ascontiguousarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 (RNE) -> bfloat16 bit patterns (RNE on the low 16 bits)."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((f.view(np.uint32)[nan] >> 16) | 0x0040).astype(np.uint16)
    return out


def _e4m3_magnitudes() -> np.ndarray:
    """Magnitudes of the 127 finite non-negative OCP E4M3 codes 0x00..0x7E, increasing."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
    return vals


_E4M3_MAG = _e4m3_magnitudes()
E4M3_MAX = 448.0


def to_e4m3_bits(y: np.ndarray) -> np.ndarray:
    """float64 -> OCP E4M3 bytes: nearest code, ties to the even code, saturating at +-448.

    NaN maps to 0x7F.  Values beyond +-448 saturate instead of producing NaN, so that a tensor
    scaled to max|x| = 448 never rounds its maximum into the NaN code.
    """
    y = np.ascontiguousarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_MAG, mag, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _E4M3_MAG[hi] - mag
    d_lo = mag - _E4M3_MAG[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((lo & 1) == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code |= (np.signbit(y).astype(np.uint8) << 7)
    code[np.isnan(y)] = 0x7F
    return code


def e4m3_scale(x: np.ndarray) -> np.float32:
    """Per-tensor dequantisation scale: fp32(max|x| / 448), or 1 for an all-zero tensor."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    return np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)


def _nearest_code(y: np.ndarray, mags: np.ndarray, sign_shift: int) -> np.ndarray:
    """Nearest code among increasing non-negative magnitudes `mags` (code = index), ties to
    the even code, saturating at the largest; the sign goes to bit `sign_shift`."""
    mag = np.minimum(np.abs(y), mags[-1])
    top = mags.size - 1
    hi = np.clip(np.searchsorted(mags, mag, side="left"), 0, top)
    lo = np.clip(hi - 1, 0, top)
    d_hi = mags[hi] - mag
    d_lo = mag - mags[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((lo & 1) == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << sign_shift)


def _e5m2_magnitudes() -> np.ndarray:
    """Magnitudes of the 124 finite non-negative OCP E5M2 codes 0x00..0x7B, increasing."""
    vals = np.empty(124, dtype=np.float64)
    for code in range(124):
        e, m = code >> 2, code & 3
        vals[code] = m * 2.0 ** -16 if e == 0 else (4 + m) * 2.0 ** (e - 17)
    return vals


_E5M2_MAG = _e5m2_magnitudes()
E5M2_MAX = 57344.0


def to_e5m2_bits(y: np.ndarray) -> np.ndarray:
    """float64 -> OCP E5M2 bytes: nearest code, ties to even, saturating at +-57344; NaN -> 0x7F."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    code = _nearest_code(y, _E5M2_MAG, 7)
    code[np.isnan(y)] = 0x7F
    return code


# OCP E2M1 magnitudes for codes 0..7 (exponent bias 1, one mantissa bit; no inf or NaN).
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def to_e2m1_codes(y: np.ndarray) -> np.ndarray:
    """float64 -> OCP E2M1 4-bit codes (one per uint8): nearest, ties to even, saturating at
    +-6.  NaN has no code; it must not occur."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError("E2M1 has no NaN")
    return _nearest_code(y, _E2M1_MAG, 3)


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes two per byte along the last axis: element 2i in the low nibble of
    byte i, element 2i+1 in the high nibble.  The last axis must be even."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("E2M1 rows must hold an even number of elements")
    return np.ascontiguousarray((c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4))


def _fp6_magnitudes(mbits: int, bias: int) -> np.ndarray:
    """Magnitudes of the 32 non-negative codes of an OCP 6-bit type with `mbits` mantissa bits
    and exponent bias `bias` (no infinities or NaN), increasing with the code."""
    vals = np.empty(32, dtype=np.float64)
    for code in range(32):
        e, m = code >> mbits, code & ((1 << mbits) - 1)
        vals[code] = (m * 2.0 ** (1 - bias - mbits) if e == 0
                      else ((1 << mbits) + m) * 2.0 ** (e - bias - mbits))
    return vals


# OCP MX v1.0 6-bit types: E2M3 (bias 1, largest 7.5) and E3M2 (bias 3, largest 28).
_FP6_MAG = {"e2m3": _fp6_magnitudes(3, 1), "e3m2": _fp6_magnitudes(2, 3)}
E2M3_MAX = 7.5
E3M2_MAX = 28.0


def to_fp6_codes(y: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> 6-bit codes of `dtype` (one per uint8, sign in bit 5): nearest, ties to even,
    saturating.  NaN has no code; it must not occur."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError(f"{dtype} has no NaN")
    return _nearest_code(y, _FP6_MAG[dtype], 5)


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """Pack 6-bit codes four per three bytes along the last axis: element i occupies bits
    6i .. 6i+5 of the row's byte string read as one little-endian integer.  The last axis must
    be a multiple of 4."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).astype(np.uint32) & 63
    if c.shape[-1] % 4:
        raise ValueError("6-bit rows must hold a multiple of 4 elements")
    w = c[..., 0::4] | (c[..., 1::4] << 6) | (c[..., 2::4] << 12) | (c[..., 3::4] << 18)
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 4 * 3,), dtype=np.uint8)
    out[..., 0::3] = w & 255
    out[..., 1::3] = (w >> 8) & 255
    out[..., 2::3] = (w >> 16) & 255
    return out


# Largest binade of each MX element format (2^emax <= max finite < 2^(emax+1)).
MX_EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2, "e2m3": 2, "e3m2": 4}


def mx_quantize(x: np.ndarray, elem: str):
    """OCP microscaling quantisation of a rows x K float64 matrix (K a multiple of 32): every
    run of 32 consecutive values in a row shares the E8M0 scale 2^X with
    X = floor(log2(max|v|)) - emax(elem) (X clamped to [-127, 127]; an all-zero block takes
    X = 0); the elements are v / 2^X rounded to `elem`, saturating.
    Returns (element storage, rows x K (K/2 bytes packed for e2m1, 3K/4 for the 6-bit types),
    uint8 scales rows x K/32)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blk = x.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blk), axis=2)
    X = np.zeros_like(amax, dtype=np.int64)
    nz = amax > 0
    X[nz] = np.floor(np.log2(amax[nz])).astype(np.int64) - MX_EMAX[elem]
    X = np.clip(X, -127, 127)
    scaled = (blk / np.ldexp(1.0, X)[..., None]).reshape(rows, K)
    if elem == "e4m3":
        q = to_e4m3_bits(scaled)
    elif elem == "e5m2":
        q = to_e5m2_bits(scaled)
    elif elem == "e2m1":
        q = pack_e2m1(to_e2m1_codes(scaled))
    elif elem in FP6:
        q = pack_fp6(to_fp6_codes(scaled, elem))
    else:
        raise ValueError(f"no MX element format {elem!r}")
    return q, (X + 127).astype(np.uint8)


def encode(x: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Encode float64 values to the storage of `dtype` (fp8 types encode x / scale; E2M1 packs
    two codes per byte along the last axis)."""
    if dtype == "f32":
        return to_f32(x)
    if dtype == "f16":
        return to_f16_bits(x)
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "e4m3":
        return to_e4m3_bits(np.asarray(x, dtype=np.float64) / float(scale))
    if dtype == "e5m2":
        return to_e5m2_bits(np.asarray(x, dtype=np.float64) / float(scale))
    if dtype == "e2m1":
        return pack_e2m1(to_e2m1_codes(np.asarray(x, dtype=np.float64) / float(scale)))
    if dtype in FP6:
        return pack_fp6(to_fp6_codes(np.asarray(x, dtype=np.float64) / float(scale), dtype))
    raise ValueError(f"unknown dtype {dtype!r}")


def fp8_scale(x: np.ndarray, dtype: str) -> np.float32:
    """Per-tensor dequantisation scale: fp32(max|x| / max finite of `dtype`), 1 if all zero."""
    top = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX, "e2m1": E2M1_MAX, "e2m3": E2M3_MAX,
           "e3m2": E3M2_MAX}[dtype]
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    return np.float32(amax / top) if amax > 0 else np.float32(1.0)


# --------------------------------------------------------------------------------------------
# Problems
# --------------------------------------------------------------------------------------------

@dataclasses.dataclass
class Problem:
    """One GEMM call's inputs, as storage bytes, plus the call's scalars.

    A is stored M x K (row-major, lda = K) or, with trans_a, K x M (lda = M); B is stored K x N
    (ldb = N) or, with trans_b, N x K (ldb = K).  C holds C_in in the output type (all zero
    when beta == 0) and is M x N with ldc = N.
    """
    name: str
    M: int
    N: int
    K: int
    trans_a: bool
    trans_b: bool
    alpha: float
    beta: float
    a_type: str
    b_type: str
    c_type: str
    epilogue: int
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    bias: Optional[np.ndarray]
    scale_a: float = 1.0
    scale_b: float = 1.0
    recipe: dict = dataclasses.field(default_factory=dict)
    # OCP MX block scales (E8M0 bytes): sa_blk[i, k // 32] for row i of op(A), sb_blk[j, k // 32]
    # for column j of op(B); None for per-tensor scaling.
    sa_blk: Optional[np.ndarray] = None
    sb_blk: Optional[np.ndarray] = None

    @property
    def mx(self) -> bool:
        return self.sa_blk is not None

    @property
    def ldsa(self) -> int:
        return self.sa_blk.shape[1] if self.sa_blk is not None else 0

    @property
    def ldsb(self) -> int:
        return self.sb_blk.shape[1] if self.sb_blk is not None else 0

    @property
    def lda(self) -> int:
        return self.M if self.trans_a else self.K

    @property
    def ldb(self) -> int:
        return self.K if self.trans_b else self.N

    @property
    def ldc(self) -> int:
        return self.N

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def recipe_hash(self) -> str:
        blob = json.dumps(self.recipe, sort_keys=True).encode()
        return hashlib.sha256(blob).hexdigest()[:16]


def _draw(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind, p = dist
    if kind == "uniform":
        lo, hi = p
        return rng.uniform(lo, hi, size=shape)
    if kind == "normal":
        return rng.normal(0.0, p, size=shape)
    if kind == "int":
        lo, hi = p
        return rng.integers(lo, hi + 1, size=shape).astype(np.float64)
    raise ValueError(kind)


def make_problem(M: int, N: int, K: int, *, a_type: str = "f32", c_type: Optional[str] = None,
                 b_type: Optional[str] = None, trans_a: bool = False, trans_b: bool = False,
                 alpha: float = 1.0, beta: float = 0.0, epilogue: int = EPI_NONE, seed: int = 0,
                 dist_a=("uniform", (-1.0, 1.0)), dist_b=("uniform", (-1.0, 1.0)),
                 dist_c=("uniform", (-1.0, 1.0)), bias_std: float = 0.1,
                 fp8_scaled: bool = True, mx: bool = False, name: str = "") -> Problem:
    """Draw a seeded problem.  `dist_*` is ("uniform", (lo, hi)), ("normal", std) or
    ("int", (lo, hi)).  For fp8 inputs each operand gets its own per-tensor scale when
    `fp8_scaled`, else scale 1 (the draws must then already be representable).  With `mx`
    (8-bit or E2M1 inputs) the operands are quantised in OCP MX blocks of 32 along K instead,
    and the per-tensor scales are 1.  `b_type` defaults to `a_type`."""
    b_type = b_type or a_type
    c_type = c_type or OUT_TYPE[a_type]
    rng = np.random.default_rng(seed)
    a = _draw(rng, (M, K), dist_a)
    b = _draw(rng, (K, N), dist_b)
    c_in = _draw(rng, (M, N), dist_c) if beta != 0.0 else None
    bias = (rng.normal(0.0, bias_std, size=N).astype(np.float32)
            if epilogue & EPI_BIAS else None)
    sa = sb = np.float32(1.0)
    sa_blk = sb_blk = None
    if mx:
        # quantise op(A) by rows and op(B) by columns (rows of B^T), then store as asked
        qa, sa_blk = mx_quantize(a, a_type)
        qb, sb_blk = mx_quantize(b.T, b_type)
        if a_type in PACKED or b_type in PACKED:
            if trans_a or not trans_b:
                raise ValueError("packed MX operands are stored K-contiguous (A M x K, B N x K)")
            A, B = qa, qb
        else:
            A = np.ascontiguousarray(qa.T if trans_a else qa)
            B = np.ascontiguousarray(qb if trans_b else qb.T)
    else:
        if a_type in FP8 + FP6 and fp8_scaled:
            sa = fp8_scale(a, a_type)
        if b_type in FP8 + FP6 and fp8_scaled:
            sb = fp8_scale(b, b_type)
        a_st = np.ascontiguousarray(a.T if trans_a else a)
        b_st = np.ascontiguousarray(b.T if trans_b else b)
        A = encode(a_st, a_type, float(sa))
        B = encode(b_st, b_type, float(sb))
    C = (encode(c_in, c_type) if c_in is not None
         else np.zeros((M, N), dtype=STORAGE[c_type]))
    recipe = dict(name=name, M=M, N=N, K=K, a_type=a_type, c_type=c_type, trans_a=trans_a,
                  trans_b=trans_b, alpha=alpha, beta=beta, epilogue=epilogue, seed=seed,
                  dist_a=list(map(str, dist_a)), dist_b=list(map(str, dist_b)),
                  dist_c=list(map(str, dist_c)), bias_std=bias_std, fp8_scaled=fp8_scaled,
                  b_type=b_type, mx=mx, rng="numpy.default_rng(PCG64)", order="A,B,C_in,bias")
    return Problem(name=name or f"{a_type}_{M}x{N}x{K}", M=M, N=N, K=K, trans_a=trans_a,
                   trans_b=trans_b, alpha=float(alpha), beta=float(beta), a_type=a_type,
                   b_type=b_type, c_type=c_type, epilogue=epilogue, A=A, B=B, C=C, bias=bias,
                   scale_a=float(sa), scale_b=float(sb), recipe=recipe, sa_blk=sa_blk,
                   sb_blk=sb_blk)


# The named workloads.

def fp32_256() -> Problem:
    """fp32 C = A*B, 256^3, row-major, alpha=1, beta=0, U[-1,1], seed 0."""
    return make_problem(256, 256, 256, a_type="f32", seed=0, name="fp32_256")


def fp32_1000_ragged(trans_a: bool = False) -> Problem:
    """fp32 C = 1.5*A*B - 0.5*C, 1000^3 (ragged against every tile), U[-1,1], seed 1."""
    return make_problem(1000, 1000, 1000, a_type="f32", trans_a=trans_a, alpha=1.5, beta=-0.5,
                        seed=1, name="fp32_1000_" + ("tn" if trans_a else "nn"))


def fp16_square(n: int) -> Problem:
    """fp16 C = A*B, n^3, A,B ~ N(0, 0.5^2) rounded to fp16, fp16 output, seed 2."""
    return make_problem(n, n, n, a_type="f16", seed=2, dist_a=("normal", 0.5),
                        dist_b=("normal", 0.5), name=f"fp16_{n}")


def bf16_bias_gelu(n: int, epilogue: int = EPI_BIAS | EPI_GELU) -> Problem:
    """bf16 C = GELU(A*B + bias), n^3, A ~ N(0,1), B ~ N(0,1/K), bias ~ N(0,0.1^2), seed 3.

    The bias is drawn for every epilogue value, so the unfused run (epilogue 0 in the GEMM,
    then a separate bias+GELU pass) sees the same bias as the fused run."""
    p = make_problem(n, n, n, a_type="bf16", seed=3, dist_a=("normal", 1.0),
                     dist_b=("normal", 1.0 / np.sqrt(n)), epilogue=EPI_BIAS | EPI_GELU,
                     name=f"bf16_bias_gelu_{n}")
    p.epilogue = epilogue
    return p


def fp8_4096(n: int = 4096) -> Problem:
    """fp8-E4M3 C = (sa*sb)*A*B, n^3, A,B ~ N(0,1), per-tensor scale max|x| -> 448, bf16 out."""
    return make_problem(n, n, n, a_type="e4m3", c_type="bf16", seed=4, dist_a=("normal", 1.0),
                        dist_b=("normal", 1.0), name=f"fp8_{n}")


def bf16_twin_of_fp8(n: int = 4096) -> Problem:
    """The same float64 draws as fp8_4096, rounded to bf16 instead, bf16 out, no epilogue."""
    return make_problem(n, n, n, a_type="bf16", c_type="bf16", seed=4, dist_a=("normal", 1.0),
                        dist_b=("normal", 1.0), name=f"bf16_{n}")


def e5m2_4096(n: int = 4096) -> Problem:
    """fp8-E5M2 C = (sa*sb)*A*B, n^3, A,B ~ N(0,1), per-tensor scale max|x| -> 57344, bf16 out."""
    return make_problem(n, n, n, a_type="e5m2", c_type="bf16", seed=5, dist_a=("normal", 1.0),
                        dist_b=("normal", 1.0), name=f"e5m2_{n}")


def mxfp8_4096(n: int = 4096) -> Problem:
    """MXFP8 (E4M3 elements, E8M0 scale per 32 k) C = A*B, n^3, row-major A and B,
    A,B ~ N(0,1), bf16 out, seed 5."""
    return make_problem(n, n, n, a_type="e4m3", c_type="bf16", seed=5, mx=True,
                        dist_a=("normal", 1.0), dist_b=("normal", 1.0), name=f"mxfp8_{n}")


def mxfp6_4096(n: int = 4096, elem: str = "e2m3") -> Problem:
    """MXFP6 (E2M3 elements packed four per three bytes, E8M0 scale per 32 k) C = A*B, n^3,
    A stored M x K and B stored N x K, A,B ~ N(0,1), bf16 out, seed 8."""
    return make_problem(n, n, n, a_type=elem, c_type="bf16", trans_b=True, seed=8, mx=True,
                        dist_a=("normal", 1.0), dist_b=("normal", 1.0), name=f"mxfp6_{elem}_{n}")


def mxfp4_4096(n: int = 4096) -> Problem:
    """MXFP4 (E2M1 elements packed two per byte, E8M0 scale per 32 k) C = A*B, n^3, A stored
    M x K and B stored N x K (both K-contiguous, as packed operands are), A,B ~ N(0,1), bf16
    out, seed 5."""
    return make_problem(n, n, n, a_type="e2m1", c_type="bf16", trans_b=True, seed=5, mx=True,
                        dist_a=("normal", 1.0), dist_b=("normal", 1.0), name=f"mxfp4_{n}")


# --------------------------------------------------------------------------------------------
# Group-quantized weights (C = X W^T with W stored as affine codes; see oracle.c for the
# definition): the decode matrix-vector product and the prefill matrix product
# --------------------------------------------------------------------------------------------

@dataclasses.dataclass
class QProblem:
    """Activations X (M x K, row-major, ldx = K, storage of x_type), codes Wq (N rows of
    K * bits / 8 bytes, 4-bit codes two per byte with the low nibble first), scales and offsets
    (N x K / group, storage of x_type) such that w[j, k] = s[j, k // G] * q[j, k] + o[j, k // G];
    C (M x N, x_type) holds C_in (zero when beta == 0)."""
    name: str
    M: int
    N: int
    K: int
    bits: int
    group: int
    x_type: str
    alpha: float
    beta: float
    epilogue: int
    X: np.ndarray
    Wq: np.ndarray
    scales: np.ndarray
    offsets: np.ndarray
    C: np.ndarray
    bias: Optional[np.ndarray]
    recipe: dict = dataclasses.field(default_factory=dict)

    @property
    def ldx(self) -> int:
        return self.K

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def weight_bytes(self) -> int:
        return int(self.Wq.nbytes + self.scales.nbytes + self.offsets.nbytes)


def q_codes(w: np.ndarray, bits: int, group: int, x_type: str):
    """Affine group quantization of a rows x K float64 matrix, one (scale, offset) per `group`
    consecutive values of a row: offset o = min, scale s = (max - min) / (2^bits - 1), both
    rounded to x_type; codes q = round((w - o) / s) clipped to [0, 2^bits - 1] (q = 0 where
    s = 0).  Returns (uint8 codes rows x K, scales, offsets as x_type storage)."""
    rows, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if K == 0:
        z = np.zeros((rows, 0), dtype=STORAGE[x_type])
        return np.zeros((rows, 0), dtype=np.uint8), z, z.copy()
    blk = w.reshape(rows, K // group, group)
    lo, hi = blk.min(axis=2), blk.max(axis=2)
    top = (1 << bits) - 1
    S = encode((hi - lo) / top, x_type)
    O = encode(lo, x_type)
    dec = (lambda v: v.view(np.float16).astype(np.float64)) if x_type == "f16" else \
          (lambda v: (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    s, o = dec(S), dec(O)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[..., None] > 0, np.rint((blk - o[..., None]) / s[..., None]), 0.0)
    q = np.clip(q, 0, top).astype(np.uint8).reshape(rows, K)
    return q, S, O


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Store codes: 8-bit one per byte; 4-bit two per byte along the row, low nibble first."""
    if bits == 8:
        return np.ascontiguousarray(q, dtype=np.uint8)
    if bits == 4:
        return pack_e2m1(q)
    raise ValueError(f"bits must be 4 or 8, not {bits}")


def make_qproblem(M: int, N: int, K: int, *, bits: int = 4, group: int = 64,
                  x_type: str = "bf16", alpha: float = 1.0, beta: float = 0.0,
                  epilogue: int = EPI_NONE, seed: int = 0, x_std: float = 1.0,
                  w_std: Optional[float] = None, bias_std: float = 0.1,
                  name: str = "") -> QProblem:
    """Seeded problem: X ~ N(0, x_std^2), W ~ N(0, w_std^2) (default 1/K) quantized by q_codes,
    C_in ~ U[-1, 1] when beta != 0, bias ~ N(0, bias_std^2) with the BIAS epilogue.  Draw
    order: X, W, C_in, bias."""
    if x_type not in ("bf16", "f16"):
        raise ValueError("activations are bf16 or f16")
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, x_std, size=(M, K))
    w = rng.normal(0.0, w_std if w_std is not None else 1.0 / np.sqrt(max(K, 1)), size=(N, K))
    c_in = rng.uniform(-1.0, 1.0, size=(M, N)) if beta != 0.0 else None
    bias = rng.normal(0.0, bias_std, size=N).astype(np.float32) if epilogue & EPI_BIAS else None
    q, S, O = q_codes(w, bits, group, x_type)
    C = encode(c_in, x_type) if c_in is not None else np.zeros((M, N), dtype=STORAGE[x_type])
    recipe = dict(name=name, M=M, N=N, K=K, bits=bits, group=group, x_type=x_type, alpha=alpha,
                  beta=beta, epilogue=epilogue, seed=seed, x_std=x_std, w_std=w_std,
                  bias_std=bias_std, rng="numpy.default_rng(PCG64)", order="X,W,C_in,bias")
    return QProblem(name=name or f"q{bits}_{M}x{N}x{K}", M=M, N=N, K=K, bits=bits, group=group,
                    x_type=x_type, alpha=float(alpha), beta=float(beta), epilogue=epilogue,
                    X=encode(x, x_type), Wq=pack_codes(q, bits), scales=S, offsets=O, C=C,
                    bias=bias, recipe=recipe)


def q4_decode(N: int = 28672, K: int = 8192, seed: int = 6) -> QProblem:
    """Decode step of a large-model MLP projection: one token (M = 1), 4-bit weights in groups
    of 64, bf16 activations and output.  N x K = 28672 x 8192 is the up-projection shape of the
    70B-class open models: 117 MiB of codes and 7.3 MiB of scales and offsets per matrix."""
    return make_qproblem(1, N, K, bits=4, group=64, seed=seed, name=f"q4_decode_{N}x{K}")


def q4_prefill(n: int = 4096, seed: int = 7) -> QProblem:
    """Prefill: M = N = K = n, 4-bit weights in groups of 64, bf16 activations and output."""
    return make_qproblem(n, n, n, bits=4, group=64, seed=seed, name=f"q4_prefill_{n}")
