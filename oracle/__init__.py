"""CPU oracle for the tiled GEMM: a float64 triple loop over the exact input bytes.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  It shares no code with the HIP library and imports nothing
from it.  The arithmetic lives in oracle.c (plain C, gcc -O3 -fopenmp -ffp-contract=off); this
module only marshals numpy arrays into it.  See oracle.c for the definition that is computed and
the passages of the pages it follows.

Parity pins (tests/test_oracle.py): exact brute force with fractions.Fraction on every shape in
{1..4}^3, identity and permutation matrices, rank-1 closed forms, alpha/beta linearity,
A*B == (B^T A^T)^T, an exhaustive OCP E4M3 table, bf16 ties-to-even, closed-form GELU values, and
a numpy float64 matmul cross-check, exhaustive OCP E5M2 / E2M1 / E2M3 / E3M2 / E8M0 tables,
6-bit packing, exact block-scaled (MX) brute force, and for the group-quantized product (tests/test_oracle_q.py)
exact brute force, the unit-scale reduction to the plain product, nibble order, group
locality and offset-only closed forms.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

TYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3, "e5m2": 4, "e2m1": 5, "e2m3": 6, "e3m2": 7}
# Packed types: (elements, bytes) per packing unit along a row.
PACKED = {"e2m1": (2, 1), "e2m3": (4, 3), "e3m2": (4, 3)}
EPI_BIAS = 1
EPI_GELU = 2

_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_dbl = ctypes.c_double
_vp = ctypes.c_void_p
_PROBLEM = [_i64, _i64, _i64, _int, _int, _dbl, _vp, _i64, _dbl, _vp, _i64, _dbl, _dbl, _vp,
            _i64, _int, _int, _int, ctypes.c_uint, _vp]


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_decode.argtypes = [_int, _vp, _i64, _vp]
        L.oracle_decode.restype = _int
        L.oracle_gelu.argtypes = [_dbl]
        L.oracle_gelu.restype = _dbl
        L.oracle_gemm.argtypes = _PROBLEM + [_vp, _vp]
        L.oracle_gemm.restype = _int
        L.oracle_gemm_rows.argtypes = _PROBLEM + [_i64, _i64, _vp, _vp]
        L.oracle_gemm_rows.restype = _int
        L.oracle_gemm_points.argtypes = _PROBLEM + [_i64, _vp, _vp, _vp, _vp]
        L.oracle_gemm_points.restype = _int
        _MX = [_vp, _i64, _vp, _i64]
        L.oracle_decode_e8m0.argtypes = [_vp, _i64, _vp]
        L.oracle_decode_e8m0.restype = _int
        L.oracle_gemm_mx.argtypes = _PROBLEM + _MX + [_vp, _vp]
        L.oracle_gemm_mx.restype = _int
        L.oracle_gemm_mx_points.argtypes = _PROBLEM + _MX + [_i64, _vp, _vp, _vp, _vp]
        L.oracle_gemm_mx_points.restype = _int
        _Q = [_i64, _i64, _i64, _dbl, _vp, _i64, _int, _vp, _i64, _int, _i64, _vp, _vp, _i64,
              _int, _dbl, _vp, _i64, _int, ctypes.c_uint, _vp]
        L.oracle_qgemm.argtypes = _Q + [_vp, _vp]
        L.oracle_qgemm.restype = _int
        L.oracle_qgemm_points.argtypes = _Q + [_i64, _vp, _vp, _vp, _vp]
        L.oracle_qgemm_points.restype = _int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = _int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(dtype: str, stored: np.ndarray) -> np.ndarray:
    """Decode stored words/bytes of `dtype` to float64 with the oracle's own decoders (E2M1:
    two elements per byte along the last axis, low nibble first; E2M3 / E3M2: four elements per
    three bytes along the last axis, element i at bits 6i of the little-endian byte string)."""
    a = np.ascontiguousarray(stored)
    if dtype in PACKED:
        e, b = PACKED[dtype]
        if a.shape[-1] % b:
            raise ValueError(f"{dtype}: last axis of {a.shape[-1]} bytes is not whole units")
        n = a.size // b * e
        shape = a.shape[:-1] + (a.shape[-1] // b * e,)
    else:
        n, shape = a.size, a.shape
    out = np.empty(shape, dtype=np.float64)
    rc = lib().oracle_decode(TYPE_CODE[dtype], _ptr(a), n, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_decode({dtype}) failed: {rc}")
    return out


def decode_e8m0(stored: np.ndarray) -> np.ndarray:
    """Decode E8M0 block-scale bytes to float64 (2^(e-127), NaN for 255)."""
    a = np.ascontiguousarray(stored, dtype=np.uint8)
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_decode_e8m0(_ptr(a), a.size, _ptr(out))
    return out


def gelu(t: float) -> float:
    return lib().oracle_gelu(float(t))


def _args(M, N, K, trans_a, trans_b, alpha, A, lda, scale_a, B, ldb, scale_b, beta, C, ldc,
          a_type, b_type, c_type, epilogue, bias):
    return (M, N, K, int(bool(trans_a)), int(bool(trans_b)), float(alpha), _ptr(A), lda,
            float(scale_a), _ptr(B), ldb, float(scale_b), float(beta),
            _ptr(C) if beta != 0.0 else None, ldc, TYPE_CODE[a_type], TYPE_CODE[b_type],
            TYPE_CODE[c_type], int(epilogue), _ptr(bias))


def _problem_args(p):
    A = np.ascontiguousarray(p.A)
    B = np.ascontiguousarray(p.B)
    C = np.ascontiguousarray(p.C)
    bias = None if p.bias is None else np.ascontiguousarray(p.bias, dtype=np.float32)
    keep = (A, B, C, bias)
    return keep, _args(p.M, p.N, p.K, p.trans_a, p.trans_b, p.alpha, A, p.lda, p.scale_a, B,
                       p.ldb, p.scale_b, p.beta, C, p.ldc, p.a_type, p.b_type, p.c_type,
                       p.epilogue, bias)


def _mx_args(p):
    """(keep, args) for the block scales of an MX problem (fields sa_blk, sb_blk)."""
    sa = np.ascontiguousarray(p.sa_blk, dtype=np.uint8)
    sb = np.ascontiguousarray(p.sb_blk, dtype=np.uint8)
    return (sa, sb), (_ptr(sa), sa.shape[1], _ptr(sb), sb.shape[1])


def gemm(p) -> Tuple[np.ndarray, np.ndarray]:
    """Full reference (Cref, D), each M x N float64, for a problem with the fields of
    workloads.Problem (M, N, K, trans_a, trans_b, alpha, beta, a_type, b_type, c_type,
    epilogue, A, B, C, bias, scale_a, scale_b, lda, ldb, ldc)."""
    keep, args = _problem_args(p)
    Cref = np.empty((p.M, p.N), dtype=np.float64)
    D = np.empty((p.M, p.N), dtype=np.float64)
    if getattr(p, "sa_blk", None) is not None:
        keep2, mx = _mx_args(p)
        rc = lib().oracle_gemm_mx(*args, *mx, _ptr(Cref), _ptr(D))
        del keep2
    else:
        rc = lib().oracle_gemm(*args, _ptr(Cref), _ptr(D))
    del keep
    if rc != 0:
        raise ValueError(f"oracle_gemm failed: {rc}")
    return Cref, D


def gemm_raw(M, N, K, trans_a, trans_b, alpha, A, lda, scale_a, B, ldb, scale_b, beta, C, ldc,
             a_type, b_type, c_type, epilogue=0, bias=None) -> Tuple[np.ndarray, np.ndarray]:
    """(Cref, D) for explicit BLAS-style arguments, including leading dimensions larger than
    the logical ones.  A, B, C are flat or 2-D arrays of storage words."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    C = None if C is None else np.ascontiguousarray(C)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    Cref = np.empty((M, N), dtype=np.float64)
    D = np.empty((M, N), dtype=np.float64)
    rc = lib().oracle_gemm(*_args(M, N, K, trans_a, trans_b, alpha, A, lda, scale_a, B, ldb,
                                  scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue,
                                  bias), _ptr(Cref), _ptr(D))
    if rc != 0:
        raise ValueError(f"oracle_gemm failed: {rc}")
    return Cref, D


def gemm_rows(p, row0: int, nrows: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rows [row0, row0+nrows) of (Cref, D)."""
    keep, args = _problem_args(p)
    Cref = np.empty((nrows, p.N), dtype=np.float64)
    D = np.empty((nrows, p.N), dtype=np.float64)
    rc = lib().oracle_gemm_rows(*args, row0, nrows, _ptr(Cref), _ptr(D))
    del keep
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows failed: {rc}")
    return Cref, D


def gemm_points(p, rows: np.ndarray, cols: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(Cref, D) at the listed output entries, each computed on its own."""
    keep, args = _problem_args(p)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    Cref = np.empty(r.size, dtype=np.float64)
    D = np.empty(r.size, dtype=np.float64)
    if getattr(p, "sa_blk", None) is not None:
        keep2, mx = _mx_args(p)
        rc = lib().oracle_gemm_mx_points(*args, *mx, r.size, _ptr(r), _ptr(c), _ptr(Cref),
                                         _ptr(D))
        del keep2
    else:
        rc = lib().oracle_gemm_points(*args, r.size, _ptr(r), _ptr(c), _ptr(Cref), _ptr(D))
    del keep
    if rc != 0:
        raise ValueError(f"oracle_gemm_points failed: {rc}")
    return Cref, D


def _q_args(q):
    """(keep, args) for a group-quantized problem with the fields of workloads.QProblem."""
    X = np.ascontiguousarray(q.X)
    W = np.ascontiguousarray(q.Wq, dtype=np.uint8)
    S = np.ascontiguousarray(q.scales)
    O = np.ascontiguousarray(q.offsets)
    C = np.ascontiguousarray(q.C)
    bias = None if q.bias is None else np.ascontiguousarray(q.bias, dtype=np.float32)
    keep = (X, W, S, O, C, bias)
    args = (q.M, q.N, q.K, float(q.alpha), _ptr(X), q.ldx, TYPE_CODE[q.x_type], _ptr(W),
            W.shape[1], int(q.bits), int(q.group), _ptr(S), _ptr(O), S.shape[1],
            TYPE_CODE[q.x_type], float(q.beta), _ptr(C) if q.beta != 0.0 else None, q.N,
            TYPE_CODE[q.x_type], int(q.epilogue), _ptr(bias))
    return keep, args


def qgemm(q) -> Tuple[np.ndarray, np.ndarray]:
    """(Cref, D), each M x N float64, for C = epi(alpha X W^T + beta C + bias) with W affine
    group-quantized (oracle.c: w = s*q + o per row and group of G consecutive k)."""
    keep, args = _q_args(q)
    Cref = np.empty((q.M, q.N), dtype=np.float64)
    D = np.empty((q.M, q.N), dtype=np.float64)
    rc = lib().oracle_qgemm(*args, _ptr(Cref), _ptr(D))
    del keep
    if rc != 0:
        raise ValueError(f"oracle_qgemm failed: {rc}")
    return Cref, D


def qgemm_points(q, rows: np.ndarray, cols: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(Cref, D) of the quantized product at the listed entries, each computed on its own."""
    keep, args = _q_args(q)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    Cref = np.empty(r.size, dtype=np.float64)
    D = np.empty(r.size, dtype=np.float64)
    rc = lib().oracle_qgemm_points(*args, r.size, _ptr(r), _ptr(c), _ptr(Cref), _ptr(D))
    del keep
    if rc != 0:
        raise ValueError(f"oracle_qgemm_points failed: {rc}")
    return Cref, D


def num_threads() -> int:
    return lib().oracle_num_threads()
