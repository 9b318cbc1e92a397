"""Test harness: runs a workloads.Problem through the C ABI on cuda:0 and gates it against the
oracle.  Shared by the GPU parity tests; imports the oracle (test infrastructure) and the
binding, never the other way round."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W
from oracle import gate


def to_device(a: np.ndarray, dev="cuda:0"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def from_device(t, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype in ("f16", "bf16"):
        a = a.view(np.uint16)
    return a


class Device:
    """Device copies of one problem's operands."""

    def __init__(self, p: W.Problem, dev="cuda:0"):
        self.p = p
        self.A = to_device(p.A, dev)
        self.B = to_device(p.B, dev)
        self.C = to_device(p.C, dev)
        self.bias = to_device(p.bias, dev) if p.bias is not None else None
        self.sa = to_device(p.sa_blk, dev) if p.sa_blk is not None else None
        self.sb = to_device(p.sb_blk, dev) if p.sb_blk is not None else None

    def reset_c(self):
        import torch
        self.C.copy_(to_device(self.p.C, self.C.device))


def run(g, p: W.Problem, kernel: int = 0, dev: Device | None = None, epilogue=None,
        workspace=None, workspace_bytes: int = 0):
    """Run on the GPU; returns (stored C bytes as numpy, decoded float64 C)."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    d = dev or Device(p)
    tmm.run(g.handle, d.A, d.B, d.C, M=p.M, N=p.N, K=p.K, trans_a=p.trans_a, trans_b=p.trans_b,
            alpha=p.alpha, beta=p.beta, a_type=p.a_type, b_type=p.b_type, c_type=p.c_type,
            epilogue=p.epilogue if epilogue is None else epilogue, bias=d.bias,
            scale_a=p.scale_a, scale_b=p.scale_b, sa_blk=d.sa, sb_blk=d.sb,
            ldsa=p.ldsa or None, ldsb=p.ldsb or None, kernel=kernel, workspace=workspace,
            workspace_bytes=workspace_bytes)
    torch.cuda.synchronize()
    raw = from_device(d.C, p.c_type)
    return raw, oracle.decode(p.c_type, raw)


_ORACLE_CACHE: dict = {}


def oracle_full(p: W.Problem):
    """oracle.gemm(p), kept for the last two workloads gated (the fused and the unfused runs of
    one workload share it; a 4096^3 reference is two 128 MiB arrays)."""
    key = (p.recipe_hash(), p.alpha, p.beta, p.epilogue)
    if key not in _ORACLE_CACHE:
        if len(_ORACLE_CACHE) >= 2:
            _ORACLE_CACHE.pop(next(iter(_ORACLE_CACHE)))
        _ORACLE_CACHE[key] = oracle.gemm(p)
    return _ORACLE_CACHE[key]


def gate_full(p: W.Problem, got: np.ndarray, roundings: int = 1, cache: bool = False):
    """Every output entry against the oracle (cache=True: reuse the reference of the same
    workload, for named workloads whose inputs never change)."""
    Cref, D = oracle_full(p) if cache else oracle.gemm(p)
    cin = oracle.decode(p.c_type, p.C) if p.beta != 0 else None
    return gate.check(got, Cref, D, gate.tolerance(p.K, p.c_type, roundings, _gelu(p)), p.c_type,
                      p.beta, cin)


def _gelu(p: W.Problem) -> bool:
    return bool(p.epilogue & W.EPI_GELU)


def sample_points(M: int, N: int, n: int = 1024, seed: int = 0, tile: int = 32):
    """Sample output coordinates: every corner of the matrix, entries on the first and last row
    and column of a spread of tiles (where staging and store masks change), and random ones."""
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, 0, M - 1]
    cols = [0, 0, N - 1, N - 1]
    for t in range(0, max(M, N), tile * 7):
        for off in (0, tile - 1):
            rows.append(min(M - 1, t + off))
            cols.append(int(rng.integers(N)))
            rows.append(int(rng.integers(M)))
            cols.append(min(N - 1, t + off))
    k = max(0, n - len(rows))
    rows += list(rng.integers(0, M, k))
    cols += list(rng.integers(0, N, k))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def gate_sampled(p: W.Problem, got: np.ndarray, n: int = 2048, seed: int = 0,
                 roundings: int = 1):
    rows, cols = sample_points(p.M, p.N, n, seed)
    Cref, D = oracle.gemm_points(p, rows, cols)
    cin = oracle.decode(p.c_type, p.C[rows, cols]) if p.beta != 0 else None
    return gate.check(got[rows, cols], Cref, D,
                      gate.tolerance(p.K, p.c_type, roundings, _gelu(p)), p.c_type, p.beta, cin)


POISON = {"f32": np.float32(np.nan).view(np.uint32), "f16": 0xFFFF, "bf16": 0xFFFF,
          "e4m3": 0xFF, "e5m2": 0xFF, "e2m1": 0xFF,   # e2m1 has no NaN: 0xFF is (-6, -6)
          "e2m3": 0xFF, "e3m2": 0xFF}                 # nor the 6-bit types: all -max


def padded_storage(stored: np.ndarray, dtype: str, ld: int) -> np.ndarray:
    """Copy a stored matrix into rows of length ld (elements), filling the padding with NaN
    patterns (packed E2M1 rows hold ld / 2 bytes, packed 6-bit rows 3 ld / 4)."""
    words = stored.view(np.uint32) if stored.dtype == np.float32 else stored
    width = ld // 2 if dtype == "e2m1" else (ld // 4 * 3 if dtype in W.FP6 else ld)
    out = np.full((stored.shape[0], width), POISON[dtype], dtype=words.dtype)
    out[:, :stored.shape[1]] = words
    return out.view(np.float32) if stored.dtype == np.float32 else out


def aligned_ld(width: int, mult: int = 16) -> int:
    """A leading dimension >= width that keeps 16-byte alignment for every element size."""
    return ((width + mult - 1) // mult) * mult + mult


def run_padded(g, p: W.Problem, ld_fn=aligned_ld, kernel: int = 0, workspace=None,
               workspace_bytes: int = 0):
    """Run with padded leading dimensions (padding poisoned with NaN).  Returns the decoded
    logical C, the kernel family gemm_run picked, and whether C's padding came back intact."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    lda, ldb, ldc = ld_fn(p.lda), ld_fn(p.ldb), ld_fn(p.ldc)
    if p.a_type == "e2m1":  # whole 16-byte packed rows
        lda, ldb = -(-lda // 32) * 32, -(-ldb // 32) * 32
    if p.a_type in W.FP6:  # whole 16-byte packed rows: 64 elements are 48 bytes
        lda, ldb = -(-lda // 64) * 64, -(-ldb // 64) * 64
    Ah = padded_storage(p.A, p.a_type, lda)
    Bh = padded_storage(p.B, p.b_type, ldb)
    Ch = padded_storage(p.C, p.c_type, ldc)
    A, B, C = to_device(Ah), to_device(Bh), to_device(Ch)
    bias = to_device(p.bias) if p.bias is not None else None
    kname = tmm.select_kernel(g.handle, p.M, p.N, p.K, trans_a=p.trans_a, trans_b=p.trans_b,
                              a_type=p.a_type, b_type=p.b_type, A=A, B=B, C=C,
                              epilogue=p.epilogue, bias=bias, lda=lda, ldb=ldb, ldc=ldc)
    sa = sb = None
    ldsa = ldsb = None
    if p.sa_blk is not None:
        # scale rows padded to 16-byte multiples with NaN scales (0xFF) that must never be used
        ldsa = ldsb = -(-p.ldsa // 16) * 16
        sa = to_device(padded_storage(p.sa_blk, "e4m3", ldsa))
        sb = to_device(padded_storage(p.sb_blk, "e4m3", ldsb))
    tmm.run(g.handle, A, B, C, M=p.M, N=p.N, K=p.K, trans_a=p.trans_a, trans_b=p.trans_b,
            alpha=p.alpha, beta=p.beta, a_type=p.a_type, b_type=p.b_type, c_type=p.c_type,
            epilogue=p.epilogue, bias=bias, scale_a=p.scale_a, scale_b=p.scale_b, lda=lda,
            ldb=ldb, ldc=ldc, sa_blk=sa, sb_blk=sb, ldsa=ldsa, ldsb=ldsb, kernel=kernel,
            workspace=workspace, workspace_bytes=workspace_bytes)
    torch.cuda.synchronize()
    raw = from_device(C, p.c_type)
    pad_ok = bool(np.array_equal(raw.view(np.uint8).reshape(p.M, -1)[:, p.N * W.ESIZE[p.c_type]:],
                                 Ch.view(np.uint8).reshape(p.M, -1)[:, p.N * W.ESIZE[p.c_type]:]))
    return oracle.decode(p.c_type, np.ascontiguousarray(raw[:, :p.N])), kname, pad_ok


def mfma_aligned(p: W.Problem) -> bool:
    es = W.ESIZE[p.a_type]
    return (p.lda * es) % 16 == 0 and (p.ldb * es) % 16 == 0 and p.ldc % 4 == 0
