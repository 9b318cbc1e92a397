"""gemm_run_noalloc, the entry point that allocates nothing (its workspace is the library's
static device array): through the C ABI, against gemm_run_ws_kernel with a caller-provided
workspace on the same kernel, on two calls in a row (the second smaller), and its size limit.

The kernel that uses the scratch (the K loop split across two workgroups) is deterministic, so
the two entry points must agree bit for bit; each result is also gated against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as W

import gemm_harness as H

pytestmark = pytest.mark.gpu

SPLIT = 9  # GEMM_KERNEL_MFMA_256x128_SK2


@pytest.fixture(scope="module")
def g():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    h = tmm.Gemm(0)
    yield h
    h.close()


def _args(tmm, p, d):
    return (p.M, p.N, p.K, int(p.trans_a), int(p.trans_b), float(p.alpha), d.A.data_ptr(), p.lda,
            float(p.scale_a), d.B.data_ptr(), p.ldb, float(p.scale_b), float(p.beta),
            d.C.data_ptr(), p.ldc, tmm.DTYPE[p.a_type], tmm.DTYPE[p.b_type], tmm.DTYPE[p.c_type],
            p.epilogue, d.bias.data_ptr() if d.bias is not None else None)


def _noalloc_vs_ws(g, p):
    import torch
    import tiled_matrix_multiply_amd as tmm
    d = H.Device(p)
    assert tmm.gemm_run_noalloc(g.handle, SPLIT, None, *_args(tmm, p, d)) == tmm.GEMM_OK
    torch.cuda.synchronize()
    got_noalloc = H.from_device(d.C, p.c_type).copy()
    nbytes = tmm.split_k_workspace_bytes(p.M, p.N)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    d.reset_c()
    assert tmm.gemm_run_ws_kernel(g.handle, SPLIT, None, *_args(tmm, p, d), ws.data_ptr(),
                                  nbytes) == tmm.GEMM_OK
    torch.cuda.synchronize()
    got_ws = H.from_device(d.C, p.c_type)
    assert np.array_equal(got_noalloc, got_ws)
    res = H.gate_full(p, oracle.decode(p.c_type, got_noalloc))
    print(f"[noalloc] {p.a_type} {p.M}x{p.N}x{p.K}: {res}", flush=True)
    assert res.ok, res


def test_noalloc_matches_workspace_entry_two_calls(g):
    """Two calls in a row on the shared static array, the second with a smaller problem of the
    other 16-bit type and another layout."""
    p1 = W.make_problem(1024, 2048, 1536, a_type="bf16", seed=31, alpha=0.75, beta=0.5,
                        dist_a=("normal", 1.0), dist_b=("normal", 1536 ** -0.5),
                        dist_c=("normal", 1.0), epilogue=W.EPI_BIAS | W.EPI_GELU)
    _noalloc_vs_ws(g, p1)
    p2 = W.make_problem(520, 392, 1000, a_type="f16", seed=32, trans_a=True, trans_b=True,
                        dist_a=("normal", 1.0), dist_b=("normal", 1.0), epilogue=W.EPI_BIAS)
    _noalloc_vs_ws(g, p2)


def test_noalloc_limit_and_auto(g):
    """An output of more tiles than the static array holds is refused before any launch; AUTO
    (which uses no scratch) runs as gemm_run."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    big = W.make_problem(4096, 2304, 64, a_type="f16", seed=33)     # 16 x 18 = 288 tiles
    d = H.Device(big)
    before = H.from_device(d.C, "f16").copy()
    assert tmm.gemm_run_noalloc(g.handle, SPLIT, None, *_args(tmm, big, d)) == tmm.GEMM_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert np.array_equal(H.from_device(d.C, "f16"), before)
    assert "scratch" in tmm.gemm_status_string(tmm.GEMM_ERR_TOO_LARGE)
    p = W.make_problem(300, 270, 500, a_type="bf16", seed=34, dist_a=("normal", 1.0),
                       dist_b=("normal", 1.0), epilogue=W.EPI_GELU)
    d = H.Device(p)
    assert tmm.gemm_run_noalloc(g.handle, 0, None, *_args(tmm, p, d)) == tmm.GEMM_OK
    torch.cuda.synchronize()
    a = H.from_device(d.C, "bf16").copy()
    d.reset_c()
    H.run(g, p, dev=d)
    assert np.array_equal(a, H.from_device(d.C, "bf16"))
