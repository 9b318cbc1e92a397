"""GPU parity of the 256 x 128 tile and of its K loop split across two workgroups (the
mid-size regime: fewer output tiles than compute units), called through gemm_run_ws /
gemm_run_ws_kernel, against the float64 oracle.

The split kernel hands the first workgroup's fp32 partial sums to the second through a
workspace; both orders of arrival give the same sum (fp32 addition is commutative), so repeated
runs must agree bit for bit, and the workspace must come back ready for the next call.
"""
import itertools
import zlib

import numpy as np
import pytest

import oracle
import workloads as W

import gemm_harness as H

pytestmark = pytest.mark.gpu

KERNELS = {"wide": 8, "split": 9}


@pytest.fixture(scope="module")
def g():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    h = tmm.Gemm(0)
    yield h
    h.close()


def _workspace(M, N):
    import torch
    import tiled_matrix_multiply_amd as tmm
    nbytes = tmm.split_k_workspace_bytes(M, N)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    assert ws.data_ptr() % 256 == 0
    return ws, nbytes


def _report(name, res):
    print(f"[splitk] {name}: {res}", flush=True)


@pytest.mark.parametrize("dtype,kernel,ta,tb",
                         list(itertools.product(["f16", "bf16"], ["wide", "split"], [False, True],
                                                [False, True])))
def test_integer_inputs_bit_exact(g, dtype, kernel, ta, tb):
    """Integer inputs in [-4, 4]: exact in any accumulation order and any split of K, so the
    result must equal the exact value rounded once, in every layout; ragged M, N and K."""
    M, N, K = 300, 270, 1000
    seed = zlib.crc32(f"sk/{dtype}/{kernel}/{ta}/{tb}".encode()) & 0xFFFF
    p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, seed=seed,
                       dist_a=("int", (-4, 4)), dist_b=("int", (-4, 4)), fp8_scaled=False,
                       alpha=2.0, beta=-1.0, dist_c=("int", (-8, 8)), epilogue=W.EPI_BIAS)
    p.bias = np.round(p.bias * 30).astype(np.float32)
    ws, nbytes = _workspace(M, N)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS[kernel], workspace=ws,
                                      workspace_bytes=nbytes)
    Cref, _ = oracle.gemm(p)
    expect = oracle.decode(p.c_type, W.encode(Cref, p.c_type))
    bad = np.argwhere(got != expect)
    assert pad_ok
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("K", [1, 8, 64, 72, 128, 136, 520, 4104])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_short_and_ragged_k(g, dtype, K):
    """K of 1 .. 65 K tiles, so the second half may be empty (one tile) or one tile shorter
    than the first; beta, bias and GELU together, gated on every entry."""
    M, N = 520, 392
    p = W.make_problem(M, N, K, a_type=dtype, alpha=1.25, beta=-0.5, seed=K + 7,
                       dist_a=("normal", 1.0), dist_b=("normal", 1.0),
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    ws, nbytes = _workspace(M, N)
    got, kname, pad_ok = H.run_padded(g, p, kernel=KERNELS["split"], workspace=ws,
                                      workspace_bytes=nbytes)
    res = H.gate_full(p, got)
    _report(f"{dtype} {M}x{N}x{K} split", res)
    assert pad_ok and res.ok, res


@pytest.mark.parametrize("name,n", [("fp16", 2048), ("bf16_gelu", 2048), ("bf16_gelu", 1536)])
def test_named_workloads_every_entry(g, name, n):
    """The 2048^3 workloads (and 1536^3) through the split kernel, named, with a workspace of the
    size the header states: every output entry meets the oracle's gate, a second call on the
    same workspace gives the same bits, and the workspace comes back ready (counters even, flags
    at half the counters).  AUTO with a workspace picks no split for them (gemm_workspace_bytes
    reports 0) and matches gemm_run."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.fp16_square(n) if name == "fp16" else W.bf16_bias_gelu(n)
    d = H.Device(p)
    need = tmm.gemm_workspace_bytes(g.handle, p.M, p.N, p.K, 0, 0, d.A.data_ptr(), p.lda,
                                    d.B.data_ptr(), p.ldb, d.C.data_ptr(), p.ldc,
                                    tmm.DTYPE[p.a_type], tmm.DTYPE[p.b_type],
                                    tmm.DTYPE[p.c_type], p.epilogue,
                                    d.bias.data_ptr() if d.bias is not None else None)
    assert need == 0, need
    ws, nbytes = _workspace(p.M, p.N)
    raw1, got = H.run(g, p, kernel=KERNELS["split"], dev=d, workspace=ws, workspace_bytes=nbytes)
    res = H.gate_full(p, got, cache=True)
    _report(f"{name} {n}^3 (split kernel)", res)
    assert res.ok, res
    d.reset_c()
    raw2, _ = H.run(g, p, kernel=KERNELS["split"], dev=d, workspace=ws, workspace_bytes=nbytes)
    assert np.array_equal(raw1, raw2)
    tiles, slot = (-(-p.M // 256)) * (-(-p.N // 128)), tmm.SPLIT_K_SLOT_BYTES // 4
    words = ws.cpu().numpy().view(np.uint32)
    sync = np.array([(words[t * slot], words[t * slot + 1]) for t in range(tiles)])
    assert (sync[:, 0] % 2 == 0).all() and (sync[:, 1] == sync[:, 0] // 2).all()
    d.reset_c()
    raw3, _ = H.run(g, p, dev=d, workspace=ws, workspace_bytes=nbytes)
    d.reset_c()
    raw4, _ = H.run(g, p, dev=d)
    assert np.array_equal(raw3, raw4)


def test_split_matches_unsplit_wide_tile(g):
    """The split kernel against the same tile without the split, and against the 128 x 128
    tile gemm_run picks, on one problem: all gated; the split result is reproducible bit for
    bit over five calls."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(1024, 2048, 3072, a_type="bf16", seed=91, dist_a=("normal", 1.0),
                       dist_b=("normal", 3072 ** -0.5), epilogue=W.EPI_BIAS | W.EPI_GELU)
    d = H.Device(p)
    ws, nbytes = _workspace(p.M, p.N)
    outs = []
    for _ in range(5):
        d.reset_c()
        raw, got = H.run(g, p, kernel=KERNELS["split"], dev=d, workspace=ws, workspace_bytes=nbytes)
        outs.append(raw)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    res = H.gate_full(p, got, cache=True)
    _report("bf16 1024x2048x3072 split", res)
    assert res.ok
    d.reset_c()
    _, wide = H.run(g, p, kernel=KERNELS["wide"], dev=d)
    assert H.gate_full(p, wide, cache=True).ok


@pytest.mark.parametrize("dtype,M,N,K,ta,tb", [("bf16", 1100, 4104, 520, False, False),
                                                ("f16", 2304, 2056, 200, True, True)])
def test_auto_takes_wide_tile(g, dtype, M, N, K, ta, tb):
    """Shapes whose 128 x 128 tiles need more than one round of the compute units and whose
    256 x 128 tiles fit in one: gemm_run picks the 256 x 128 tile, and every entry of the
    result (ragged M, N and K, padded leading dimensions, beta, bias and GELU) meets the
    oracle's gate."""
    p = W.make_problem(M, N, K, a_type=dtype, trans_a=ta, trans_b=tb, alpha=0.75, beta=0.5,
                       seed=M + K, dist_a=("normal", 1.0), dist_b=("normal", K ** -0.5),
                       epilogue=W.EPI_BIAS | W.EPI_GELU)
    got, kname, pad_ok = H.run_padded(g, p)
    res = H.gate_full(p, got)
    _report(f"{dtype} {M}x{N}x{K} AUTO ({kname})", res)
    assert kname == "mfma256x128"
    assert pad_ok and res.ok, res


def test_workspace_validation(g):
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(512, 512, 512, a_type="f16", seed=3)
    d = H.Device(p)
    ws, nbytes = _workspace(p.M, p.N)
    args = (p.M, p.N, p.K, 0, 0, 1.0, d.A.data_ptr(), p.lda, 1.0, d.B.data_ptr(), p.ldb, 1.0, 0.0,
            d.C.data_ptr(), p.ldc, tmm.GEMM_F16, tmm.GEMM_F16, tmm.GEMM_F16, 0, None)
    split = tmm.GEMM_KERNEL_MFMA_256x128_SK2
    # too small, missing, misaligned, negative
    assert tmm.gemm_run_ws_kernel(g.handle, split, None, *args, ws.data_ptr(), nbytes - 256) == tmm.GEMM_ERR_INVALID_VALUE
    assert tmm.gemm_run_ws_kernel(g.handle, split, None, *args, None, 0) == tmm.GEMM_ERR_INVALID_VALUE
    assert tmm.gemm_run_ws_kernel(g.handle, split, None, *args, ws.data_ptr() + 16, nbytes - 256) == tmm.GEMM_ERR_INVALID_VALUE
    assert tmm.gemm_run_ws(g.handle, None, *args, ws.data_ptr(), -1) == tmm.GEMM_ERR_INVALID_VALUE
    # fp32 is not a type of the wide tile
    p32 = W.make_problem(512, 512, 512, a_type="f32", seed=3)
    d32 = H.Device(p32)
    a32 = (512, 512, 512, 0, 0, 1.0, d32.A.data_ptr(), 512, 1.0, d32.B.data_ptr(), 512, 1.0, 0.0,
           d32.C.data_ptr(), 512, tmm.GEMM_F32, tmm.GEMM_F32, tmm.GEMM_F32, 0, None)
    assert tmm.gemm_run_ws_kernel(g.handle, split, None, *a32, ws.data_ptr(), nbytes) == tmm.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_workspace_slots_survive_calls_of_other_sizes(g):
    """Tile t's counter, flag and partial sums live in slot t whatever the size of the call, so a
    smaller call on a shared workspace touches only its own slots: after a 32-tile call and an
    8-tile call, slots 8..31 still hold what the first call left (counter 2, flag 1), and a third,
    32-tile call is correct and equal to the first bit for bit."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    big = W.make_problem(1024, 1024, 1024, a_type="bf16", seed=41, dist_a=("normal", 1.0),
                         dist_b=("normal", 1.0 / 32), epilogue=W.EPI_BIAS | W.EPI_GELU)
    small = W.make_problem(512, 512, 768, a_type="bf16", seed=42, dist_a=("normal", 1.0),
                           dist_b=("normal", 1.0 / 32), epilogue=W.EPI_BIAS | W.EPI_GELU)
    ws, nbytes = _workspace(big.M, big.N)
    slot = tmm.SPLIT_K_SLOT_BYTES
    tiles_big, tiles_small = (1024 // 256) * (1024 // 128), (512 // 256) * (512 // 128)
    assert nbytes == tiles_big * slot and tiles_small == 8

    def sync_words():
        w = ws.cpu().numpy().view(np.uint32)
        return np.array([(w[t * slot // 4], w[t * slot // 4 + 1]) for t in range(tiles_big)])

    db = H.Device(big)
    first, _ = H.run(g, big, kernel=KERNELS["split"], dev=db, workspace=ws, workspace_bytes=nbytes)
    assert (sync_words() == [2, 1]).all()
    ds = H.Device(small)
    got_small, _ = H.run(g, small, kernel=KERNELS["split"], dev=ds, workspace=ws,
                         workspace_bytes=nbytes)
    words = sync_words()
    assert (words[:tiles_small] == [4, 2]).all() and (words[tiles_small:] == [2, 1]).all(), words
    assert H.gate_full(small, oracle.decode(small.c_type, got_small)).ok
    db.reset_c()
    third, _ = H.run(g, big, kernel=KERNELS["split"], dev=db, workspace=ws, workspace_bytes=nbytes)
    assert np.array_equal(first, third)
    res = H.gate_full(big, oracle.decode(big.c_type, third))
    _report("slots across sizes 1024^2 / 512^2 / 1024^2", res)
    assert res.ok, res
    torch.cuda.synchronize()
