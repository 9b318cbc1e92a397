"""The library's calls allocate nothing, keep no per-call host state and record no memset, so a
HIP graph can capture them: a captured gemm_run (bf16 GEMM + bias + GELU, and block-scaled fp8),
a captured gemm_run_q (the quantized decode) and the two kernels that meet through a caller
workspace (the K loop split across two workgroups, and stream-K) are replayed several times,
with the program's own eager work and synchronisations between replays, and every replay must
equal the eager result bit for bit."""
import numpy as np
import pytest

import workloads as W

import gemm_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_matrix_multiply_amd as tmm
    h = tmm.Gemm(0)
    yield h
    h.close()


def _capture_and_replay(call, C, dtype, reps=4):
    """Run `call` eagerly, capture it in a graph, then replay `reps` times, each after the
    output has been cleared by an eager fill kernel; return the eager result and the replays."""
    import torch
    C.zero_()
    call()
    torch.cuda.synchronize()
    eager = H.from_device(C, dtype).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up launch off the default stream before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    outs = []
    for _ in range(reps):
        C.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        outs.append(H.from_device(C, dtype).copy())
    return eager, outs


@pytest.mark.parametrize("name", ["bf16_bias_gelu", "mxfp8"])
def test_gemm_run_in_a_graph(g, name):
    import tiled_matrix_multiply_amd as tmm
    p = W.bf16_bias_gelu(512) if name == "bf16_bias_gelu" else W.mxfp8_4096(512)
    d = H.Device(p)

    def call():
        tmm.run(g.handle, d.A, d.B, d.C, M=p.M, N=p.N, K=p.K, trans_a=p.trans_a,
                trans_b=p.trans_b, alpha=p.alpha, beta=p.beta, a_type=p.a_type,
                b_type=p.b_type, c_type=p.c_type, epilogue=p.epilogue, bias=d.bias,
                scale_a=p.scale_a, scale_b=p.scale_b, sa_blk=d.sa, sb_blk=d.sb)

    eager, outs = _capture_and_replay(call, d.C, p.c_type)
    assert np.any(eager != 0)
    for i, o in enumerate(outs):
        assert np.array_equal(o, eager), f"replay {i}"
    # the eager result is also the oracle's, within the gate
    res = H.gate_full(p, __import__("oracle").decode(p.c_type, eager))
    assert res.ok, res


def test_gemm_run_q_in_a_graph(g):
    import tiled_matrix_multiply_amd as tmm
    q = W.make_qproblem(1, 4096, 2048, bits=4, group=64, seed=21,
                        epilogue=W.EPI_BIAS | W.EPI_GELU)
    X, Wq = H.to_device(q.X), H.to_device(q.Wq)
    S, O = H.to_device(q.scales), H.to_device(q.offsets)
    C = H.to_device(q.C)
    bias = H.to_device(q.bias)

    def call():
        tmm.run_q(g.handle, X, Wq, S, O, C, M=q.M, N=q.N, K=q.K, bits=q.bits, group=q.group,
                  x_type=q.x_type, alpha=q.alpha, beta=q.beta, epilogue=q.epilogue, bias=bias)

    eager, outs = _capture_and_replay(call, C, q.x_type)
    assert np.any(eager != 0)
    for i, o in enumerate(outs):
        assert np.array_equal(o, eager), f"replay {i}"


@pytest.mark.parametrize("kernel", [9, 10])  # GEMM_KERNEL_MFMA_256x128_SK2, GEMM_KERNEL_MFMA_256_SK
def test_split_kernels_in_a_graph(g, kernel):
    """The two kernels that exchange partial sums through a workspace leave it ready for the
    next call from inside the kernel (no memset to record), so a captured call replays
    correctly: every replay equals the eager run bit for bit, and the workspace's counters come
    back ready each time.  1000 x 1304 x 3000 cuts stream-K's tiles into up to 11 parts."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    p = W.make_problem(1000, 1304, 3000, a_type="bf16", seed=81, dist_a=("normal", 1.0),
                       dist_b=("normal", 3000 ** -0.5), epilogue=W.EPI_BIAS | W.EPI_GELU)
    d = H.Device(p)
    nbytes = tmm.gemm_kernel_workspace_bytes(g.handle, kernel, p.M, p.N)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")

    def call():
        tmm.run(g.handle, d.A, d.B, d.C, M=p.M, N=p.N, K=p.K, alpha=p.alpha, beta=p.beta,
                a_type=p.a_type, c_type=p.c_type, epilogue=p.epilogue, bias=d.bias,
                kernel=kernel, workspace=ws, workspace_bytes=nbytes)

    eager, outs = _capture_and_replay(call, d.C, p.c_type)
    assert np.any(eager != 0)
    for i, o in enumerate(outs):
        assert np.array_equal(o, eager), f"replay {i}"
    res = H.gate_full(p, __import__("oracle").decode(p.c_type, eager))
    assert res.ok, res
    words = ws.cpu().numpy().view(np.uint32)
    if kernel == 10:
        cu = torch.cuda.get_device_properties(0).multi_processor_count
        tiles = (-(-p.M // 256)) * (-(-p.N // 256))
        off = 2 * cu * 256 * 256
        assert (words[off:off + 2 * tiles] == 0).all()
    else:
        slot = tmm.SPLIT_K_SLOT_BYTES // 4
        tiles = (-(-p.M // 256)) * (-(-p.N // 128))
        sync = np.array([(words[t * slot], words[t * slot + 1]) for t in range(tiles)])
        assert (sync[:, 0] % 2 == 0).all() and (sync[:, 1] == sync[:, 0] // 2).all()
