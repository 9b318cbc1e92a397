"""The library's calls allocate nothing, keep no per-call host state and record no memset, so a
HIP graph can capture them: a captured gemm_run (bf16 GEMM + bias + GELU, and block-scaled fp8)
and a captured gemm_run_q (the quantized decode) are replayed several times, with the program's
own eager work and synchronisations between replays, and every replay must equal the eager
result bit for bit."""
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
