#!/usr/bin/env python3
"""Benchmark of the tiled GEMM on one MI355X.

Headline: bf16 GEMM + bias + erf-GELU, fused into the GEMM epilogue, M = N = K = 4096
(A ~ N(0,1), B ~ N(0,1/K), bias ~ N(0,0.1^2), seed 3).  One step = one fused GEMM call over
that problem with every input already resident in HBM.  Throughput is 2*M*N*K per step
(epilogue FLOPs are not counted).  Then the sweeps: fp32 256^3 and 1000^3 (NN and TN),
fp16 n^3, bf16 fused versus unfused n^3 for n in {512, 1024, 2048, 4096}, and fp8-E4M3 versus
bf16 at 4096^3.  Each cell: warm up for >= 200 ms, then R timed reps with one HIP event pair
per rep on the stream the kernel runs on; median and a percentile-bootstrap 95% CI
(10^4 resamples, seed 0), as "Rigel" (arXiv 2606.12765), section 3 reports its cells.  The
headline's timed steps come after a time-based settle (--settle-seconds of back-to-back steps)
and the --warmup steps.  Clock ("Rigel" section 3: the clock state decides the results): the
headline's roofline carries the shader clock held during the kernel, from the committed
counter summary of the same sources (GRBM_GUI_ACTIVE per dispatch time), and every timed
region is followed by an in-kernel probe of the clock it left the chip at.  A measured
streaming-read and copy bandwidth stands beside the 8 TB/s HBM figure as the practical ceiling
of the bandwidth-bound cells ("Case Study: The Tiled GEMM", its bandwidth roofline).

Prints ONE JSON line.  Only --gpus 1 is supported: the library runs on a single GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s & % MFMA peak: bf16 GEMM+bias+GELU 4096³; fp32/fp16/fp8 sweeps"
# MI355X published dense peaks (256 CUs at 2.4 GHz).
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2,
               "e2m1": 10066.3, "e2m3": 10066.3, "e3m2": 10066.3}
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_bf16_bias_gelu_4096.txt")


# The files the headline kernel is built from: its template, its instantiation, the host code
# that picks its tile and launches it, and the build flags.  Other kernels' sources do not
# change it, so a stored counter measurement stays valid across their edits.
HEADLINE_SOURCES = ("tiled_matrix_multiply_amd/csrc/common.hpp",
                    "tiled_matrix_multiply_amd/csrc/mfma.hpp",
                    "tiled_matrix_multiply_amd/csrc/mfma_bf16.hip",
                    "tiled_matrix_multiply_amd/csrc/api.cpp",
                    "tiled_matrix_multiply_amd/csrc/handle.hpp",
                    "tiled_matrix_multiply_amd/build.py",
                    "include/gemm.h")


def source_hash(files=HEADLINE_SOURCES) -> str:
    """Hash of the sources of a kernel: ties a stored counter measurement to the kernel it saw."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def bootstrap_ci(x: np.ndarray, n_boot: int = 10000, seed: int = 0):
    """Percentile bootstrap 95% CI of the median."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, len(x), size=(n_boot, len(x)))
    meds = np.median(x[idx], axis=1)
    return float(np.percentile(meds, 2.5)), float(np.percentile(meds, 97.5))


class ClockProbe:
    """The shader clock a timed region left the chip at, read in-kernel: gemm_probe_clock
    enqueued on the same stream right behind the region's last launch, `workgroups` one-wave
    workgroups each timing `us` microseconds of the constant-rate counter against the
    shader-clock cycle counter.  The clock recovers within microseconds once the matrix-core
    load ends, so this reads the state between runs (near 2.4 GHz), not the power-held clock
    during the kernel; that one comes from the counter summary (read_counters)."""

    def __init__(self, g, workgroups: int = 256, us: int = 40):
        import torch
        import tiled_matrix_multiply_amd as tmm
        self.tmm = tmm
        self.h = g.handle
        self.wg, self.us = workgroups, us
        self.buf = torch.zeros(4 * workgroups, dtype=torch.int64, device="cuda:0")
        self.khz = tmm.gemm_wall_clock_khz(self.h)

    def enqueue(self, stream):
        st = self.tmm.gemm_probe_clock(self.h, stream, self.buf.data_ptr(), self.wg, self.us)
        if st != 0:
            raise RuntimeError(f"gemm_probe_clock: {self.tmm.gemm_status_string(st)}")

    def read(self):
        """After a synchronisation: mean, min and max over the workgroups (MHz)."""
        v = self.buf.cpu().numpy().reshape(-1, 4).astype(np.float64)
        mhz = (v[:, 2] - v[:, 0]) / (v[:, 3] - v[:, 1]) * self.khz / 1000.0
        return {"mean": round(float(mhz.mean()), 1), "min": round(float(mhz.min()), 1),
                "max": round(float(mhz.max()), 1), "workgroups": int(mhz.size),
                "source": "s_memtime / s_memrealtime probe right after the timed launches"}


def hbm_ceiling(g, nbytes: int = 1 << 30, reps: int = 20) -> dict:
    """Measured HBM ceiling with the library's bandwidth probe over `nbytes` (4x the 256 MB
    last-level cache, so every rep streams from HBM): a read-only stream and a copy, each timed
    with one event pair around `reps` launches after a warm-up.  GB/s counts bytes read (plus
    bytes written for the copy)."""
    import torch
    import tiled_matrix_multiply_amd as tmm
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.current_stream()
    out = {"bytes": nbytes, "reps": reps, "kind": "library bandwidth probe: 16-byte loads, "
                                                   "4 in flight per thread"}
    for mode, d, moved in (("read", None, nbytes), ("copy", dst.data_ptr(), 2 * nbytes)):
        def launch():
            st = tmm.gemm_probe_bandwidth(g.handle, s.cuda_stream, src.data_ptr(), d, nbytes,
                                          sink.data_ptr())
            if st != 0:
                raise RuntimeError(f"gemm_probe_bandwidth: {tmm.gemm_status_string(st)}")
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            launch()
        e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{mode}_gbs"] = round(moved / (ms * 1e-3) / 1e9, 1)
        out[f"{mode}_us"] = round(ms * 1e3, 2)
        print(f"[bench] HBM {mode} probe over {nbytes >> 20} MiB: {ms * 1e3:.1f} us, "
              f"{out[f'{mode}_gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    del src, dst
    torch.cuda.empty_cache()
    return out


class Cell:
    """Device-resident operands of one workload and the call that runs it."""

    def __init__(self, g, p, unfused: bool = False):
        import torch
        import tiled_matrix_multiply_amd as tmm

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to("cuda:0")

        self.p = p
        self.unfused = unfused
        self.launches_per_step = 2 if unfused else 1
        self._dev, self._C0 = dev, p.C  # to restore C before the gate's fresh step
        self.A, self.B, self.C = dev(p.A), dev(p.B), dev(p.C)
        self.bias = dev(p.bias) if p.bias is not None else None
        self.stream = torch.cuda.current_stream()
        s = self.stream.cuda_stream
        h = g.handle
        epi = 0 if unfused else p.epilogue
        dt = tmm.DTYPE
        args = (p.M, p.N, p.K, int(p.trans_a), int(p.trans_b), float(p.alpha), self.A.data_ptr(),
                p.lda, float(p.scale_a), self.B.data_ptr(), p.ldb, float(p.scale_b),
                float(p.beta), self.C.data_ptr(), p.ldc, dt[p.a_type], dt[p.b_type],
                dt[p.c_type], epi, self.bias.data_ptr() if self.bias is not None else None)
        self.kernel = tmm.KERNEL_NAME[tmm.gemm_select_kernel(
            h, p.M, p.N, p.K, int(p.trans_a), int(p.trans_b), self.A.data_ptr(), p.lda,
            self.B.data_ptr(), p.ldb, self.C.data_ptr(), p.ldc, dt[p.a_type], dt[p.b_type],
            dt[p.c_type], epi, args[-1])]
        run = tmm.library().gemm_run
        # A workspace, when the library would use one for these arguments (the K loop of
        # mid-size 16-bit products split across workgroups): allocated and zeroed once, here,
        # outside every timed region.
        self.ws = None
        self.ws_bytes = 0
        if not p.mx:
            need = tmm.gemm_workspace_bytes(h, *args[:5], args[6], args[7], args[9], args[10],
                                            args[13], args[14], args[15], args[16], args[17],
                                            epi, args[-1])
            if need > 0:
                self.ws_bytes = need
                self.ws = torch.zeros(need // 4, dtype=torch.int32, device="cuda:0")
                args = args + (self.ws.data_ptr(), need)
                run = tmm.library().gemm_run_ws
                self.kernel = "mfma256x128_sk2"
        if p.mx:
            # OCP MX block scales: one E8M0 byte per 32 k of each row of op(A) / column of op(B)
            self.sa, self.sb = dev(p.sa_blk), dev(p.sb_blk)
            args = (p.M, p.N, p.K, int(p.trans_a), int(p.trans_b), float(p.alpha),
                    self.A.data_ptr(), p.lda, self.sa.data_ptr(), p.ldsa, self.B.data_ptr(),
                    p.ldb, self.sb.data_ptr(), p.ldsb, float(p.beta), self.C.data_ptr(), p.ldc,
                    dt[p.a_type], dt[p.b_type], dt[p.c_type], epi,
                    self.bias.data_ptr() if self.bias is not None else None)
            run = tmm.library().gemm_run_mx
        bias_gelu = tmm.library().gemm_bias_gelu
        post = (h, s, p.M, p.N, self.C.data_ptr(), p.ldc, dt[p.c_type], args[-1], p.epilogue)

        def step(stream=None):
            sh = s if stream is None else stream
            st = run(h, sh, *args)
            if st != 0:
                raise RuntimeError(f"gemm_run: {tmm.gemm_status_string(st)}")
            if unfused:
                st = bias_gelu(h, sh, *post[2:])
                if st != 0:
                    raise RuntimeError(f"gemm_bias_gelu: {tmm.gemm_status_string(st)}")
        self.step = step

    def settle(self, seconds: float, min_steps: int = 3) -> int:
        """Back-to-back steps for at least `seconds` of wall time (clocks and power settle);
        returns the number of steps run."""
        import torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while n < min_steps or time.perf_counter() - t0 < seconds:
            self.step()
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return n

    def time(self, reps: int, warmup_s: float = 0.2, warmup_min: int = 3, clock=None):
        """Per-rep durations (ms) from HIP event pairs on the kernel's stream, after a time-based
        warm-up; `clock` (a ClockProbe) is queued right behind the timed launches, its reading
        kept in self.sclk."""
        import torch
        self.settle(warmup_s, warmup_min)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for s, e in ev:
            s.record(self.stream)
            self.step()
            e.record(self.stream)
        torch.cuda.synchronize()
        ms = np.array([s.elapsed_time(e) for s, e in ev], dtype=np.float64)
        # the same launches back to back between one event pair (no per-launch event in the
        # stream): the launch-to-launch period, which the per-launch pairs inflate for small
        # problems
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            self.step()
        e1.record(self.stream)
        if clock is not None:
            clock.enqueue(self.stream.cuda_stream)
        torch.cuda.synchronize()
        self.b2b_ms = e0.elapsed_time(e1) / reps
        self.sclk = clock.read() if clock is not None else None
        return ms

    def result_sample(self, n: int = 512, seed: int = 0) -> dict:
        """One fresh step (C first restored to its initial contents when beta != 0, since the
        timed steps fed each result back in) and the stored output words at n seeded points,
        for the checksum gate of the CPU leg."""
        import torch
        p = self.p
        if p.beta != 0:
            self.C.copy_(self._dev(self._C0))
        self.step()
        torch.cuda.synchronize()
        out = self.C.cpu().numpy()
        rows, cols = gate_points(p.M, p.N, n, seed)
        raw = out[rows, cols]
        return {"rows": rows, "cols": cols, "raw": raw.view(np.uint16) if raw.dtype == np.int16 else raw}

    def algorithmic_bytes(self) -> int:
        p = self.p
        import workloads as W
        cs = W.ESIZE[p.c_type]
        b = int(p.M * p.K * W.ESIZE[p.a_type] + p.K * p.N * W.ESIZE[p.b_type]) + p.M * p.N * cs
        if p.mx:
            b += p.sa_blk.size + p.sb_blk.size
        if p.beta != 0:
            b += p.M * p.N * cs
        if p.bias is not None:
            b += 4 * p.N
        if self.unfused:
            b += 2 * p.M * p.N * cs   # the second pass reads and writes C again
        return b


class QCell:
    """Device-resident operands of one group-quantized workload.  `copies` > 1 keeps that many
    copies of the weights (codes, scales, offsets) and steps through them, so that a launch
    reads its weights from HBM rather than from the 256 MB last-level cache."""

    def __init__(self, g, q, copies: int = 1):
        import torch
        import tiled_matrix_multiply_amd as tmm

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to("cuda:0")

        self.p = q
        self.launches_per_step = 1
        self._dev, self._C0 = dev, q.C
        self.X, self.C = dev(q.X), dev(q.C)
        self.bias = dev(q.bias) if q.bias is not None else None
        self.W = [(dev(q.Wq), dev(q.scales), dev(q.offsets)) for _ in range(copies)]
        self.stream = torch.cuda.current_stream()
        s = self.stream.cuda_stream
        h = g.handle
        run = tmm.library().gemm_run_q
        bptr = self.bias.data_ptr() if self.bias is not None else None
        xt = tmm.DTYPE[q.x_type]
        w0 = self.W[0]
        self.kernel = tmm.KERNEL_NAME[tmm.gemm_select_kernel_q(
            h, q.M, q.N, q.K, self.X.data_ptr(), q.ldx, w0[0].data_ptr(), q.Wq.shape[1], q.bits,
            q.group, w0[1].data_ptr(), w0[2].data_ptr(), q.scales.shape[1], self.C.data_ptr(),
            q.N, xt, q.epilogue, bptr)]
        self.args = [(h, s, q.M, q.N, q.K, float(q.alpha), self.X.data_ptr(), q.ldx,
                      w[0].data_ptr(), q.Wq.shape[1], q.bits, q.group, w[1].data_ptr(),
                      w[2].data_ptr(), q.scales.shape[1], float(q.beta), self.C.data_ptr(), q.N,
                      xt, q.epilogue, bptr) for w in self.W]
        self.i = 0

        def step(stream=None):
            a = self.args[self.i]
            st = run(a[0], a[1] if stream is None else stream, *a[2:])
            self.i = (self.i + 1) % len(self.args)
            if st != 0:
                raise RuntimeError(f"gemm_run_q: {tmm.gemm_status_string(st)}")
        self.step = step

    settle = Cell.settle
    time = Cell.time
    result_sample = Cell.result_sample

    def algorithmic_bytes(self) -> int:
        q = self.p
        b = q.weight_bytes() + q.X.nbytes + q.M * q.N * 2
        if q.beta != 0:
            b += q.M * q.N * 2
        if q.bias is not None:
            b += 4 * q.N
        return int(b)


def sweep_cells():
    """Every sweep cell as (name, dtype, make), make(g) building its device operands (a Cell
    or a QCell).  The timed sweep and the counter pass both walk this list."""
    import workloads as W
    cells = [("fp32 256", "f32", lambda g: Cell(g, W.fp32_256())),
             ("fp32 1000 a=1.5 b=-0.5 NN", "f32", lambda g: Cell(g, W.fp32_1000_ragged(False))),
             ("fp32 1000 a=1.5 b=-0.5 TN", "f32", lambda g: Cell(g, W.fp32_1000_ragged(True)))]
    for n in (512, 1024, 2048, 4096):
        cells.append((f"fp16 {n}", "f16", lambda g, n=n: Cell(g, W.fp16_square(n))))
    for n in (512, 1024, 2048, 4096):
        cells.append((f"bf16+bias+GELU fused {n}", "bf16",
                      lambda g, n=n: Cell(g, W.bf16_bias_gelu(n))))
        cells.append((f"bf16 GEMM then bias+GELU {n}", "bf16",
                      lambda g, n=n: Cell(g, W.bf16_bias_gelu(n), unfused=True)))
    cells += [
        ("fp8 e4m3 4096 (scaled, bf16 out)", "e4m3", lambda g: Cell(g, W.fp8_4096(4096))),
        ("bf16 4096 (fp8 twin)", "bf16", lambda g: Cell(g, W.bf16_twin_of_fp8(4096))),
        ("fp8 e5m2 4096 (scaled, bf16 out)", "e5m2", lambda g: Cell(g, W.e5m2_4096(4096))),
        ("mxfp8 e4m3 4096 (E8M0 / 32 k)", "e4m3", lambda g: Cell(g, W.mxfp8_4096(4096))),
        ("mxfp6 e2m3 4096 (E8M0 / 32 k)", "e2m3", lambda g: Cell(g, W.mxfp6_4096(4096))),
        ("mxfp4 e2m1 4096 (E8M0 / 32 k)", "e2m1", lambda g: Cell(g, W.mxfp4_4096(4096))),
        # Quantized decode: one token through a 28672 x 8192 projection with 4-bit weights in
        # groups of 64; three weight copies (397 MB) are cycled so that every launch streams
        # its weights from HBM.  Bound by HBM: GB/s against 8 TB/s is its roofline.
        ("q4 decode 1x28672x8192 (G=64)", "bf16", lambda g: QCell(g, W.q4_decode(), copies=3)),
        # Quantized prefill: 4096 tokens through a 4096 x 4096 projection, 4-bit weights in
        # groups of 64 dequantised into the bf16 matrix-core kernel; MFMA-bound like the bf16
        # GEMM it replaces (compare with "bf16 4096").
        ("q4 prefill 4096^3 (G=64)", "bf16", lambda g: QCell(g, W.q4_prefill())),
    ]
    return cells


def counter_pass(g, reps: int, copy_bytes: int) -> None:
    """Untimed: every sweep cell `reps` steps in list order, then a plain device copy of
    `copy_bytes` three times.  A counter run over it (rocprofv3 --pmc) sees the library's
    dispatches in that order; the manifest printed to stderr gives each cell's count."""
    import torch
    for name, dtype, make in sweep_cells():
        c = make(g)
        for _ in range(reps):
            c.step()
        torch.cuda.synchronize()
        print(f"[counter-pass] cell={name!r} kernel={c.kernel} dtype={dtype} "
              f"dispatches={reps * c.launches_per_step} flops={c.p.flops} "
              f"bytes={c.algorithmic_bytes()}", file=sys.stderr, flush=True)
        del c
        torch.cuda.empty_cache()
    if copy_bytes:
        src = torch.empty(copy_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[counter-pass] copied {copy_bytes} bytes 3 times", file=sys.stderr, flush=True)


def recipe_hash(recipe: dict) -> str:
    """Hash of a workload's input recipe (sizes, types, distributions, seed, RNG, draw order)."""
    blob = json.dumps(recipe, sort_keys=True, default=str).encode()
    return hashlib.sha256(blob).hexdigest()[:16]


def graph_time(cell, per_graph: int = 20, replays: int = 20):
    """Per-step period (ms) with `per_graph` steps captured in one HIP graph and replayed
    `replays` times between one event pair: the GPU's own launch-to-launch period, without the
    host's per-call cost, which bounds the back-to-back loop of the small cells.  None if the
    capture fails (the timed results stand without it)."""
    import torch
    try:
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # a launch off the default stream before capture
            cell.step(side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream().cuda_stream
            for _ in range(per_graph):
                cell.step(cs)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (replays * per_graph)
        del graph
        return ms
    except RuntimeError as e:
        print(f"[bench] graph timing unavailable: {e}", file=sys.stderr, flush=True)
        return None


def summarize(name, cell: Cell, ms: np.ndarray, dtype: str) -> dict:
    p = cell.p
    med = float(np.median(ms))
    lo, hi = bootstrap_ci(ms)
    tf = p.flops / (med * 1e-3) / 1e12
    row = {"cell": name, "kernel": cell.kernel, "M": p.M, "N": p.N, "K": p.K, "dtype": dtype,
           "seed": p.recipe.get("seed"), "recipe_hash": recipe_hash(p.recipe),
           "flops": int(p.flops), "reps": int(len(ms)), "median_us": round(med * 1e3, 3),
           "ci95_us": [round(hi_ * 1e3, 3) for hi_ in (lo, hi)],
           # the spread of single reps: a second clock state would show as a wide p5..p95
           "p05_us": round(float(np.percentile(ms, 5)) * 1e3, 3),
           "p95_us": round(float(np.percentile(ms, 95)) * 1e3, 3),
           "tflops": round(tf, 2),
           "tflops_ci95": [round(p.flops / (hi * 1e-3) / 1e12, 2),
                           round(p.flops / (lo * 1e-3) / 1e12, 2)],
           "pct_peak": round(100 * tf / PEAK_TFLOPS[dtype], 2),
           "alg_bytes": int(cell.algorithmic_bytes()),
           "gbs": round(cell.algorithmic_bytes() / (med * 1e-3) / 1e9, 1),
           "back_to_back_us": round(getattr(cell, "b2b_ms", float("nan")) * 1e3, 3),
           "sclk_after_run_mhz": getattr(cell, "sclk", None)}
    print(f"[bench] {name:34s} {cell.kernel:8s} {row['median_us']:10.2f} us  "
          f"{row['tflops']:8.1f} TFLOP/s  {row['pct_peak']:5.1f}% of {dtype} peak  "
          f"{row['gbs']:8.1f} GB/s  (back to back {row['back_to_back_us']:.2f} us)"
          f"{'' if row['sclk_after_run_mhz'] is None else '  sclk after %.0f MHz' % row['sclk_after_run_mhz']['mean']}",
          file=sys.stderr, flush=True)
    return row


def read_counters(src_hash: str) -> dict:
    """Figures from the committed counter summary of the headline kernel, if it saw this
    source: HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size)
    and the shader clock during the kernel (GRBM_GUI_ACTIVE cycles / 8 XCDs / duration)."""
    out = {"traffic": None, "sclk_in_kernel_mhz": None, "mfma_busy": None}
    try:
        fields = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    fields[k.strip()] = v.split()[0] if v.split() else ""
        if fields.get("source_hash") != src_hash:
            return out
        out["traffic"] = int(float(fields["hbm_bytes_per_launch"]))
        out["sclk_in_kernel_mhz"] = float(fields["shader_clock_in_kernel_mhz"])
        out["mfma_busy"] = float(fields["mfma_busy_fraction"])
    except (OSError, KeyError, ValueError):
        pass
    return out


def gate_points(M: int, N: int, n: int, seed: int):
    """n output coordinates for the checksum gate: the four corners, then seeded uniform
    draws (numpy PCG64)."""
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, max(0, n - 4))])
    cols = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, max(0, n - 4))])
    return rows.astype(np.int64), cols.astype(np.int64)


def gate_sample(p, sample: dict, quantized: bool, unfused: bool):
    """The checksum gate ("Rigel" section 3: a float64 reference from the same stored bytes,
    per-dtype tolerance) on a cell's sampled outputs: part of the CPU leg, which alone calls
    the oracle.  Returns the gate's verdict as a dict."""
    import oracle
    from oracle import gate
    import workloads as W
    rows, cols = sample["rows"], sample["cols"]
    if quantized:
        Cref, D = oracle.qgemm_points(p, rows, cols)
        ct = p.x_type
    else:
        Cref, D = oracle.gemm_points(p, rows, cols)
        ct = p.c_type
    gelu = bool(p.epilogue & W.EPI_GELU)
    tol = gate.tolerance(p.K, ct, 2 if unfused else 1, gelu)
    cin = oracle.decode(ct, p.C[rows, cols]) if p.beta != 0 else None
    res = gate.check(oracle.decode(ct, sample["raw"]), Cref, D, tol, ct, p.beta, cin)
    return {"n": res.n_checked, "max_err": res.max_err, "tol": res.tol, "pass": res.ok,
            "c_type": ct, "roundings": 2 if unfused else 1, "gelu": gelu}


CSV_FIELDS = ("cell", "kernel", "dtype", "c_type", "M", "N", "K", "flops", "seed", "recipe_hash",
              "reps", "median_us", "ci95_lo_us", "ci95_hi_us", "p05_us", "p95_us", "tflops",
              "peak_tflops",
              "pct_peak", "alg_bytes", "gbs", "graph_us", "sclk_after_run_mhz", "gate_n",
              "gate_max_err", "gate_tol", "gate_roundings", "gate_gelu", "gate_pass", "commit",
              "sources", "gpu", "cus", "hip", "torch")


def write_csv(path: str, rows: list, prov: dict, src_hash: str) -> None:
    """One line per cell (the headline first): the raw measurements, the derived rates and the
    gate's numbers, with the provenance each line needs to be used ("Rigel" section 3)."""
    import csv
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=CSV_FIELDS)
        w.writeheader()
        for r in rows:
            gt = r.get("gate") or {}
            w.writerow({"cell": r["cell"], "kernel": r["kernel"], "dtype": r["dtype"],
                        "c_type": gt.get("c_type", ""), "M": r["M"], "N": r["N"], "K": r["K"],
                        "flops": r["flops"], "seed": r["seed"], "recipe_hash": r["recipe_hash"],
                        "reps": r["reps"], "median_us": r["median_us"],
                        "ci95_lo_us": r["ci95_us"][0], "ci95_hi_us": r["ci95_us"][1],
                        "p05_us": r.get("p05_us", ""), "p95_us": r.get("p95_us", ""),
                        "tflops": r["tflops"], "peak_tflops": PEAK_TFLOPS[r["dtype"]],
                        "pct_peak": r["pct_peak"], "alg_bytes": r.get("alg_bytes", ""),
                        "gbs": r.get("gbs", ""), "graph_us": r.get("graph_us"),
                        "sclk_after_run_mhz": (r.get("sclk_after_run_mhz") or {}).get("mean", ""),
                        "gate_n": gt.get("n", ""), "gate_max_err": gt.get("max_err", ""),
                        "gate_tol": gt.get("tol", ""), "gate_roundings": gt.get("roundings", ""),
                        "gate_gelu": gt.get("gelu", ""), "gate_pass": gt.get("pass", ""),
                        "commit": prov.get("git_commit") or "", "sources": src_hash,
                        "gpu": f'{prov.get("gpu", "")} {prov.get("gcn_arch", "")}'.strip(),
                        "cus": prov.get("cus", ""), "hip": prov.get("hip", ""),
                        "torch": prov.get("torch", "")})


# The re-verifier restates what it checks from the published figures, not from the code that
# wrote the file: the dense peaks of MI355X per input type (TFLOP/s) and the gate's tolerance,
# K 2^-23 + (1 + (roundings - 1) 1.1289) u_out + 4 2^-24 (+ 16 2^-24 with GELU), with u_out
# the unit roundoff of the output type.
_RV_PEAK = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2,
            "e2m1": 10066.3, "e2m3": 10066.3, "e3m2": 10066.3}
_RV_U = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def reverify(path: str) -> int:
    """Re-derive every line's rates and gate verdict from its raw columns and report the lines
    that disagree (no GPU, no oracle): flops = 2 M N K; TFLOP/s from the median; the % of the
    type's peak; GB/s from the algorithmic bytes and the median; the median inside its 95%
    interval and between the 5th and 95th percentiles of the reps; pass exactly when
    max_err <= tol, with the tolerance recomputed; provenance present.  Returns the number of
    disagreeing lines."""
    import csv
    bad = 0
    with open(path, newline="") as fh:
        lines = list(csv.DictReader(fh))
    for ln in lines:
        why = []
        M, N, K = int(ln["M"]), int(ln["N"]), int(ln["K"])
        med = float(ln["median_us"])
        if int(float(ln["flops"])) != 2 * M * N * K:
            why.append("flops")
        tf = 2.0 * M * N * K / (med * 1e-6) / 1e12
        if abs(tf - float(ln["tflops"])) > 0.01 + 1e-3 * tf:
            why.append(f"tflops {ln['tflops']} vs {tf:.2f}")
        peak = _RV_PEAK.get(ln["dtype"])
        if peak is None or abs(float(ln["peak_tflops"]) - peak) > 1e-6:
            why.append("peak")
        elif abs(100 * tf / peak - float(ln["pct_peak"])) > 0.02:
            why.append(f"pct_peak {ln['pct_peak']} vs {100 * tf / peak:.2f}")
        if not float(ln["ci95_lo_us"]) <= med <= float(ln["ci95_hi_us"]):
            why.append("median outside its interval")
        if ln.get("p05_us") not in (None, "") and not (
                float(ln["p05_us"]) <= med <= float(ln["p95_us"])):
            why.append("median outside p5..p95")
        if ln.get("alg_bytes") not in (None, ""):
            gbs = int(float(ln["alg_bytes"])) / (med * 1e-6) / 1e9
            if abs(gbs - float(ln["gbs"])) > 0.1 + 1e-3 * gbs:
                why.append(f"gbs {ln['gbs']} vs {gbs:.1f}")
        if ln["gate_pass"] == "":
            why.append("not gated")
        else:
            u = _RV_U.get(ln["c_type"])
            rnd = int(ln["gate_roundings"])
            gelu = ln["gate_gelu"] == "True"
            tol = (K * 2.0 ** -23 + (1.0 + (rnd - 1) * 1.1289) * u + 4 * 2.0 ** -24
                   + (16 * 2.0 ** -24 if gelu else 0.0)) if u is not None else None
            if tol is None or abs(tol - float(ln["gate_tol"])) > 1e-12 * max(1.0, tol):
                why.append("tolerance")
            verdict = float(ln["gate_max_err"]) <= float(ln["gate_tol"])
            if verdict != (ln["gate_pass"] == "True"):
                why.append("verdict")
            if not verdict:
                why.append("fails the gate")
        # a tree copied without its history has no commit; the source hash names it instead
        for f in ("sources", "gpu", "cus", "recipe_hash", "seed"):
            if ln[f] in ("", "None"):
                why.append(f"no {f}")
        if why:
            bad += 1
            print(f"[reverify] {ln['cell']}: " + "; ".join(why))
    print(f"[reverify] {len(lines) - bad} of {len(lines)} lines agree")
    return bad


def _span(ln: dict) -> str:
    if ln.get("p05_us") in (None, ""):
        return "—"
    return f"{float(ln['p05_us']):.2f}–{float(ln['p95_us']):.2f}"


def replot(path: str) -> str:
    """The table of cells regenerated from the CSV alone (no GPU): markdown, one row per cell."""
    import csv
    with open(path, newline="") as fh:
        lines = list(csv.DictReader(fh))
    out = ["| Cell | Kernel | Median (95% CI) | p5–p95 | TFLOP/s | % of peak | GB/s | Gate |",
           "|---|---|---|---|---|---|---|---|"]
    for ln in lines:
        gate = ("—" if ln["gate_pass"] == "" else
                f"{'pass' if ln['gate_pass'] == 'True' else 'FAIL'} ({float(ln['gate_max_err']) / float(ln['gate_tol']):.1%} of tol, n={ln['gate_n']})")
        out.append(f"| {ln['cell']} | {ln['kernel']} | {float(ln['median_us']):.2f} µs "
                   f"({float(ln['ci95_lo_us']):.2f}–{float(ln['ci95_hi_us']):.2f}) | "
                   f"{_span(ln)} | "
                   f"{float(ln['tflops']):.1f} | {float(ln['pct_peak']):.1f} | "
                   f"{ln.get('gbs') or '—'} | {gate} |")
    return "\n".join(out)


def cpu_baseline(p, target_s: float) -> dict:
    """The oracle, as it stands, on a bounded sample of the headline problem: the first rows
    of the M x N result (all N columns, full K), timed with a monotonic clock."""
    import oracle
    oracle.lib()
    t0 = time.perf_counter()
    oracle.gemm_rows(p, 0, 8)
    t_probe = time.perf_counter() - t0
    rows = int(max(8, min(p.M, 8 * target_s / max(t_probe, 1e-3))))
    t0 = time.perf_counter()
    ref = oracle.gemm_rows(p, 0, rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * p.N * p.K
    cpu_baseline.computed = (rows, ref)  # the rows it computed, for the headline's gate
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {p.M}x{p.N}x{p.K} bf16+bias+GELU problem "
                      f"(all {p.N} columns, K={p.K}, float64, plus the |a*b| denominator sums), "
                      f"{dt:.1f} s",
            "seconds": round(dt, 2)}


def provenance(src_hash: str) -> dict:
    import torch
    prop = torch.cuda.get_device_properties(0)
    try:
        hipcc = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True,
                               text=True, timeout=30).stdout.splitlines()[0]
    except Exception:
        hipcc = "unknown"
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        commit = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                                capture_output=True, text=True, timeout=10).stdout.strip()
    except Exception:
        commit = ""
    return {"gpu": prop.name, "gcn_arch": getattr(prop, "gcnArchName", ""),
            "cus": prop.multi_processor_count, "hip": torch.version.hip, "hipcc": hipcc,
            "torch": torch.__version__, "host_cpu": cpu,
            "host_cores": len(os.sched_getaffinity(0)), "source_hash": src_hash,
            "git_commit": commit or None, "python": platform.python_version()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300, help="timed steps (headline)")
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed warm-up steps (headline), run after the time-based settle")
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="back-to-back headline steps for at least this long before the warm-up "
                         "steps, whatever --warmup says (clocks and power settle)")
    ap.add_argument("--reps", type=int, default=300, help="timed reps per sweep cell")
    ap.add_argument("--no-sweeps", action="store_true")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle CPU baseline and, with it, the checksum gate")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--headline-only-loop", type=int, default=0,
                    help="run only N headline steps (for profiler passes) and exit")
    ap.add_argument("--loop-cell", default="headline",
                    choices=["headline", "q4_decode", "q4_prefill"],
                    help="with --headline-only-loop: the workload to run instead of the headline")
    ap.add_argument("--counter-pass", type=int, default=0,
                    help="run every sweep cell this many times, untimed, for counter runs, and exit")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="with --headline-only-loop: also run a plain device copy of this many "
                         "bytes three times (a known-size reference for HBM byte counters)")
    ap.add_argument("--csv", default="",
                    help="also write one line per cell (measurements, rates, gate, provenance) "
                         "to this CSV file")
    ap.add_argument("--reverify", default="",
                    help="re-derive every rate and gate verdict of a results CSV and exit "
                         "(no GPU); nonzero exit status when a line disagrees")
    ap.add_argument("--replot", default="",
                    help="print the table of cells regenerated from a results CSV and exit "
                         "(no GPU)")
    args = ap.parse_args()

    if args.reverify:
        sys.exit(1 if reverify(args.reverify) else 0)
    if args.replot:
        print(replot(args.replot))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE={world}) requested, but the library is a "
              f"single-GPU GEMM: there is no sharded path and no collective. Run --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_matrix_multiply_amd as tmm
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    g = tmm.Gemm(0)
    src_hash = source_hash()

    head_p = W.bf16_bias_gelu(4096)
    head = Cell(g, head_p)
    print(f"[bench] headline: bf16 GEMM+bias+GELU 4096^3 fused, kernel {head.kernel}",
          file=sys.stderr, flush=True)

    if args.counter_pass:
        counter_pass(g, args.counter_pass, args.copy_bytes)
        return

    if args.headline_only_loop:
        if args.loop_cell == "headline":
            loop = head
        else:
            # the decode cycles three weight copies, as in the sweep, so that each launch reads
            # its weights from HBM
            qp = W.q4_decode() if args.loop_cell == "q4_decode" else W.q4_prefill()
            loop = QCell(g, qp, copies=3 if args.loop_cell == "q4_decode" else 1)
            print(f"[bench] loop cell {args.loop_cell}, kernel {loop.kernel}", file=sys.stderr)
        for _ in range(args.headline_only_loop):
            loop.step()
        torch.cuda.synchronize()
        print(f"[bench] ran {args.headline_only_loop} {args.loop_cell} steps", file=sys.stderr)
        if args.copy_bytes:
            src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(f"[bench] copied {args.copy_bytes} bytes 3 times", file=sys.stderr)
        return

    # Headline.  A time-based settle (>= --settle-seconds of back-to-back steps, whatever
    # --warmup says: the clock and power state need wall time, not a step count), then the W
    # untimed warm-up steps, then exactly K back-to-back steps between two synchronisations,
    # with one HIP event pair around them on the launch stream: their period is the average
    # launch period (launch to launch), from which the roofline's achieved rate is taken.  The
    # shader clock is sampled over the end of the settle and the timed steps.  A second pass
    # times each step with its own event pair for the median and its bootstrap CI.
    clock = ClockProbe(g)
    settle_steps = head.settle(args.settle_seconds)
    for _ in range(args.warmup):
        head.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(head.stream)
    for _ in range(args.steps):
        head.step()
    e1.record(head.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the clock right behind a second, identical run of K steps (not inside the timed region)
    for _ in range(args.steps):
        head.step()
    clock.enqueue(head.stream.cuda_stream)
    torch.cuda.synchronize()
    head_sclk = clock.read()
    ms_per_step = wall * 1e3 / args.steps
    value = head_p.flops / (ms_per_step * 1e-3) / 1e12
    period_ms = e0.elapsed_time(e1) / args.steps
    achieved = head_p.flops / (period_ms * 1e-3) / 1e12
    print(f"[bench] headline: settle {settle_steps} steps ({args.settle_seconds:.2f} s), warm-up "
          f"{args.warmup}, {args.steps} timed steps: {period_ms * 1e3:.2f} us per launch "
          f"({achieved:.1f} TFLOP/s), wall {ms_per_step * 1e3:.2f} us per step"
          f"{'' if head_sclk is None else ', sclk %.0f MHz' % head_sclk['mean']}",
          file=sys.stderr, flush=True)
    ms = head.time(max(args.steps, 30), warmup_s=0.05, clock=clock)
    head_row = summarize("bf16+bias+GELU fused 4096 (headline)", head, ms, "bf16")

    hbm = None if args.no_sweeps else hbm_ceiling(g)
    sweeps = []
    gate_in = []  # (sweep index, problem, quantized, unfused, sampled outputs)
    if not args.no_sweeps:
        for name, dtype, make in sweep_cells():
            c = make(g)
            row = summarize(name, c, c.time(args.reps, clock=clock), dtype)
            if not args.no_cpu:
                gate_in.append((len(sweeps), c.p, isinstance(c, QCell), getattr(c, "unfused", False),
                                c.result_sample(seed=len(sweeps))))
            gms = graph_time(c)
            row["graph_us"] = round(gms * 1e3, 3) if gms is not None else None
            if gms is not None:
                print(f"[bench] {'':34s} {row['graph_us']:.2f} us per step in a HIP graph",
                      file=sys.stderr, flush=True)
            if isinstance(c, QCell) and c.p.M <= 4:
                row["pct_hbm"] = round(100 * row["gbs"] / PEAK_HBM_GBS, 2)
                if hbm is not None:
                    row["pct_read_ceiling"] = round(100 * row["gbs"] / hbm["read_gbs"], 2)
                    row["pct_copy_ceiling"] = round(100 * row["gbs"] / hbm["copy_gbs"], 2)
                print(f"[bench] {'':34s} {row['pct_hbm']:.1f}% of HBM peak"
                      f"{'' if hbm is None else ', %.1f%% of the measured read ceiling' % row['pct_read_ceiling']} "
                      f"({c.algorithmic_bytes() / 1e6:.1f} MB per launch)", file=sys.stderr,
                      flush=True)
            sweeps.append(row)
            del c
            torch.cuda.empty_cache()

    cpu = None
    head_gate = None
    gate_failures = None  # None: not gated (--no-cpu)
    if not args.no_cpu:
        print("[bench] timing the oracle on the host (bounded sample) ...", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(head_p, args.cpu_seconds)
        # The checksum gate on what the oracle computed here: the headline's sampled rows (all
        # columns), and each sweep cell's sampled outputs.
        import oracle
        from oracle import gate
        rows, (Cref, D) = cpu_baseline.computed
        got = head.C[:rows].cpu().numpy().view(np.uint16)
        tol = gate.tolerance(head_p.K, "bf16", 1, True)
        res = gate.check(oracle.decode("bf16", got), Cref, D, tol, "bf16")
        head_gate = {"n": res.n_checked, "max_err": res.max_err, "tol": res.tol, "pass": res.ok,
                     "c_type": "bf16", "roundings": 1, "gelu": True}
        head_row["gate"] = head_gate
        for i, pp, quantized, unfused, sample in gate_in:
            sweeps[i]["gate"] = gate_sample(pp, sample, quantized, unfused)
        n_pass = sum(1 for r in sweeps if r.get("gate", {}).get("pass")) + int(head_gate["pass"])
        print(f"[bench] checksum gate: {n_pass} of {len(sweeps) + 1} cells pass "
              f"(headline: {res})", file=sys.stderr, flush=True)
        # a cell that fails its gate is reported by name: its rate is not a result
        gate_failures = [r["cell"] for r in [head_row] + sweeps
                         if r.get("gate") is not None and not r["gate"]["pass"]]
        if gate_failures:
            print(f"[bench] FAIL: these cells do not match the oracle: {gate_failures}",
                  file=sys.stderr, flush=True)

    counters = read_counters(src_hash)
    kclk = counters["sclk_in_kernel_mhz"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": args.settle_seconds, "steps": settle_steps},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy draws: A~N(0,1), B~N(0,1/K), bias~N(0,0.01); bf16 RNE)",
        "config": {"workload": "bf16 GEMM + bias + erf-GELU fused, M=N=K=4096, row-major NN, "
                               "fp32 accumulate, bf16 out",
                   "M": 4096, "N": 4096, "K": 4096, "kernel": head.kernel,
                   "seed": head_p.recipe["seed"], "recipe_hash": recipe_hash(head_p.recipe)},
        "pct_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
        "median_tflops": head_row["tflops"],
        "ci95_tflops": head_row["tflops_ci95"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": counters["traffic"],
                     "launch_period_us": round(period_ms * 1e3, 3),
                     "flops_per_launch": head_p.flops,
                     # the clock the power controller held during the kernel (counter pass of
                     # this source), and the frac against the peak at that clock
                     "sclk_in_kernel_mhz": kclk,
                     "frac_at_in_kernel_sclk": (round(achieved / (PEAK_TFLOPS["bf16"] * kclk / 2400.0), 4)
                                                if kclk else None),
                     "mfma_busy": counters["mfma_busy"],
                     # a probe queued right behind a second run: the clock has recovered by then
                     "sclk_after_run_mhz": head_sclk},
        "sclk_after_run_mhz": head_sclk["mean"] if head_sclk else None,
        "hbm_copy_gbs": hbm["copy_gbs"] if hbm else None,
        "hbm_read_gbs": hbm["read_gbs"] if hbm else None,
        "hbm_ceiling": hbm,
        "cpu_baseline": cpu,
        "gate": head_gate,
        "gate_failures": gate_failures,
        "sweeps": sweeps,
        "provenance": provenance(src_hash),
    }
    if args.csv:
        write_csv(args.csv, [head_row] + sweeps, out["provenance"], src_hash)
    print(json.dumps(out), flush=True)
    g.close()


if __name__ == "__main__":
    main()
