"""Host-side pieces of bench.py that need no GPU: the counter-summary reader, the bootstrap
confidence interval, the source hash, the single-GPU refusal, the gate's sample points, and the
re-verifier and replot of a results CSV."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _summary(tmp_path, source_hash):
    f = tmp_path / "traffic.txt"
    f.write_text("# header = ignored\n"
                 f"source_hash = {source_hash}\n"
                 "hbm_bytes_per_launch = 235408250\n"
                 "mfma_busy_fraction = 0.528   (SQ_VALU_MFMA_BUSY_CYCLES / ...)\n"
                 "shader_clock_in_kernel_mhz = 1991   (GRBM_GUI_ACTIVE / 8 XCDs / ...)\n")
    return str(f)


def test_read_counters_matches_only_its_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, "abc123"))
    got = bench.read_counters("abc123")
    assert got == {"traffic": 235408250, "sclk_in_kernel_mhz": 1991.0, "mfma_busy": 0.528}
    # a summary taken from other sources is not reported
    assert bench.read_counters("def456") == {"traffic": None, "sclk_in_kernel_mhz": None,
                                             "mfma_busy": None}


def test_read_counters_missing_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.read_counters("abc123")["traffic"] is None


def test_source_hash_tracks_content(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hpp", tmp_path / "b.hpp"
    a.write_text("one")
    b.write_text("two")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash(("a.hpp", "b.hpp"))
    assert h == bench.source_hash(("a.hpp", "b.hpp")) and len(h) == 16
    b.write_text("two, edited")
    assert bench.source_hash(("a.hpp", "b.hpp")) != h


def test_bootstrap_ci_brackets_the_median():
    x = np.random.default_rng(1).normal(100.0, 3.0, size=300)
    lo, hi = bench.bootstrap_ci(x)
    assert lo < np.median(x) < hi
    assert hi - lo < 2.0  # about 2 x 1.96 x 1.25 sigma / sqrt(300)
    assert (lo, hi) == bench.bootstrap_ci(x)  # fixed seed: reproducible


def test_bootstrap_ci_of_a_constant_sample():
    assert bench.bootstrap_ci(np.full(50, 7.0)) == (7.0, 7.0)


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and r.stdout == ""


def _results_csv(path, **override):
    """A two-line results CSV whose derived columns follow from its raw ones."""
    import csv
    M = N = K = 4096
    med = 113.2
    tf = 2.0 * M * N * K / (med * 1e-6) / 1e12
    tol = K * 2.0 ** -23 + 2.0 ** -8 + 4 * 2.0 ** -24 + 16 * 2.0 ** -24
    base = {"cell": "bf16+bias+GELU fused 4096 (headline)", "kernel": "mfma256", "dtype": "bf16",
            "c_type": "bf16", "M": M, "N": N, "K": K, "flops": 2 * M * N * K, "seed": 3,
            "recipe_hash": "abc", "reps": 300, "median_us": med, "ci95_lo_us": 113.0,
            "ci95_hi_us": 113.5, "p05_us": 112.1, "p95_us": 115.0, "tflops": round(tf, 2), "peak_tflops": 2516.6,
            "pct_peak": round(100 * tf / 2516.6, 2), "alg_bytes": 100663296 + 16384,
            "gbs": round((100663296 + 16384) / (med * 1e-6) / 1e9, 1), "graph_us": 113.1,
            "sclk_after_run_mhz": 2410.0, "gate_n": 4096,
            "gate_max_err": tol / 10, "gate_tol": tol, "gate_roundings": 1, "gate_gelu": True,
            "gate_pass": True, "commit": "deadbee", "sources": "0123", "gpu": "MI355X",
            "cus": 256}
    M2, K2 = 1000, 1000
    med2 = 27.0
    tf2 = 2.0 * M2 * M2 * K2 / (med2 * 1e-6) / 1e12
    second = dict(base, cell="fp32 1000", kernel="mfma64", dtype="f32", c_type="f32", M=M2, N=M2,
                  K=K2, flops=2 * M2 * M2 * K2, median_us=med2, ci95_lo_us=26.9, ci95_hi_us=27.1,
                  p05_us=26.5, p95_us=27.6,
                  tflops=round(tf2, 2), peak_tflops=157.3, pct_peak=round(100 * tf2 / 157.3, 2),
                  alg_bytes=16000000, gbs=round(16000000 / (med2 * 1e-6) / 1e9, 1),
                  gate_tol=K2 * 2.0 ** -23 + 2.0 ** -24 + 4 * 2.0 ** -24, gate_gelu=False,
                  gate_max_err=1e-7)
    second.update(override)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=bench.CSV_FIELDS)
        w.writeheader()
        w.writerow(base)
        w.writerow(second)


def test_reverify_agrees_with_a_consistent_csv(tmp_path):
    path = tmp_path / "cells.csv"
    _results_csv(path)
    assert bench.reverify(str(path)) == 0
    table = bench.replot(str(path))
    assert "fp32 1000" in table and "mfma256" in table and "pass" in table


@pytest.mark.parametrize("override", [
    {"tflops": 80.0},                        # a rate that does not follow from the median
    {"pct_peak": 50.0},                      # a fraction of the wrong peak
    {"flops": 2 * 1000 ** 3 + 2},            # flops that are not 2 M N K
    {"gate_pass": False},                    # a verdict the numbers contradict
    {"gate_max_err": 1.0, "gate_pass": False},  # an honest failure still counts as a bad line
    {"gate_tol": 1e-3},                      # a tolerance not recomputable from K and the type
    {"ci95_lo_us": 27.5},                    # a median outside its interval
    {"gbs": 1000.0},                         # a bandwidth that does not follow from the median
    {"p95_us": 26.95},                       # a median above the 95th percentile
    {"sources": ""},                         # missing provenance
])
def test_reverify_catches_each_inconsistency(tmp_path, override):
    path = tmp_path / "cells.csv"
    _results_csv(path, **override)
    assert bench.reverify(str(path)) == 1


def test_gate_points_include_the_corners():
    rows, cols = bench.gate_points(300, 500, 64, 0)
    assert len(rows) == len(cols) == 64
    assert {(0, 0), (0, 499), (299, 0), (299, 499)} <= set(zip(rows.tolist(), cols.tolist()))
    assert rows.max() < 300 and cols.max() < 500


def test_the_committed_results_csv_reverifies(capsys):
    """The results CSV kept beside the profiles re-derives line by line, every cell passes its
    gate, and every sweep cell is present."""
    path = os.path.join(ROOT, "profiles", "bench_cells.csv")
    assert bench.reverify(path) == 0
    out = capsys.readouterr().out
    assert out.strip().splitlines()[-1] == "[reverify] 24 of 24 lines agree"


def test_write_csv_carries_the_provenance(tmp_path):
    """The commit, the architecture and the CU count reach their columns; the derived columns
    of the line written re-verify."""
    import csv
    M = N = K = 1024
    med = 10.0
    row = {"cell": "fp16 1024", "kernel": "mfma64", "dtype": "f16", "M": M, "N": N, "K": K,
           "flops": 2 * M * N * K, "seed": 2, "recipe_hash": "abc", "reps": 300,
           "median_us": med, "ci95_us": (9.9, 10.1),
           "tflops": round(2.0 * M * N * K / (med * 1e-6) / 1e12, 2),
           "pct_peak": round(100 * 2.0 * M * N * K / (med * 1e-6) / 1e12 / 2516.6, 2),
           "graph_us": 9.0,
           "gate": {"n": 512, "max_err": 1e-5, "tol": K * 2.0 ** -23 + 2.0 ** -11 + 4 * 2.0 ** -24,
                    "pass": True, "c_type": "f16", "roundings": 1, "gelu": False}}
    prov = {"git_commit": "abc1234", "gpu": "AMD Radeon Graphics", "gcn_arch": "gfx950:sramecc+",
            "cus": 256}
    path = tmp_path / "cells.csv"
    bench.write_csv(str(path), [row], prov, "0123456789abcdef")
    with open(path) as fh:
        line = next(csv.DictReader(fh))
    assert line["commit"] == "abc1234"
    assert line["gpu"] == "AMD Radeon Graphics gfx950:sramecc+"
    assert line["cus"] == "256" and line["sources"] == "0123456789abcdef"
    assert bench.reverify(str(path)) == 0
