"""Host-side pieces of bench.py that need no GPU: the counter-summary reader, the bootstrap
confidence interval, the source hash and the single-GPU refusal."""
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
