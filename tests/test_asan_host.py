"""The host code of the C ABI under AddressSanitizer, on the CPU: tests/asan/run.sh compiles
api.cpp and qapi.cpp instrumented (host code only), links them with the device objects of the
normal build, and runs tests/asan/driver.c over the argument checks, null handles and
gemm_create without a GPU.  Any sanitizer report makes the driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUN = os.path.join(ROOT, "tests", "asan", "run.sh")
BUILD = os.path.join(ROOT, "tiled_matrix_multiply_amd", "_build")


def test_host_code_is_clean_under_asan():
    if not os.path.exists("/opt/rocm/llvm/bin/clang") or shutil.which("bash") is None:
        pytest.skip("no ROCm clang")
    if not os.path.exists(RUN):
        pytest.skip("tests/asan is not in this copy of the tree")
    assert os.path.exists(os.path.join(BUILD, "api.o")), "build the library first"
    r = subprocess.run(["bash", RUN], capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("[asan]")]
    assert line and "null-handle checks ok" in line[0], out[-2000:]
