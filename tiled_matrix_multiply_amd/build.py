"""Builds tiled_matrix_multiply_amd/libgemm.so from csrc/ with hipcc for gfx950 only.

Every source is compiled in parallel into _build/, then linked into one shared library whose
exported symbols are exactly the C ABI of include/gemm.h.

Beside it, libgemm_lds_poison.so: the same library with the matrix-core kernels of the main
families (fp32, fp16, bf16, per-tensor and block-scaled E4M3, E2M1 and E2M3, quantized B)
built with
GEMM_DEBUG_POISON_LDS, which fills every LDS stage with all-ones words before it is refilled.
It is a race check for the staged K loop: its results must equal libgemm.so's bit for bit.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemm.so")
LIB_POISON = os.path.join(PKG, "libgemm_lds_poison.so")
POISON_SOURCES = ("mfma_f32.hip", "mfma_f16.hip", "mfma_bf16.hip", "mfma_e4m3.hip",
                  "mfma_mx_e4m3.hip", "mfma_e2m1.hip", "mfma_e2m3.hip", "qmfma.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
]
# Device code: gfx950 only; packed fp32 instructions are disabled for all HIP code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool, poison: bool = False) -> str:
    stem = os.path.splitext(src)[0] + ("_lds_poison" if poison else "")
    obj = os.path.join(BUILD, stem + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC, *COMMON] + (["-DGEMM_DEBUG_POISON_LDS"] if poison else [])
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    cmd += ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return obj


def _link(objs: list, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    srcs = sources()
    poison = [s for s in srcs if s in POISON_SOURCES]
    assert len(poison) == len(POISON_SOURCES), "a race-check source is missing from csrc/"
    # the largest translation units first, so the pool does not end on one of them
    work = [(s, True) for s in poison] + [(s, False) for s in srcs]
    jobs = jobs or min(len(work), max(1, os.cpu_count() or 1), 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        built = dict(zip(work, ex.map(lambda w: _compile(w[0], verbose, w[1]), work)))
    _link([built[(s, False)] for s in srcs], LIB, verbose)
    _link([built[(s, s in POISON_SOURCES)] for s in srcs], LIB_POISON, verbose)
    if verbose:
        print(f"built {LIB} and {LIB_POISON} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
