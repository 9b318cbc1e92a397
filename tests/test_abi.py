"""C ABI checks that need no GPU: every declared symbol is exported, argument validation and
status codes behave as include/gemm.h states, and the binding has no fallback path."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")

tmm = pytest.importorskip("tiled_matrix_multiply_amd")

F32, F16, BF16, E4M3 = tmm.GEMM_F32, tmm.GEMM_F16, tmm.GEMM_BF16, tmm.GEMM_E4M3
BIAS, GELU = tmm.GEMM_EPI_BIAS, tmm.GEMM_EPI_GELU


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GEMM_API\s+[\w\s\*]*?\b(gemm_\w+)\s*\(", text)))


@pytest.mark.parametrize("lib", ["libgemm.so", "libgemm_lds_poison.so"])
def test_every_declared_symbol_is_exported(lib):
    """The library and its LDS race-check build both export exactly the C ABI."""
    syms = declared_symbols()
    assert len(syms) == 23, syms
    assert sorted(tmm.EXPORTS) == syms
    path = os.path.join(os.path.dirname(tmm.LIB_PATH), lib)
    nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    for s in syms:
        assert s in exported, s
        assert hasattr(tmm.library(), s)
    # nothing but the C ABI is exported
    assert {s for s in exported if not s.startswith("gemm_")} == set(), exported


def test_measurement_helpers_validate_without_a_gpu():
    """The clock and bandwidth probes refuse a null handle before touching a device."""
    assert tmm.gemm_probe_clock(None, None, 0x1000, 256, 40) == tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_wall_clock_khz(None) == tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_kernel_workspace_bytes(None, tmm.GEMM_KERNEL_MFMA_256_SK, 512,
                                           512) == tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_probe_bandwidth(None, None, 0x1000, None, 1 << 20,
                                    0x2000) == tmm.GEMM_ERR_INVALID_HANDLE


def test_status_strings():
    for code in range(0, -9, -1):
        s = tmm.gemm_status_string(code)
        assert s.startswith("GEMM_")
    assert tmm.gemm_status_string(-99) == "GEMM_ERR_UNKNOWN"


# Fake, well-separated device addresses: gemm_check_args never dereferences them.
PA, PB, PC, PBIAS = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def chk(M=64, N=48, K=32, ta=0, tb=0, A=PA, lda=None, B=PB, ldb=None, C=PC, ldc=None, at=F32,
        bt=None, ct=None, epi=0, bias=None):
    bt = at if bt is None else bt
    ct = (BF16 if at == E4M3 else at) if ct is None else ct
    lda = (M if ta else K) if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tmm.gemm_check_args(M, N, K, ta, tb, A, lda, B, ldb, C, ldc, at, bt, ct, epi, bias)


def test_valid_arguments():
    assert chk() == tmm.GEMM_OK
    for at in (F32, F16, BF16, E4M3):
        for ta in (0, 1):
            for tb in (0, 1):
                assert chk(at=at, ta=ta, tb=tb, epi=BIAS | GELU, bias=PBIAS) == tmm.GEMM_OK


def test_invalid_values():
    V = tmm.GEMM_ERR_INVALID_VALUE
    assert chk(M=-1) == V and chk(N=-1) == V and chk(K=-1) == V
    assert chk(ta=2) == V and chk(tb=-1) == V
    assert chk(epi=4) == V
    assert chk(C=None) == V
    assert chk(A=None) == V and chk(B=None) == V
    assert chk(lda=31) == V                 # lda < K
    assert chk(ta=1, lda=63) == V           # A stored K x M: lda < M
    assert chk(ldb=47) == V                 # ldb < N
    assert chk(tb=1, ldb=31) == V           # B stored N x K: ldb < K
    assert chk(ldc=47) == V
    assert chk(epi=BIAS, bias=None) == V


def test_unsupported_tuples_and_sizes():
    U = tmm.GEMM_ERR_UNSUPPORTED
    assert chk(at=F32, ct=BF16) == U
    assert chk(at=E4M3, ct=E4M3) == U
    assert chk(at=E4M3, ct=F32) == U
    assert chk(at=BF16, bt=F16, ct=BF16) == U
    assert chk(at=7) == U
    assert chk(M=2 ** 31, lda=None) == U


def test_degenerate_sizes():
    OK = tmm.GEMM_OK
    assert chk(M=0, A=None, B=None, C=None) == OK          # no-op
    assert chk(N=0, A=None, B=None, C=None) == OK
    assert chk(K=0, A=None, B=None, lda=0, ldb=48) == OK   # C = epi(beta*C)
    assert chk(K=0, A=None, B=None, C=None) == tmm.GEMM_ERR_INVALID_VALUE


def test_aliasing():
    AL = tmm.GEMM_ERR_ALIAS
    assert chk(C=PA) == AL
    assert chk(C=PB + 4 * 100) == AL
    assert chk(C=PA + 4 * (64 * 32 - 1)) == AL              # overlaps A's last element
    assert chk(C=PA + 4 * (64 * 32)) == tmm.GEMM_OK          # just past A
    assert chk(epi=BIAS, bias=PC + 8) == AL


def test_null_handle_rejected_without_device():
    H = tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_run(None, None, 4, 4, 4, 0, 0, 1.0, PA, 4, 1.0, PB, 4, 1.0, 0.0, PC, 4, F32,
                        F32, F32, 0, None) == H
    assert tmm.gemm_run_kernel(None, 0, None, 4, 4, 4, 0, 0, 1.0, PA, 4, 1.0, PB, 4, 1.0, 0.0, PC,
                               4, F32, F32, F32, 0, None) == H
    assert tmm.gemm_select_kernel(None, 4, 4, 4, 0, 0, PA, 4, PB, 4, PC, 4, F32, F32, F32, 0,
                                  None) == H
    assert tmm.gemm_bias_gelu(None, None, 4, 4, PC, 4, F32, PBIAS, BIAS) == H
    tmm.gemm_destroy(None)


def test_create_without_gpu_reports_device_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(tmm.GemmError) as e:
        tmm.gemm_create(0)
    assert e.value.status == tmm.GEMM_ERR_DEVICE


def test_binding_fails_loudly_without_library(tmp_path):
    """No CPU fallback: importing the binding without libgemm.so raises ImportError."""
    pkg = tmp_path / "tiled_matrix_multiply_amd"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(os.path.join(ROOT, "tiled_matrix_multiply_amd",
                                                       "__init__.py")).read())
    code = "import tiled_matrix_multiply_amd"
    res = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True,
                         text=True)
    assert res.returncode != 0 and "ImportError" in res.stderr and "libgemm.so" in res.stderr


def test_product_path_never_touches_oracle():
    """Neither the library sources nor the binding import, load or name the oracle."""
    pkg = os.path.join(ROOT, "tiled_matrix_multiply_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, os.path.join(dirpath, f)


# --- 8- and 4-bit types and OCP MX block scales ------------------------------------------------

E5M2, E2M1 = tmm.GEMM_E5M2, tmm.GEMM_E2M1
PSA, PSB = 0x50000000, 0x60000000


def chk_mx(M=64, N=48, K=64, ta=0, tb=0, A=PA, lda=None, sa=PSA, ldsa=None, B=PB, ldb=None,
           sb=PSB, ldsb=None, C=PC, ldc=None, at=E4M3, bt=None, ct=BF16, epi=0, bias=None):
    bt = at if bt is None else bt
    lda = (M if ta else K) if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldsa = K // 32 if ldsa is None else ldsa
    ldsb = K // 32 if ldsb is None else ldsb
    ldc = N if ldc is None else ldc
    return tmm.gemm_check_args_mx(M, N, K, ta, tb, A, lda, sa, ldsa, B, ldb, sb, ldsb, C, ldc,
                                  at, bt, ct, epi, bias)


def test_low_precision_type_tuples():
    OK, U = tmm.GEMM_OK, tmm.GEMM_ERR_UNSUPPORTED
    for at in (E4M3, E5M2):
        for bt in (E4M3, E5M2):
            assert chk(at=at, bt=bt, ct=BF16) == OK
            assert chk(at=at, bt=bt, ct=F32) == U
    assert chk(at=E2M1, ct=BF16, tb=1) == OK
    assert chk(at=E2M1, bt=E4M3, ct=BF16) == U
    assert chk(at=E4M3, bt=E2M1, ct=BF16) == U
    assert chk(at=E2M1, ct=E2M1) == U


def test_packed_fp4_byte_ranges():
    """E2M1 rows take half a byte per element: A (64 x 32, lda 32) spans 1024 bytes."""
    AL, OK = tmm.GEMM_ERR_ALIAS, tmm.GEMM_OK
    assert chk(at=E2M1, ct=BF16, C=PA + 1023) == AL
    assert chk(at=E2M1, ct=BF16, C=PA + 1024) == OK
    # an odd element count rounds the last partly used byte up
    assert chk(at=E2M1, ct=BF16, M=1, K=3, lda=3, C=PA + 1) == AL
    assert chk(at=E2M1, ct=BF16, M=1, K=3, lda=3, C=PA + 2) == OK


def test_fp6_arguments():
    """The 6-bit types: any E2M3 / E3M2 pair with BF16 out, stored K-contiguous (A M x K, B N x
    K) with K, lda and ldb multiples of 4; rows take 3/4 of a byte per element."""
    OK, U, AL = tmm.GEMM_OK, tmm.GEMM_ERR_UNSUPPORTED, tmm.GEMM_ERR_ALIAS
    E2M3, E3M2 = tmm.GEMM_E2M3, tmm.GEMM_E3M2
    for at in (E2M3, E3M2):
        for bt in (E2M3, E3M2):
            assert chk(at=at, bt=bt, ct=BF16, tb=1) == OK
            assert chk_mx(at=at, bt=bt, tb=1) == OK
    assert chk(at=E2M3, ct=E2M3, tb=1) == U and chk(at=E2M3, ct=F32, tb=1) == U
    assert chk(at=E2M3, bt=E4M3, ct=BF16, tb=1) == U and chk(at=E2M1, bt=E3M2, ct=BF16, tb=1) == U
    assert chk(at=E2M3, ct=BF16, tb=0) == U and chk(at=E2M3, ct=BF16, ta=1, tb=1) == U
    assert chk(at=E2M3, ct=BF16, tb=1, K=30, lda=32, ldb=32) == U   # K % 4
    assert chk(at=E2M3, ct=BF16, tb=1, lda=34) == U                 # lda % 4
    # A: 64 rows x 32 elements (lda 32) = 64 * 24 bytes
    assert chk(at=E2M3, ct=BF16, tb=1, C=PA + 64 * 24 - 1) == AL
    assert chk(at=E2M3, ct=BF16, tb=1, C=PA + 64 * 24) == OK


def test_mx_arguments():
    OK, V, U, AL = (tmm.GEMM_OK, tmm.GEMM_ERR_INVALID_VALUE, tmm.GEMM_ERR_UNSUPPORTED,
                    tmm.GEMM_ERR_ALIAS)
    assert chk_mx() == OK
    assert chk_mx(at=E5M2, bt=E4M3) == OK and chk_mx(ta=1, tb=1) == OK
    assert chk_mx(at=E2M1, tb=1) == OK
    assert chk_mx(K=48, ldsa=2, ldsb=2) == V      # K must be a multiple of 32
    assert chk_mx(sa=None) == V and chk_mx(sb=None) == V
    assert chk_mx(ldsa=1) == V and chk_mx(ldsb=1) == V
    assert chk_mx(K=0, A=None, B=None, sa=None, sb=None, lda=0, ldb=48) == OK
    assert chk_mx(at=F16, ct=F16) == U and chk_mx(at=BF16, ct=BF16) == U
    assert chk_mx(C=PSA + 10) == AL               # C overlaps the A scales (64 x 2 bytes)
    assert chk_mx(C=PSA + 128) == OK
    assert chk_mx(C=PSB + 95) == AL and chk_mx(C=PSB + 96) == OK


def test_mx_null_handle():
    assert tmm.gemm_run_mx(None, None, 4, 4, 32, 0, 0, 1.0, PA, 32, PSA, 1, PB, 4, PSB, 1, 0.0,
                           PC, 4, E4M3, E4M3, BF16, 0, None) == tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_run_mx_kernel(None, 0, None, 4, 4, 32, 0, 0, 1.0, PA, 32, PSA, 1, PB, 4, PSB,
                                  1, 0.0, PC, 4, E4M3, E4M3, BF16, 0,
                                  None) == tmm.GEMM_ERR_INVALID_HANDLE


# Group-quantized entry points: fake addresses as above.
PX, PW, PS, PO = 0x50000000, 0x60000000, 0x70000000, 0x78000000


def chk_q(M=4, N=48, K=256, X=PX, ldx=None, W=PW, ldw=None, bits=4, group=64, S=PS, O=PO,
          ldg=None, C=PC, ldc=None, xt=BF16, epi=0, bias=None):
    ldx = K if ldx is None else ldx
    ldw = K * bits // 8 if ldw is None else ldw
    ldg = K // group if (ldg is None and group) else (ldg or 0)
    ldc = N if ldc is None else ldc
    return tmm.gemm_check_args_q(M, N, K, X, ldx, W, ldw, bits, group, S, O, ldg, C, ldc, xt,
                                 epi, bias)


def test_q_arguments():
    OK, V, U, AL = (tmm.GEMM_OK, tmm.GEMM_ERR_INVALID_VALUE, tmm.GEMM_ERR_UNSUPPORTED,
                    tmm.GEMM_ERR_ALIAS)
    assert chk_q() == OK and chk_q(bits=8) == OK and chk_q(xt=F16) == OK
    assert chk_q(epi=BIAS | GELU, bias=PBIAS) == OK
    assert chk_q(xt=F32) == U and chk_q(xt=E4M3) == U
    assert chk_q(bits=3) == V and chk_q(bits=2) == V
    assert chk_q(group=0, ldg=4) == V and chk_q(group=48) == V      # K % group != 0
    assert chk_q(K=255, group=1, ldg=255) == V                      # odd K with 4-bit codes
    assert chk_q(K=255, bits=8, group=1, ldg=255) == OK
    assert chk_q(ldx=255) == V and chk_q(ldw=127) == V and chk_q(ldg=3) == V
    assert chk_q(ldc=47) == V and chk_q(C=None) == V
    assert chk_q(X=None) == V and chk_q(W=None) == V and chk_q(S=None) == V and chk_q(O=None) == V
    assert chk_q(epi=BIAS) == V and chk_q(epi=8) == V
    assert chk_q(M=-1) == V
    assert chk_q(M=0, C=None) == OK and chk_q(N=0, C=None) == OK
    assert chk_q(K=0, X=None, W=None, S=None, O=None, ldx=0, ldw=0, ldg=0) == OK
    # C (4 x 48 bf16 = 384 bytes) against each input
    assert chk_q(C=PX + 10) == AL and chk_q(C=PW + 100) == AL
    assert chk_q(C=PS + 2) == AL and chk_q(C=PO + 2) == AL
    assert chk_q(C=PX - 384) == OK and chk_q(C=PX - 383) == AL
    assert chk_q(C=PBIAS, epi=BIAS, bias=PBIAS + 4) == AL


def test_q_null_handle():
    assert tmm.gemm_run_q(None, None, 1, 8, 64, 1.0, PX, 64, PW, 32, 4, 64, PS, PO, 1, 0.0, PC, 8,
                          BF16, 0, None) == tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_run_q_kernel(None, 5, None, 1, 8, 64, 1.0, PX, 64, PW, 32, 4, 64, PS, PO, 1,
                                 0.0, PC, 8, BF16, 0, None) == tmm.GEMM_ERR_INVALID_HANDLE
    assert tmm.gemm_select_kernel_q(None, 1, 8, 64, PX, 64, PW, 32, 4, 64, PS, PO, 1, PC, 8,
                                    BF16, 0, None) == tmm.GEMM_ERR_INVALID_HANDLE
