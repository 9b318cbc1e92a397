"""Python binding of the tiled GEMM library for MI355X (gfx950).

This module only marshals arguments into libgemm.so (the C ABI of include/gemm.h): every step
of the computation runs in the library's HIP kernels.  The names mirror the C entry points
(gemm_create, gemm_run, ...).  PyTorch is used only for device memory and the current HIP
stream, and only inside the tensor helpers (`run`, `bias_gelu`).

Importing this package loads libgemm.so and raises ImportError if it has not been built:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm.so")

# gemm_status_t
GEMM_OK = 0
GEMM_ERR_INVALID_HANDLE = -1
GEMM_ERR_INVALID_VALUE = -2
GEMM_ERR_UNSUPPORTED = -3
GEMM_ERR_ALIAS = -4
GEMM_ERR_DEVICE = -5
GEMM_ERR_LAUNCH = -6
GEMM_ERR_NO_MEMORY = -7
GEMM_ERR_TOO_LARGE = -8

# gemm_dtype_t
GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_E4M3, GEMM_E5M2, GEMM_E2M1 = 0, 1, 2, 3, 4, 5
GEMM_E2M3, GEMM_E3M2 = 6, 7
DTYPE = {"f32": GEMM_F32, "f16": GEMM_F16, "bf16": GEMM_BF16, "e4m3": GEMM_E4M3,
         "e5m2": GEMM_E5M2, "e2m1": GEMM_E2M1, "e2m3": GEMM_E2M3, "e3m2": GEMM_E3M2}
LOWP = ("e4m3", "e5m2", "e2m1", "e2m3", "e3m2")  # output bf16

# epilogue bits
GEMM_EPI_NONE, GEMM_EPI_BIAS, GEMM_EPI_GELU = 0, 1, 2

# gemm_kernel_t
GEMM_KERNEL_AUTO = 0
GEMM_KERNEL_SIMT = 1
GEMM_KERNEL_MFMA_64 = 2
GEMM_KERNEL_MFMA_128 = 3
GEMM_KERNEL_MFMA_256 = 4
GEMM_KERNEL_QGEMV = 5
GEMM_KERNEL_QMFMA = 6
GEMM_KERNEL_MFMA_32 = 7
GEMM_KERNEL_MFMA_256x128 = 8
GEMM_KERNEL_MFMA_256x128_SK2 = 9
GEMM_KERNEL_MFMA_256_SK = 10
KERNEL_NAME = {0: "auto", 1: "simt", 2: "mfma64", 3: "mfma128", 4: "mfma256", 5: "qgemv",
               6: "qmfma", 7: "mfma32", 8: "mfma256x128", 9: "mfma256x128_sk2", 10: "mfma256_sk"}

# Every symbol include/gemm.h declares.
EXPORTS = ("gemm_create", "gemm_destroy", "gemm_check_args", "gemm_run", "gemm_run_kernel",
           "gemm_run_mx", "gemm_run_mx_kernel", "gemm_check_args_mx", "gemm_select_kernel",
           "gemm_bias_gelu", "gemm_status_string", "gemm_run_q", "gemm_run_q_kernel",
           "gemm_check_args_q", "gemm_select_kernel_q", "gemm_probe_clock",
           "gemm_wall_clock_khz", "gemm_probe_bandwidth", "gemm_run_ws", "gemm_run_ws_kernel",
           "gemm_workspace_bytes", "gemm_run_noalloc", "gemm_kernel_workspace_bytes")

# libgemm.so must resolve its libamdhip64.so.7 dependency to the HIP runtime instance that owns
# the caller's device pointers and streams.  PyTorch ships its own runtime (soname
# libamdhip64.so.7, but its libraries ask for plain "libamdhip64.so"): if libgemm.so were loaded
# first, the system runtime would come in and torch would then load a second one beside it.
# Loading torch first makes libgemm.so bind to torch's runtime.
try:
    import torch as _torch  # noqa: F401
except ImportError:
    _torch = None

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as "
                      f"g; g.build()' or python tiled_matrix_multiply_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_u32 = ctypes.c_uint32
_vp = ctypes.c_void_p

_lib.gemm_create.argtypes = [ctypes.POINTER(_vp), _int]
_lib.gemm_create.restype = _int
_lib.gemm_destroy.argtypes = [_vp]
_lib.gemm_destroy.restype = _int
_lib.gemm_check_args.argtypes = [_i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64, _vp, _i64,
                                 _int, _int, _int, _u32, _vp]
_lib.gemm_check_args.restype = _int
_RUN = [_i64, _i64, _i64, _int, _int, _f32, _vp, _i64, _f32, _vp, _i64, _f32, _f32, _vp, _i64,
        _int, _int, _int, _u32, _vp]
_lib.gemm_run.argtypes = [_vp, _vp] + _RUN
_lib.gemm_run.restype = _int
_lib.gemm_run_kernel.argtypes = [_vp, _int, _vp] + _RUN
_lib.gemm_run_kernel.restype = _int
_RUN_MX = [_i64, _i64, _i64, _int, _int, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _f32,
           _vp, _i64, _int, _int, _int, _u32, _vp]
_lib.gemm_run_mx.argtypes = [_vp, _vp] + _RUN_MX
_lib.gemm_run_mx.restype = _int
_lib.gemm_run_mx_kernel.argtypes = [_vp, _int, _vp] + _RUN_MX
_lib.gemm_run_mx_kernel.restype = _int
_lib.gemm_check_args_mx.argtypes = [_i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64, _vp, _i64,
                                    _vp, _i64, _vp, _i64, _int, _int, _int, _u32, _vp]
_lib.gemm_check_args_mx.restype = _int
_lib.gemm_select_kernel.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64, _vp,
                                    _i64, _int, _int, _int, _u32, _vp]
_lib.gemm_select_kernel.restype = _int
_lib.gemm_bias_gelu.argtypes = [_vp, _vp, _i64, _i64, _vp, _i64, _int, _vp, _u32]
_lib.gemm_bias_gelu.restype = _int
_Q = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _int, _i64, _vp, _vp, _i64, _f32, _vp,
      _i64, _int, _u32, _vp]
_lib.gemm_run_q.argtypes = [_vp, _vp] + _Q
_lib.gemm_run_q.restype = _int
_lib.gemm_run_q_kernel.argtypes = [_vp, _int, _vp] + _Q
_lib.gemm_run_q_kernel.restype = _int
_QCHK = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _i64, _vp, _vp, _i64, _vp, _i64, _int,
         _u32, _vp]
_lib.gemm_check_args_q.argtypes = _QCHK
_lib.gemm_check_args_q.restype = _int
_lib.gemm_select_kernel_q.argtypes = [_vp] + _QCHK
_lib.gemm_select_kernel_q.restype = _int
_lib.gemm_run_ws.argtypes = [_vp, _vp] + _RUN + [_vp, _i64]
_lib.gemm_run_ws.restype = _int
_lib.gemm_run_ws_kernel.argtypes = [_vp, _int, _vp] + _RUN + [_vp, _i64]
_lib.gemm_run_ws_kernel.restype = _int
_lib.gemm_run_noalloc.argtypes = [_vp, _int, _vp] + _RUN
_lib.gemm_run_noalloc.restype = _int
_lib.gemm_workspace_bytes.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64,
                                      _vp, _i64, _int, _int, _int, _u32, _vp]
_lib.gemm_workspace_bytes.restype = _i64
_lib.gemm_kernel_workspace_bytes.argtypes = [_vp, _int, _i64, _i64]
_lib.gemm_kernel_workspace_bytes.restype = _i64
_lib.gemm_probe_clock.argtypes = [_vp, _vp, _vp, _int, _int]
_lib.gemm_probe_clock.restype = _int
_lib.gemm_wall_clock_khz.argtypes = [_vp]
_lib.gemm_wall_clock_khz.restype = _int
_lib.gemm_probe_bandwidth.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp]
_lib.gemm_probe_bandwidth.restype = _int
_lib.gemm_status_string.argtypes = [_int]
_lib.gemm_status_string.restype = ctypes.c_char_p


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        super().__init__(f"{where}: {gemm_status_string(status)} ({status})")


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib


# ----------------------------------------------------------------- C ABI, same names --

def gemm_status_string(status: int) -> str:
    return _lib.gemm_status_string(int(status)).decode()


def gemm_create(device: int = 0) -> int:
    """Create a handle for HIP device `device`; returns the opaque handle value."""
    h = _vp()
    st = _lib.gemm_create(ctypes.byref(h), int(device))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_create")
    return h.value


def gemm_destroy(handle) -> None:
    st = _lib.gemm_destroy(handle)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_destroy")


def gemm_check_args(M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
                    epilogue, bias) -> int:
    """Pointers are integers (device addresses) or None.  Returns the status code."""
    return _lib.gemm_check_args(M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type,
                                c_type, epilogue, bias)


def gemm_run(handle, stream, M, N, K, transA, transB, alpha, A, lda, scale_a, B, ldb, scale_b,
             beta, C, ldc, a_type, b_type, c_type, epilogue, bias) -> int:
    """Raw entry point: returns the status code (no exception)."""
    return _lib.gemm_run(handle, stream, M, N, K, transA, transB, alpha, A, lda, scale_a, B, ldb,
                         scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue, bias)


def gemm_run_kernel(handle, kernel, stream, M, N, K, transA, transB, alpha, A, lda, scale_a, B,
                    ldb, scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue, bias) -> int:
    return _lib.gemm_run_kernel(handle, kernel, stream, M, N, K, transA, transB, alpha, A, lda,
                                scale_a, B, ldb, scale_b, beta, C, ldc, a_type, b_type, c_type,
                                epilogue, bias)


def gemm_check_args_mx(M, N, K, transA, transB, A, lda, sa, ldsa, B, ldb, sb, ldsb, C, ldc,
                       a_type, b_type, c_type, epilogue, bias) -> int:
    """Pointers are integers (device addresses) or None.  Returns the status code."""
    return _lib.gemm_check_args_mx(M, N, K, transA, transB, A, lda, sa, ldsa, B, ldb, sb, ldsb,
                                   C, ldc, a_type, b_type, c_type, epilogue, bias)


def gemm_run_mx(handle, stream, M, N, K, transA, transB, alpha, A, lda, sa, ldsa, B, ldb, sb,
                ldsb, beta, C, ldc, a_type, b_type, c_type, epilogue, bias) -> int:
    """Raw block-scaled (OCP MX) entry point: returns the status code (no exception)."""
    return _lib.gemm_run_mx(handle, stream, M, N, K, transA, transB, alpha, A, lda, sa, ldsa, B,
                            ldb, sb, ldsb, beta, C, ldc, a_type, b_type, c_type, epilogue, bias)


def gemm_run_mx_kernel(handle, kernel, stream, M, N, K, transA, transB, alpha, A, lda, sa, ldsa,
                       B, ldb, sb, ldsb, beta, C, ldc, a_type, b_type, c_type, epilogue,
                       bias) -> int:
    return _lib.gemm_run_mx_kernel(handle, kernel, stream, M, N, K, transA, transB, alpha, A,
                                   lda, sa, ldsa, B, ldb, sb, ldsb, beta, C, ldc, a_type, b_type,
                                   c_type, epilogue, bias)


def gemm_select_kernel(handle, M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type,
                       c_type, epilogue, bias) -> int:
    return _lib.gemm_select_kernel(handle, M, N, K, transA, transB, A, lda, B, ldb, C, ldc,
                                   a_type, b_type, c_type, epilogue, bias)


def gemm_bias_gelu(handle, stream, M, N, C, ldc, c_type, bias, epilogue) -> int:
    return _lib.gemm_bias_gelu(handle, stream, M, N, C, ldc, c_type, bias, epilogue)


def gemm_run_q(handle, stream, M, N, K, alpha, X, ldx, Wq, ldw, bits, group, scales, offsets,
               ldg, beta, C, ldc, x_type, epilogue, bias) -> int:
    """Raw group-quantized entry point: returns the status code (no exception)."""
    return _lib.gemm_run_q(handle, stream, M, N, K, alpha, X, ldx, Wq, ldw, bits, group, scales,
                           offsets, ldg, beta, C, ldc, x_type, epilogue, bias)


def gemm_run_q_kernel(handle, kernel, stream, M, N, K, alpha, X, ldx, Wq, ldw, bits, group,
                      scales, offsets, ldg, beta, C, ldc, x_type, epilogue, bias) -> int:
    return _lib.gemm_run_q_kernel(handle, kernel, stream, M, N, K, alpha, X, ldx, Wq, ldw, bits,
                                  group, scales, offsets, ldg, beta, C, ldc, x_type, epilogue,
                                  bias)


def gemm_check_args_q(M, N, K, X, ldx, Wq, ldw, bits, group, scales, offsets, ldg, C, ldc,
                      x_type, epilogue, bias) -> int:
    return _lib.gemm_check_args_q(M, N, K, X, ldx, Wq, ldw, bits, group, scales, offsets, ldg,
                                  C, ldc, x_type, epilogue, bias)


def gemm_select_kernel_q(handle, M, N, K, X, ldx, Wq, ldw, bits, group, scales, offsets, ldg,
                         C, ldc, x_type, epilogue, bias) -> int:
    return _lib.gemm_select_kernel_q(handle, M, N, K, X, ldx, Wq, ldw, bits, group, scales,
                                     offsets, ldg, C, ldc, x_type, epilogue, bias)


def gemm_run_ws(handle, stream, M, N, K, transA, transB, alpha, A, lda, scale_a, B, ldb,
                scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue, bias, workspace,
                workspace_bytes) -> int:
    """Raw entry point with a device workspace: returns the status code (no exception)."""
    return _lib.gemm_run_ws(handle, stream, M, N, K, transA, transB, alpha, A, lda, scale_a, B,
                            ldb, scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue, bias,
                            workspace, workspace_bytes)


def gemm_run_ws_kernel(handle, kernel, stream, M, N, K, transA, transB, alpha, A, lda, scale_a,
                       B, ldb, scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue, bias,
                       workspace, workspace_bytes) -> int:
    return _lib.gemm_run_ws_kernel(handle, kernel, stream, M, N, K, transA, transB, alpha, A,
                                   lda, scale_a, B, ldb, scale_b, beta, C, ldc, a_type, b_type,
                                   c_type, epilogue, bias, workspace, workspace_bytes)


def gemm_run_noalloc(handle, kernel, stream, M, N, K, transA, transB, alpha, A, lda, scale_a,
                     B, ldb, scale_b, beta, C, ldc, a_type, b_type, c_type, epilogue,
                     bias) -> int:
    """Raw entry point with the library's static scratch as workspace (no allocation)."""
    return _lib.gemm_run_noalloc(handle, kernel, stream, M, N, K, transA, transB, alpha, A, lda,
                                 scale_a, B, ldb, scale_b, beta, C, ldc, a_type, b_type, c_type,
                                 epilogue, bias)


def gemm_workspace_bytes(handle, M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type,
                         b_type, c_type, epilogue, bias) -> int:
    return _lib.gemm_workspace_bytes(handle, M, N, K, transA, transB, A, lda, B, ldb, C, ldc,
                                     a_type, b_type, c_type, epilogue, bias)


SPLIT_K_SLOT_BYTES = 131328  # one 256 x 128 output tile: counter and flag, then fp32 partial sums


def gemm_kernel_workspace_bytes(handle, kernel, M, N) -> int:
    return _lib.gemm_kernel_workspace_bytes(handle, kernel, M, N)


def split_k_workspace_bytes(M: int, N: int) -> int:
    """Workspace the K-split kernel (GEMM_KERNEL_MFMA_256x128_SK2) needs for an M x N output,
    as include/gemm.h states it: one 131328-byte slot per 256 x 128 tile."""
    return -(-M // 256) * -(-N // 128) * SPLIT_K_SLOT_BYTES


def gemm_probe_clock(handle, stream, out, workgroups, microseconds) -> int:
    return _lib.gemm_probe_clock(handle, stream, out, workgroups, microseconds)


def gemm_wall_clock_khz(handle) -> int:
    return _lib.gemm_wall_clock_khz(handle)


def gemm_probe_bandwidth(handle, stream, src, dst, nbytes, sink) -> int:
    return _lib.gemm_probe_bandwidth(handle, stream, src, dst, nbytes, sink)


# ----------------------------------------------------------------- tensor helpers --

def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    """Device address of a tensor; an int is taken as an address already."""
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


def run(handle, A, B, C, *, M, N, K, trans_a=False, trans_b=False, alpha=1.0, beta=0.0,
        a_type="f32", b_type=None, c_type=None, epilogue=GEMM_EPI_NONE, bias=None, scale_a=1.0,
        scale_b=1.0, lda=None, ldb=None, ldc=None, sa_blk=None, sb_blk=None, ldsa=None,
        ldsb=None, kernel=GEMM_KERNEL_AUTO, stream=None, workspace=None, workspace_bytes=0):
    """GEMM on device tensors holding storage words (A, B, C contiguous row-major unless ld*
    is given; E2M1 holds two elements per byte, E2M3 / E3M2 four per three bytes).  With
    sa_blk / sb_blk (device uint8 tensors of E8M0 scales, M x ldsa and N x ldsb) the call is
    block-scaled (gemm_run_mx).  Raises
    GemmError on a negative status.  Asynchronous on `stream` (default: torch's current
    stream)."""
    b_type = b_type or a_type
    c_type = c_type or ("bf16" if a_type in LOWP else a_type)
    lda = lda if lda is not None else (M if trans_a else K)
    ldb = ldb if ldb is not None else (K if trans_b else N)
    ldc = ldc if ldc is not None else N
    if sa_blk is not None or sb_blk is not None:
        ldsa = ldsa if ldsa is not None else K // 32
        ldsb = ldsb if ldsb is not None else K // 32
        st = gemm_run_mx_kernel(handle, kernel, _stream(stream), M, N, K, int(trans_a),
                                int(trans_b), float(alpha), _ptr(A), lda, _ptr(sa_blk), ldsa,
                                _ptr(B), ldb, _ptr(sb_blk), ldsb, float(beta), _ptr(C), ldc,
                                DTYPE[a_type], DTYPE[b_type], DTYPE[c_type], int(epilogue),
                                _ptr(bias))
        where = "gemm_run_mx"
    elif workspace is not None:
        st = gemm_run_ws_kernel(handle, kernel, _stream(stream), M, N, K, int(trans_a),
                                int(trans_b), float(alpha), _ptr(A), lda, float(scale_a),
                                _ptr(B), ldb, float(scale_b), float(beta), _ptr(C), ldc,
                                DTYPE[a_type], DTYPE[b_type], DTYPE[c_type], int(epilogue),
                                _ptr(bias), _ptr(workspace), int(workspace_bytes))
        where = "gemm_run_ws"
    else:
        st = gemm_run_kernel(handle, kernel, _stream(stream), M, N, K, int(trans_a),
                             int(trans_b), float(alpha), _ptr(A), lda, float(scale_a), _ptr(B),
                             ldb, float(scale_b), float(beta), _ptr(C), ldc, DTYPE[a_type],
                             DTYPE[b_type], DTYPE[c_type], int(epilogue), _ptr(bias))
        where = "gemm_run"
    if st != GEMM_OK:
        raise GemmError(st, where)


def bias_gelu(handle, C, bias, *, M, N, c_type, epilogue=GEMM_EPI_BIAS | GEMM_EPI_GELU,
              ldc=None, stream=None):
    """The unfused epilogue pass C = epi(C + bias) in place."""
    st = gemm_bias_gelu(handle, _stream(stream), M, N, _ptr(C), ldc if ldc is not None else N,
                        DTYPE[c_type], _ptr(bias), int(epilogue))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_bias_gelu")


def select_kernel(handle, M, N, K, *, trans_a=False, trans_b=False, a_type="f32", b_type=None,
                  A=None, B=None, C=None, epilogue=GEMM_EPI_NONE, bias=None, lda=None,
                  ldb=None, ldc=None) -> str:
    """Name of the kernel family gemm_run picks for these arguments."""
    b_type = b_type or a_type
    c_type = "bf16" if a_type in LOWP else a_type
    k = gemm_select_kernel(handle, M, N, K, int(trans_a), int(trans_b), _ptr(A),
                           lda if lda is not None else (M if trans_a else K), _ptr(B),
                           ldb if ldb is not None else (K if trans_b else N), _ptr(C),
                           ldc if ldc is not None else N, DTYPE[a_type], DTYPE[b_type],
                           DTYPE[c_type], int(epilogue), _ptr(bias))
    if k < 0:
        raise GemmError(k, "gemm_select_kernel")
    return KERNEL_NAME[k]


def run_q(handle, X, Wq, scales, offsets, C, *, M, N, K, bits, group, x_type="bf16",
          alpha=1.0, beta=0.0, epilogue=GEMM_EPI_NONE, bias=None, ldx=None, ldw=None,
          ldg=None, ldc=None, kernel=GEMM_KERNEL_AUTO, stream=None):
    """Group-quantized C = epi(alpha X W^T + beta C + bias) on device tensors of storage words
    (X, scales, offsets, C: 16-bit words; Wq: bytes).  Raises GemmError on a negative status."""
    st = gemm_run_q_kernel(handle, kernel, _stream(stream), M, N, K, float(alpha), _ptr(X),
                           ldx if ldx is not None else K, _ptr(Wq),
                           ldw if ldw is not None else K * bits // 8, int(bits), int(group),
                           _ptr(scales), _ptr(offsets), ldg if ldg is not None else K // group,
                           float(beta), _ptr(C), ldc if ldc is not None else N, DTYPE[x_type],
                           int(epilogue), _ptr(bias))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_run_q")


def select_kernel_q(handle, M, N, K, *, bits, group, x_type="bf16", X=None, Wq=None,
                    scales=None, offsets=None, C=None, epilogue=GEMM_EPI_NONE, bias=None,
                    ldx=None, ldw=None, ldg=None, ldc=None) -> str:
    """Name of the kernel gemm_run_q picks for these arguments."""
    k = gemm_select_kernel_q(handle, M, N, K, _ptr(X), ldx if ldx is not None else K, _ptr(Wq),
                             ldw if ldw is not None else K * bits // 8, int(bits), int(group),
                             _ptr(scales), _ptr(offsets), ldg if ldg is not None else K // group,
                             _ptr(C), ldc if ldc is not None else N, DTYPE[x_type],
                             int(epilogue), _ptr(bias))
    if k < 0:
        raise GemmError(k, "gemm_select_kernel_q")
    return KERNEL_NAME[k]


class Gemm:
    """Owns one handle (gemm_create / gemm_destroy)."""

    def __init__(self, device: int = 0):
        self.handle = gemm_create(device)

    def close(self):
        if self.handle:
            gemm_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, A, B, C, **kw):
        run(self.handle, A, B, C, **kw)

    def bias_gelu(self, C, bias, **kw):
        bias_gelu(self.handle, C, bias, **kw)

    def select_kernel(self, M, N, K, **kw) -> str:
        return select_kernel(self.handle, M, N, K, **kw)

    def run_q(self, X, Wq, scales, offsets, C, **kw):
        run_q(self.handle, X, Wq, scales, offsets, C, **kw)

    def select_kernel_q(self, M, N, K, **kw) -> str:
        return select_kernel_q(self.handle, M, N, K, **kw)
