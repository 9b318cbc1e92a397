// Host side of the C ABI declared in include/gemm.h: argument validation, kernel selection and
// launches.  No allocation happens per call; every launch is asynchronous on the caller's
// stream.
#include "gemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.hpp"

namespace tgemm {
hipError_t launch_simt(const GemmParams& p, int a_type, int transA, int transB, hipStream_t s);
hipError_t launch_mfma_f32(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s);
hipError_t launch_mfma_f16(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s);
hipError_t launch_mfma_bf16(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s);
hipError_t launch_mfma_e4m3(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s);
hipError_t launch_bias_gelu(void* C, int64_t ldc, int M, int N, int c_type, const float* bias,
                            uint32_t epi, int cu_count, hipStream_t s);
}  // namespace tgemm

namespace {

constexpr uint32_t kMagic = 0x47454d4du;  // "GEMM"
constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kMaxRowBytes = int64_t(1) << 23;

struct Args {
  int64_t M, N, K;
  int transA, transB;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  const void* C;
  int64_t ldc;
  gemm_dtype_t at, bt, ct;
  uint32_t epi;
  const float* bias;
};

int esize(gemm_dtype_t t) {
  switch (t) {
    case GEMM_F32: return 4;
    case GEMM_F16: return 2;
    case GEMM_BF16: return 2;
    case GEMM_E4M3: return 1;
    default: return 0;
  }
}

bool supported_tuple(gemm_dtype_t a, gemm_dtype_t b, gemm_dtype_t c) {
  if (a != b) return false;
  switch (a) {
    case GEMM_F32: return c == GEMM_F32;
    case GEMM_F16: return c == GEMM_F16;
    case GEMM_BF16: return c == GEMM_BF16;
    case GEMM_E4M3: return c == GEMM_BF16;
    default: return false;
  }
}

// Byte range [lo, hi) touched by a rows x cols row-major matrix with leading dimension ld.
struct Range {
  __int128 lo, hi;
};
Range byte_range(const void* p, int64_t rows, int64_t cols, int64_t ld, int es) {
  const __int128 lo = (__int128)(uintptr_t)p;
  if (rows <= 0 || cols <= 0) return {lo, lo};
  return {lo, lo + ((__int128)(rows - 1) * ld + cols) * es};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

gemm_status_t check(const Args& a) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_VALUE;
  if ((a.transA != 0 && a.transA != 1) || (a.transB != 0 && a.transB != 1))
    return GEMM_ERR_INVALID_VALUE;
  if (a.epi & ~(GEMM_EPI_BIAS | GEMM_EPI_GELU)) return GEMM_ERR_INVALID_VALUE;
  if (!esize(a.at) || !esize(a.bt) || !esize(a.ct)) return GEMM_ERR_UNSUPPORTED;
  if (!supported_tuple(a.at, a.bt, a.ct)) return GEMM_ERR_UNSUPPORTED;
  if (a.M > kMaxDim || a.N > kMaxDim || a.K > kMaxDim) return GEMM_ERR_UNSUPPORTED;
  if (a.M == 0 || a.N == 0) return GEMM_OK;  // nothing to compute
  if (!a.C) return GEMM_ERR_INVALID_VALUE;
  if (a.ldc < a.N) return GEMM_ERR_INVALID_VALUE;
  if ((a.epi & GEMM_EPI_BIAS) && !a.bias) return GEMM_ERR_INVALID_VALUE;
  const Range rc = byte_range(a.C, a.M, a.N, a.ldc, esize(a.ct));
  if (a.K > 0) {
    if (!a.A || !a.B) return GEMM_ERR_INVALID_VALUE;
    const int64_t a_rows = a.transA ? a.K : a.M, a_cols = a.transA ? a.M : a.K;
    const int64_t b_rows = a.transB ? a.N : a.K, b_cols = a.transB ? a.K : a.N;
    if (a.lda < a_cols || a.ldb < b_cols) return GEMM_ERR_INVALID_VALUE;
    if (overlaps(rc, byte_range(a.A, a_rows, a_cols, a.lda, esize(a.at))) ||
        overlaps(rc, byte_range(a.B, b_rows, b_cols, a.ldb, esize(a.bt))))
      return GEMM_ERR_ALIAS;
  }
  if ((a.epi & GEMM_EPI_BIAS) && overlaps(rc, byte_range(a.bias, 1, a.N, a.N, 4)))
    return GEMM_ERR_ALIAS;
  return GEMM_OK;
}

// Matrix-core kernels read 16-byte chunks of A and B and store 4-element runs of C.
bool mfma_aligned(const Args& a) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (a.K > 0) {
    if (!al16(a.A) || !al16(a.B)) return false;
    if ((a.lda * esize(a.at)) % 16 != 0 || (a.ldb * esize(a.bt)) % 16 != 0) return false;
    // per-lane 32-bit buffer offsets span up to 256 rows of a staged tile
    if (a.lda * esize(a.at) > kMaxRowBytes || a.ldb * esize(a.bt) > kMaxRowBytes) return false;
  }
  return al16(a.C) && (a.ldc % 4 == 0);
}

int64_t tiles(int64_t M, int64_t N, int64_t t) { return ((M + t - 1) / t) * ((N + t - 1) / t); }

// Largest tile that still gives every compute unit at least one workgroup.
gemm_kernel_t auto_kernel(const Args& a, int cu_count) {
  if (!mfma_aligned(a)) return GEMM_KERNEL_SIMT;
  if (tiles(a.M, a.N, 256) >= cu_count) return GEMM_KERNEL_MFMA_256;
  if (tiles(a.M, a.N, 128) >= cu_count) return GEMM_KERNEL_MFMA_128;
  return GEMM_KERNEL_MFMA_64;
}

struct DeviceGuard {
  int prev = -1;
  bool switched = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev && hipSetDevice(dev) == hipSuccess)
      switched = true;
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct gemm_handle {
  uint32_t magic;
  int device;
  int cu_count;
  char arch[64];
};

static bool valid(gemm_handle_t h) { return h && h->magic == kMagic; }

extern "C" {

gemm_status_t gemm_create(gemm_handle_t* out, int device) {
  if (!out) return GEMM_ERR_INVALID_VALUE;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) {
    (void)hipGetLastError();
    return GEMM_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return GEMM_ERR_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_DEVICE;
  gemm_handle* h = static_cast<gemm_handle*>(calloc(1, sizeof(gemm_handle)));
  if (!h) return GEMM_ERR_NO_MEMORY;
  h->magic = kMagic;
  h->device = device;
  h->cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  strncpy(h->arch, prop.gcnArchName, sizeof(h->arch) - 1);
  *out = h;
  return GEMM_OK;
}

gemm_status_t gemm_destroy(gemm_handle_t h) {
  if (!h) return GEMM_OK;
  if (h->magic != kMagic) return GEMM_ERR_INVALID_HANDLE;
  h->magic = 0;
  free(h);
  return GEMM_OK;
}

gemm_status_t gemm_check_args(int64_t M, int64_t N, int64_t K, int transA, int transB,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              const void* C, int64_t ldc, gemm_dtype_t a_type,
                              gemm_dtype_t b_type, gemm_dtype_t c_type, uint32_t epilogue,
                              const float* bias) {
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  return check(a);
}

int gemm_select_kernel(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int transA,
                       int transB, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, gemm_dtype_t a_type, gemm_dtype_t b_type,
                       gemm_dtype_t c_type, uint32_t epilogue, const float* bias) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  const gemm_status_t st = check(a);
  if (st != GEMM_OK) return st;
  return auto_kernel(a, h->cu_count);
}

gemm_status_t gemm_run_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                              int64_t N, int64_t K, int transA, int transB, float alpha,
                              const void* A, int64_t lda, float scale_a, const void* B,
                              int64_t ldb, float scale_b, float beta, void* C, int64_t ldc,
                              gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                              uint32_t epilogue, const float* bias) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  gemm_status_t st = check(a);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  if (kernel == GEMM_KERNEL_AUTO) kernel = auto_kernel(a, h->cu_count);

  tgemm::GemmParams p;
  p.A = A;
  p.B = B;
  p.C = C;
  p.bias = bias;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.alpha = alpha * scale_a * scale_b;
  p.beta = beta;
  p.epi = epilogue;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (kernel == GEMM_KERNEL_SIMT) {
    if ((M + 15) / 16 > 65535) return GEMM_ERR_UNSUPPORTED;
    p.tiles_m = (int)((M + 15) / 16);
    p.tiles_n = (int)((N + 15) / 16);
    DeviceGuard g(h->device);
    err = tgemm::launch_simt(p, a_type, transA, transB, s);
  } else if (kernel >= GEMM_KERNEL_MFMA_64 && kernel <= GEMM_KERNEL_MFMA_256) {
    if (!mfma_aligned(a)) return GEMM_ERR_UNSUPPORTED;
    const int tile = kernel - GEMM_KERNEL_MFMA_64;
    const int t = 64 << tile;
    const int64_t tm = (M + t - 1) / t, tn = (N + t - 1) / t;
    if (tm * tn > kMaxDim) return GEMM_ERR_UNSUPPORTED;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    // Storage contiguous along M (A stored K x M) or along N (B stored K x N).
    const bool a_mn = transA != 0, b_mn = transB == 0;
    DeviceGuard g(h->device);
    switch (a_type) {
      case GEMM_F32: err = tgemm::launch_mfma_f32(p, tile, a_mn, b_mn, s); break;
      case GEMM_F16: err = tgemm::launch_mfma_f16(p, tile, a_mn, b_mn, s); break;
      case GEMM_BF16: err = tgemm::launch_mfma_bf16(p, tile, a_mn, b_mn, s); break;
      case GEMM_E4M3: err = tgemm::launch_mfma_e4m3(p, tile, a_mn, b_mn, s); break;
      default: return GEMM_ERR_UNSUPPORTED;
    }
  } else {
    return GEMM_ERR_INVALID_VALUE;
  }
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

gemm_status_t gemm_run(gemm_handle_t h, void* stream, int64_t M, int64_t N, int64_t K,
                       int transA, int transB, float alpha, const void* A, int64_t lda,
                       float scale_a, const void* B, int64_t ldb, float scale_b, float beta,
                       void* C, int64_t ldc, gemm_dtype_t a_type, gemm_dtype_t b_type,
                       gemm_dtype_t c_type, uint32_t epilogue, const float* bias) {
  return gemm_run_kernel(h, GEMM_KERNEL_AUTO, stream, M, N, K, transA, transB, alpha, A, lda,
                         scale_a, B, ldb, scale_b, beta, C, ldc, a_type, b_type, c_type,
                         epilogue, bias);
}

gemm_status_t gemm_bias_gelu(gemm_handle_t h, void* stream, int64_t M, int64_t N, void* C,
                             int64_t ldc, gemm_dtype_t c_type, const float* bias,
                             uint32_t epilogue) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  if (M < 0 || N < 0) return GEMM_ERR_INVALID_VALUE;
  if (epilogue & ~(GEMM_EPI_BIAS | GEMM_EPI_GELU)) return GEMM_ERR_INVALID_VALUE;
  if (c_type != GEMM_F32 && c_type != GEMM_F16 && c_type != GEMM_BF16) return GEMM_ERR_UNSUPPORTED;
  if (M > kMaxDim || N > kMaxDim) return GEMM_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return GEMM_OK;
  if (!C || ldc < N) return GEMM_ERR_INVALID_VALUE;
  if ((epilogue & GEMM_EPI_BIAS) && !bias) return GEMM_ERR_INVALID_VALUE;
  if ((epilogue & GEMM_EPI_BIAS) &&
      overlaps(byte_range(C, M, N, ldc, esize(c_type)), byte_range(bias, 1, N, N, 4)))
    return GEMM_ERR_ALIAS;
  DeviceGuard g(h->device);
  const hipError_t err = tgemm::launch_bias_gelu(C, ldc, (int)M, (int)N, c_type, bias, epilogue,
                                                 h->cu_count, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

const char* gemm_status_string(gemm_status_t s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_HANDLE: return "GEMM_ERR_INVALID_HANDLE: null or destroyed handle";
    case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE: invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: type tuple, size or kernel not supported";
    case GEMM_ERR_ALIAS: return "GEMM_ERR_ALIAS: C overlaps an input";
    case GEMM_ERR_DEVICE: return "GEMM_ERR_DEVICE: no gfx950 device";
    case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: kernel launch failed";
    case GEMM_ERR_NO_MEMORY: return "GEMM_ERR_NO_MEMORY: host allocation failed";
    default: return "GEMM_ERR_UNKNOWN";
  }
}

}  // extern "C"
