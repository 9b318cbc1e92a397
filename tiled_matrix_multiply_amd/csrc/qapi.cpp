// Host side of the quantized-weight entry points declared in include/gemm.h (gemm_run_q and
// friends): argument validation, kernel choice and launches.  Nothing is allocated per call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"
#include "handle.hpp"
#include "quant.hpp"

namespace tgemm {
hipError_t launch_qsimt(const QParams& p, int x_type, int cu_count, hipStream_t s);
hipError_t launch_qgemv(const QParams& p, int x_type, int cu_count, hipStream_t s);
hipError_t launch_qmfma(const QParams& p, int x_type, int cu_count, hipStream_t s);
}  // namespace tgemm

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kQgemvMaxRows = 4;
constexpr int64_t kQgemvMaxLds = 80 * 1024;  // two workgroups still fit a compute unit's 160 KiB

struct QArgs {
  int64_t M, N, K;
  const void* X;
  int64_t ldx;
  const uint8_t* W;
  int64_t ldw;
  int bits;
  int64_t group;
  const void* S;
  const void* O;
  int64_t ldg;
  const void* C;
  int64_t ldc;
  gemm_dtype_t xt;
  uint32_t epi;
  const float* bias;
};

struct Range {
  __int128 lo, hi;
};
// Byte range of `rows` rows of `row_bytes` bytes, `stride` bytes apart.
Range rows_range(const void* p, int64_t rows, int64_t row_bytes, int64_t stride) {
  const __int128 lo = (__int128)(uintptr_t)p;
  if (rows <= 0 || row_bytes <= 0) return {lo, lo};
  return {lo, lo + (__int128)(rows - 1) * stride + row_bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

gemm_status_t check_q(const QArgs& a) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_VALUE;
  if (a.epi & ~(GEMM_EPI_BIAS | GEMM_EPI_GELU)) return GEMM_ERR_INVALID_VALUE;
  if (a.xt != GEMM_F16 && a.xt != GEMM_BF16) return GEMM_ERR_UNSUPPORTED;
  if (a.bits != 4 && a.bits != 8) return GEMM_ERR_INVALID_VALUE;
  if (a.group < 1 || a.K % a.group != 0) return GEMM_ERR_INVALID_VALUE;
  if (a.bits == 4 && a.K % 2 != 0) return GEMM_ERR_INVALID_VALUE;
  if (a.M > kMaxDim || a.N > kMaxDim || a.K > kMaxDim) return GEMM_ERR_UNSUPPORTED;
  if (a.M == 0 || a.N == 0) return GEMM_OK;
  if (!a.C || a.ldc < a.N) return GEMM_ERR_INVALID_VALUE;
  if ((a.epi & GEMM_EPI_BIAS) && !a.bias) return GEMM_ERR_INVALID_VALUE;
  const Range rc = rows_range(a.C, a.M, a.N * 2, a.ldc * 2);
  if (a.K > 0) {
    if (!a.X || !a.W || !a.S || !a.O) return GEMM_ERR_INVALID_VALUE;
    const int64_t kb = a.K * a.bits / 8, ng = a.K / a.group;
    if (a.ldx < a.K || a.ldw < kb || a.ldg < ng) return GEMM_ERR_INVALID_VALUE;
    if (overlaps(rc, rows_range(a.X, a.M, a.K * 2, a.ldx * 2)) ||
        overlaps(rc, rows_range(a.W, a.N, kb, a.ldw)) ||
        overlaps(rc, rows_range(a.S, a.N, ng * 2, a.ldg * 2)) ||
        overlaps(rc, rows_range(a.O, a.N, ng * 2, a.ldg * 2)))
      return GEMM_ERR_ALIAS;
  }
  if ((a.epi & GEMM_EPI_BIAS) && overlaps(rc, rows_range(a.bias, 1, a.N * 4, a.N * 4)))
    return GEMM_ERR_ALIAS;
  return GEMM_OK;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Needs of the matrix-vector kernel: 16-byte code chunks that never straddle a group, the
// staged activations within 80 KiB of LDS, and 32-bit chunk counts.
bool qgemv_ok(const QArgs& a) {
  const int ch = a.bits == 4 ? 32 : 16;
  if (a.M > kQgemvMaxRows) return false;
  if (a.K == 0) return true;
  if (a.group % ch != 0 || !al16(a.W) || a.ldw % 16 != 0) return false;
  const int64_t lds = a.M * a.K * (a.bits == 4 ? 2 : 4) + a.M * (a.K / ch) * 4;
  return lds <= kQgemvMaxLds;
}

// Needs of the matrix-core kernel (see launch_qmfma): 16-byte chunks of X, codes and C; whole
// 64-element K tiles, each thread's 32 codes inside one group; 32-bit byte offsets.
bool qmfma_ok(const QArgs& a) {
  if (a.K == 0 || a.K % 64 != 0 || a.group % 32 != 0) return false;
  if (!al16(a.X) || !al16(a.W) || !al16(a.C)) return false;
  if (a.ldx % 8 != 0 || a.ldw % 16 != 0 || a.ldc % 4 != 0) return false;
  return a.ldx * 2 <= (int64_t(1) << 23) && a.ldw <= (int64_t(1) << 23);
}

gemm_kernel_t auto_q(const QArgs& a) {
  if (a.M <= kQgemvMaxRows && qgemv_ok(a)) return GEMM_KERNEL_QGEMV;
  if (qmfma_ok(a)) return GEMM_KERNEL_QMFMA;
  return GEMM_KERNEL_SIMT;
}

bool valid(gemm_handle_t h) { return h && h->magic == tgemm::kHandleMagic; }

gemm_status_t run_q(gemm_handle_t h, gemm_kernel_t kernel, void* stream, const QArgs& a,
                    float alpha, float beta, void* C) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  const gemm_status_t st = check_q(a);
  if (st != GEMM_OK) return st;
  if (a.M == 0 || a.N == 0) return GEMM_OK;
  if (kernel == GEMM_KERNEL_AUTO) kernel = auto_q(a);
  tgemm::QParams p{};
  p.X = a.X;
  p.W = a.W;
  p.S = a.S;
  p.O = a.O;
  p.C = C;
  p.bias = a.bias;
  p.ldx = a.ldx;
  p.ldw = a.ldw;
  p.ldg = a.ldg;
  p.ldc = a.ldc;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.bits = a.bits;
  p.group = (int)a.group;
  p.alpha = alpha;
  p.beta = beta;
  p.epi = a.epi;
  const int xt = a.xt == GEMM_BF16 ? tgemm::BF16 : tgemm::F16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  tgemm::DeviceGuard g(h->device);
  switch (kernel) {
    case GEMM_KERNEL_SIMT: err = tgemm::launch_qsimt(p, xt, h->cu_count, s); break;
    case GEMM_KERNEL_QGEMV:
      if (!qgemv_ok(a)) return GEMM_ERR_UNSUPPORTED;
      if (a.K == 0) err = tgemm::launch_qsimt(p, xt, h->cu_count, s);
      else err = tgemm::launch_qgemv(p, xt, h->cu_count, s);
      break;
    case GEMM_KERNEL_QMFMA:
      if (!qmfma_ok(a)) return GEMM_ERR_UNSUPPORTED;
      err = tgemm::launch_qmfma(p, xt, h->cu_count, s);
      break;
    default: return GEMM_ERR_UNSUPPORTED;
  }
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

gemm_status_t gemm_check_args_q(int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                                const uint8_t* Wq, int64_t ldw, int bits, int64_t group,
                                const void* scales, const void* offsets, int64_t ldg,
                                const void* C, int64_t ldc, gemm_dtype_t x_type,
                                uint32_t epilogue, const float* bias) {
  const QArgs a{M, N, K, X, ldx, Wq, ldw, bits, group, scales, offsets, ldg, C, ldc, x_type,
                epilogue, bias};
  return check_q(a);
}

int gemm_select_kernel_q(gemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* X,
                         int64_t ldx, const uint8_t* Wq, int64_t ldw, int bits, int64_t group,
                         const void* scales, const void* offsets, int64_t ldg, const void* C,
                         int64_t ldc, gemm_dtype_t x_type, uint32_t epilogue,
                         const float* bias) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  const QArgs a{M, N, K, X, ldx, Wq, ldw, bits, group, scales, offsets, ldg, C, ldc, x_type,
                epilogue, bias};
  const gemm_status_t st = check_q(a);
  if (st != GEMM_OK) return st;
  return auto_q(a);
}

gemm_status_t gemm_run_q_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                                int64_t N, int64_t K, float alpha, const void* X, int64_t ldx,
                                const uint8_t* Wq, int64_t ldw, int bits, int64_t group,
                                const void* scales, const void* offsets, int64_t ldg,
                                float beta, void* C, int64_t ldc, gemm_dtype_t x_type,
                                uint32_t epilogue, const float* bias) {
  const QArgs a{M, N, K, X, ldx, Wq, ldw, bits, group, scales, offsets, ldg, C, ldc, x_type,
                epilogue, bias};
  return run_q(h, kernel, stream, a, alpha, beta, C);
}

gemm_status_t gemm_run_q(gemm_handle_t h, void* stream, int64_t M, int64_t N, int64_t K,
                         float alpha, const void* X, int64_t ldx, const uint8_t* Wq,
                         int64_t ldw, int bits, int64_t group, const void* scales,
                         const void* offsets, int64_t ldg, float beta, void* C, int64_t ldc,
                         gemm_dtype_t x_type, uint32_t epilogue, const float* bias) {
  return gemm_run_q_kernel(h, GEMM_KERNEL_AUTO, stream, M, N, K, alpha, X, ldx, Wq, ldw, bits,
                           group, scales, offsets, ldg, beta, C, ldc, x_type, epilogue, bias);
}

}  // extern "C"
