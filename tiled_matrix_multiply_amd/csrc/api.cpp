// Host side of the C ABI declared in include/gemm.h: argument validation, kernel selection and
// launches.  No allocation happens per call; every launch is asynchronous on the caller's
// stream.
#include "gemm.h"

#include <hip/hip_runtime.h>
#include <algorithm>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.hpp"
#include "handle.hpp"

namespace tgemm {
hipError_t launch_simt(const GemmParams& p, int a_type, int b_type, int transA, int transB,
                       hipStream_t s);
hipError_t launch_mfma_f32(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s,
                           int ks);
hipError_t launch_mfma_f16(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s,
                           int ks);
hipError_t launch_mfma_bf16(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s,
                            int ks);
#define TGEMM_F8_LAUNCHER(name) \
  hipError_t launch_mfma_##name(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s);
TGEMM_F8_LAUNCHER(e4m3)
TGEMM_F8_LAUNCHER(e5m2)
TGEMM_F8_LAUNCHER(e4m3_e5m2)
TGEMM_F8_LAUNCHER(e5m2_e4m3)
TGEMM_F8_LAUNCHER(mx_e4m3)
TGEMM_F8_LAUNCHER(mx_e5m2)
TGEMM_F8_LAUNCHER(mx_e4m3_e5m2)
TGEMM_F8_LAUNCHER(mx_e5m2_e4m3)
TGEMM_F8_LAUNCHER(e2m1)
TGEMM_F8_LAUNCHER(mx_e2m1)
TGEMM_F8_LAUNCHER(e2m3)
TGEMM_F8_LAUNCHER(e3m2)
TGEMM_F8_LAUNCHER(e2m3_e3m2)
TGEMM_F8_LAUNCHER(e3m2_e2m3)
TGEMM_F8_LAUNCHER(mx_e2m3)
TGEMM_F8_LAUNCHER(mx_e3m2)
TGEMM_F8_LAUNCHER(mx_e2m3_e3m2)
TGEMM_F8_LAUNCHER(mx_e3m2_e2m3)
#undef TGEMM_F8_LAUNCHER
hipError_t launch_bias_gelu(void* C, int64_t ldc, int M, int N, int c_type, const float* bias,
                            uint32_t epi, int cu_count, hipStream_t s);
hipError_t launch_clock_probe(uint64_t* out, int workgroups, uint64_t ticks, hipStream_t s);
hipError_t scratch_address(void** out);
int64_t scratch_bytes();
hipError_t launch_bandwidth_probe(const void* src, void* dst, int64_t bytes, uint32_t* sink,
                                  int cu_count, hipStream_t s);
}  // namespace tgemm

namespace {

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
  // OCP MX block scales (gemm_run_mx): mx set, sa / sb the E8M0 arrays
  bool mx;
  const uint8_t* sa;
  int64_t ldsa;
  const uint8_t* sb;
  int64_t ldsb;
};

// Storage bits per element (E2M1 packs two per byte, E2M3 / E3M2 four per three bytes).
int ebits(gemm_dtype_t t) {
  switch (t) {
    case GEMM_F32: return 32;
    case GEMM_F16: return 16;
    case GEMM_BF16: return 16;
    case GEMM_E4M3: return 8;
    case GEMM_E5M2: return 8;
    case GEMM_E2M1: return 4;
    case GEMM_E2M3: return 6;
    case GEMM_E3M2: return 6;
    default: return 0;
  }
}

bool is_fp8(gemm_dtype_t t) { return t == GEMM_E4M3 || t == GEMM_E5M2; }
bool is_fp6(gemm_dtype_t t) { return t == GEMM_E2M3 || t == GEMM_E3M2; }

bool supported_tuple(gemm_dtype_t a, gemm_dtype_t b, gemm_dtype_t c) {
  if (is_fp8(a) && is_fp8(b)) return c == GEMM_BF16;
  if (is_fp6(a) && is_fp6(b)) return c == GEMM_BF16;
  if (a != b) return false;
  switch (a) {
    case GEMM_F32: return c == GEMM_F32;
    case GEMM_F16: return c == GEMM_F16;
    case GEMM_BF16: return c == GEMM_BF16;
    case GEMM_E2M1: return c == GEMM_BF16;
    default: return false;
  }
}

// Byte range [lo, hi) touched by a rows x cols row-major matrix with leading dimension ld
// (elements of `bits` bits; a partly used last byte counts whole).
struct Range {
  __int128 lo, hi;
};
Range byte_range(const void* p, int64_t rows, int64_t cols, int64_t ld, int bits) {
  const __int128 lo = (__int128)(uintptr_t)p;
  if (rows <= 0 || cols <= 0) return {lo, lo};
  return {lo, lo + (((__int128)(rows - 1) * ld + cols) * bits + 7) / 8};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

gemm_status_t check(const Args& a) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_VALUE;
  if ((a.transA != 0 && a.transA != 1) || (a.transB != 0 && a.transB != 1))
    return GEMM_ERR_INVALID_VALUE;
  if (a.epi & ~(GEMM_EPI_BIAS | GEMM_EPI_GELU)) return GEMM_ERR_INVALID_VALUE;
  if (!ebits(a.at) || !ebits(a.bt) || !ebits(a.ct)) return GEMM_ERR_UNSUPPORTED;
  if (!supported_tuple(a.at, a.bt, a.ct)) return GEMM_ERR_UNSUPPORTED;
  if (a.mx && !(is_fp8(a.at) || a.at == GEMM_E2M1 || is_fp6(a.at))) return GEMM_ERR_UNSUPPORTED;
  // 6-bit operands: stored K-contiguous, rows starting on whole bytes
  if (is_fp6(a.at) && (a.transA != 0 || a.transB != 1 || a.K % 4 != 0 || a.lda % 4 != 0 ||
                       a.ldb % 4 != 0))
    return GEMM_ERR_UNSUPPORTED;
  if (a.M > kMaxDim || a.N > kMaxDim || a.K > kMaxDim) return GEMM_ERR_UNSUPPORTED;
  if (a.M == 0 || a.N == 0) return GEMM_OK;  // nothing to compute
  if (!a.C) return GEMM_ERR_INVALID_VALUE;
  if (a.ldc < a.N) return GEMM_ERR_INVALID_VALUE;
  if ((a.epi & GEMM_EPI_BIAS) && !a.bias) return GEMM_ERR_INVALID_VALUE;
  if (a.mx && a.K % 32 != 0) return GEMM_ERR_INVALID_VALUE;
  const Range rc = byte_range(a.C, a.M, a.N, a.ldc, ebits(a.ct));
  if (a.K > 0) {
    if (!a.A || !a.B) return GEMM_ERR_INVALID_VALUE;
    const int64_t a_rows = a.transA ? a.K : a.M, a_cols = a.transA ? a.M : a.K;
    const int64_t b_rows = a.transB ? a.N : a.K, b_cols = a.transB ? a.K : a.N;
    if (a.lda < a_cols || a.ldb < b_cols) return GEMM_ERR_INVALID_VALUE;
    if (overlaps(rc, byte_range(a.A, a_rows, a_cols, a.lda, ebits(a.at))) ||
        overlaps(rc, byte_range(a.B, b_rows, b_cols, a.ldb, ebits(a.bt))))
      return GEMM_ERR_ALIAS;
    if (a.mx) {
      const int64_t kb = a.K / 32;
      if (!a.sa || !a.sb || a.ldsa < kb || a.ldsb < kb) return GEMM_ERR_INVALID_VALUE;
      if (overlaps(rc, byte_range(a.sa, a.M, kb, a.ldsa, 8)) ||
          overlaps(rc, byte_range(a.sb, a.N, kb, a.ldsb, 8)))
        return GEMM_ERR_ALIAS;
    }
  }
  if ((a.epi & GEMM_EPI_BIAS) && overlaps(rc, byte_range(a.bias, 1, a.N, a.N, 32)))
    return GEMM_ERR_ALIAS;
  return GEMM_OK;
}

// Matrix-core kernels read 16-byte chunks of A and B and store 4-element runs of C.
bool mfma_aligned(const Args& a) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (a.at == GEMM_E2M1) {
    // packed fp4 is staged as bytes along K: A stored M x K, B stored N x K, whole bytes
    if (a.transA != 0 || a.transB != 1 || a.K % 2 != 0) return false;
  }
  if (is_fp6(a.at)) {
    // packed 6-bit rows are staged as bytes along K in whole 96-byte (128-element) K tiles
    if (a.K % 128 != 0) return false;
  }
  if (a.K > 0) {
    if (!al16(a.A) || !al16(a.B)) return false;
    const int64_t lda_bits = a.lda * ebits(a.at), ldb_bits = a.ldb * ebits(a.bt);
    if (lda_bits % 128 != 0 || ldb_bits % 128 != 0) return false;
    // per-lane 32-bit buffer offsets span up to 256 rows of a staged tile
    if (lda_bits / 8 > kMaxRowBytes || ldb_bits / 8 > kMaxRowBytes) return false;
    if (a.mx) {
      // 16-byte scale pieces per row, addressed by 32-bit offsets
      if (!al16(a.sa) || !al16(a.sb) || a.ldsa % 16 != 0 || a.ldsb % 16 != 0) return false;
      if ((__int128)a.M * a.ldsa >= ((__int128)1 << 32) - 16 ||
          (__int128)a.N * a.ldsb >= ((__int128)1 << 32) - 16)
        return false;
    }
  }
  return al16(a.C) && (a.ldc % 4 == 0);
}

int64_t tiles(int64_t M, int64_t N, int64_t t) { return ((M + t - 1) / t) * ((N + t - 1) / t); }

// K split of the 64 x 64 tile (16- and 32-bit inputs): when its tiles take at most two rounds
// of the compute units and K holds at least four tiles, two groups of waves in each workgroup
// take the even and the odd K tiles.  A small product is a chain of K tiles, each a copy, a
// barrier and a few multiplies: halving the chain took fp16 1024^3 from 8.0 to 7.3 us, and
// bf16 + bias + GELU 1024 x 2048 x 2048 (512 tiles) from 23.6 to 21.6 us.
int k_split(const Args& a, int cu_count) {
  if (a.at != GEMM_F32 && a.at != GEMM_F16 && a.at != GEMM_BF16) return 1;
  const int64_t t = tiles(a.M, a.N, 64);
  const int64_t bke = 128 / (ebits(a.at) / 8);  // K elements per staged tile
  const int64_t kt = (a.K + bke - 1) / bke;
  return (t <= 2 * (int64_t)cu_count && kt >= 4) ? 2 : 1;
}

// The 256 x 128 tile (unsplit, GEMM_KERNEL_MFMA_256x128, and split across two workgroups) takes
// fp16 and bf16 inputs only.
bool split_k_fits(const Args& a) {
  return (a.at == GEMM_F16 || a.at == GEMM_BF16) && !a.mx;
}
int64_t split_k_tiles(const Args& a) { return ((a.M + 255) / 256) * ((a.N + 127) / 128); }

// The kernel family AUTO picks: broadly, the largest tile that still keeps the compute units busy.
gemm_kernel_t auto_kernel(const Args& a, int cu_count) {
  if (!mfma_aligned(a)) return GEMM_KERNEL_SIMT;
  // 64 x 64 tiles would leave three quarters of the compute units idle: 32 x 32 tiles with the
  // K loop split four ways (16- and 32-bit inputs)
  if ((a.at == GEMM_F32 || a.at == GEMM_F16 || a.at == GEMM_BF16) && 4 * tiles(a.M, a.N, 64) <= cu_count)
    return GEMM_KERNEL_MFMA_32;
  if (tiles(a.M, a.N, 256) >= cu_count) return GEMM_KERNEL_MFMA_256;
  // Between one and two rounds of 128 x 128 workgroups, the 256 x 128 tile (16-bit inputs) does
  // the work in a single round whenever its own tiles fit on the compute units: every such
  // shape measured ran faster or equal (bf16 + bias + GELU, 128 x 128 vs 256 x 128 tile:
  // 2048 x 4096 x 4096 86.6 vs 73.2 us, 1280 x 4096 x 4096 80.1 vs 64.2 us, 2560^3 59.1 vs
  // 45.9 us, 1100 x 4104 x 4096 105.6 vs 73.1 us, 2176^3 51.6 vs 51.9 us).  At one round of
  // 128 x 128 workgroups or fewer the 128 tile stays far ahead (1024 x 4096 x 4096 46.7 vs
  // 63.3 us, 2048^2 x 8192 83.2 vs 114.5 us).
  if (split_k_fits(a) && tiles(a.M, a.N, 128) > cu_count && split_k_tiles(a) <= cu_count)
    return GEMM_KERNEL_MFMA_256x128;
  // More than two rounds of 128 x 128 workgroups cost more than one partly filled round of
  // 256 x 256 ones (bf16 + bias + GELU: 3072^3 80 vs 98 us, 3584^3 101 vs 146 us; at two
  // rounds or fewer the 128 tile beats the 256 x 256 one, 2816^3 65 vs 73 us, 4096 x 2048 x
  // 4096 85 vs 99 us, though for 16-bit inputs the 256 x 128 tile above takes most such shapes).
  if (tiles(a.M, a.N, 128) > 2 * (int64_t)cu_count) return GEMM_KERNEL_MFMA_256;
  // The 128 tile (its K loop split between two wave groups for 16- and 32-bit types) also
  // beats 64 x 64 tiles with some compute units idle, from about 9/16 of them busy: 1792^3
  // 25.0 vs 28.8 us, 1536 x 1536 x 4096 42.2 vs 47.8 us; below, 1280^3 18.3 vs 14.9 us.
  if (16 * tiles(a.M, a.N, 128) >= 9 * (int64_t)cu_count) return GEMM_KERNEL_MFMA_128;
  return GEMM_KERNEL_MFMA_64;
}

// The K loop split across two workgroups (256 x 128 tiles, 16-bit inputs, GEMM_KERNEL_MFMA_256x128_SK2)
// was built for mid-size products, whose 128 x 128 tiles give each compute unit one workgroup
// walking the whole K loop.  Measured per launch (one box, back to back), against the 128 x 128
// tile with its K loop split inside the workgroup that AUTO picks:
//   fp16 2048^3              22.2 us   split 26.7 us   (256 x 128 unsplit, 128 workgroups: 30.6 us)
//   bf16 + bias + GELU 2048^3 25.6 us  split 30.9 us
//   bf16 + bias + GELU 1536^3 20.5 us  split 25.3 us
//   bf16 + bias + GELU 2048 x 2048 x 4096   41.9 us   split 45.3 us
//   bf16 + bias + GELU 1024 x 2048 x 2048   19.2 us   split 28.3 us
// The hand-off of 128 KiB of partial sums per tile through device-coherent memory, plus the
// second half's wait, costs about what the halved K loop saves, so AUTO does not take it; it
// stays available as an explicit kernel family (gemm_run_ws_kernel).
bool split_k_wins(const Args&, int) { return false; }
// Workspace of the split kernel: one slot per 256 x 128 output tile (tgemm::kSplitSlotBytes:
// the tile's counter and flag, then its fp32 partial sums), tile t in slot t.
int64_t split_k_ws_bytes(const Args& a) { return split_k_tiles(a) * tgemm::kSplitSlotBytes; }

// Stream-K (GEMM_KERNEL_MFMA_256_SK, 256 x 256 tiles): two slots of fp32 partial sums per
// workgroup of the largest grid the device runs (one per compute unit), then an [arrive, done]
// pair of counters per output tile.  The slots come first, so that the counters sit at the same
// offset for every call on the device and calls of different sizes can share a workspace.
int64_t stream_k_slot_region(int cu_count) { return 2 * (int64_t)cu_count * tgemm::kStreamSlotBytes; }
int64_t stream_k_ws_bytes(const Args& a, int cu_count) {
  return stream_k_slot_region(cu_count) + ((8 * tiles(a.M, a.N, 256) + 255) / 256) * 256;
}
bool stream_k_wins(const Args&, int) { return false; }

using tgemm::DeviceGuard;

}  // namespace

static bool valid(gemm_handle_t h) { return h && h->magic == tgemm::kHandleMagic; }

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
  h->magic = tgemm::kHandleMagic;
  h->device = device;
  h->cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  int wall = 0;
  if (hipDeviceGetAttribute(&wall, hipDeviceAttributeWallClockRate, device) != hipSuccess) {
    (void)hipGetLastError();
    wall = 0;
  }
  h->wall_clock_khz = wall;
  {
    // the static scratch array's address on this device (for gemm_run_noalloc)
    DeviceGuard g(device);
    void* ptr = nullptr;
    if (tgemm::scratch_address(&ptr) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      free(h);
      return GEMM_ERR_DEVICE;
    }
    h->scratch = ptr;
    h->scratch_bytes = tgemm::scratch_bytes();
  }
  strncpy(h->arch, prop.gcnArchName, sizeof(h->arch) - 1);
  *out = h;
  return GEMM_OK;
}

gemm_status_t gemm_destroy(gemm_handle_t h) {
  if (!h) return GEMM_OK;
  if (h->magic != tgemm::kHandleMagic) return GEMM_ERR_INVALID_HANDLE;
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

}  // extern "C"

namespace {

// The 8- and 4-bit matrix-core launcher for an (A, B, block-scaled) combination.
using Launcher = hipError_t (*)(const tgemm::GemmParams&, int, bool, bool, hipStream_t);
Launcher f8_launcher(gemm_dtype_t at, gemm_dtype_t bt, bool mx) {
  using namespace tgemm;
  if (at == GEMM_E2M1) return mx ? launch_mfma_mx_e2m1 : launch_mfma_e2m1;
  if (is_fp6(at)) {
    const bool a3 = at == GEMM_E3M2, b3 = bt == GEMM_E3M2;
    if (mx) {
      if (!a3 && !b3) return launch_mfma_mx_e2m3;
      if (a3 && b3) return launch_mfma_mx_e3m2;
      return a3 ? launch_mfma_mx_e3m2_e2m3 : launch_mfma_mx_e2m3_e3m2;
    }
    if (!a3 && !b3) return launch_mfma_e2m3;
    if (a3 && b3) return launch_mfma_e3m2;
    return a3 ? launch_mfma_e3m2_e2m3 : launch_mfma_e2m3_e3m2;
  }
  const bool a5 = at == GEMM_E5M2, b5 = bt == GEMM_E5M2;
  if (mx) {
    if (!a5 && !b5) return launch_mfma_mx_e4m3;
    if (a5 && b5) return launch_mfma_mx_e5m2;
    return a5 ? launch_mfma_mx_e5m2_e4m3 : launch_mfma_mx_e4m3_e5m2;
  }
  if (!a5 && !b5) return launch_mfma_e4m3;
  if (a5 && b5) return launch_mfma_e5m2;
  return a5 ? launch_mfma_e5m2_e4m3 : launch_mfma_e4m3_e5m2;
}

gemm_status_t run_impl(gemm_handle_t h, gemm_kernel_t kernel, void* stream, const Args& a,
                       float alpha, float scale_a, float scale_b, float beta, void* C,
                       void* ws = nullptr, int64_t ws_bytes = 0) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  gemm_status_t st = check(a);
  if (st != GEMM_OK) return st;
  if (ws_bytes < 0 || (ws_bytes > 0 && !ws)) return GEMM_ERR_INVALID_VALUE;
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return GEMM_ERR_INVALID_VALUE;
  if (a.M == 0 || a.N == 0) return GEMM_OK;
  if (kernel == GEMM_KERNEL_AUTO) {
    kernel = auto_kernel(a, h->cu_count);
    // with a workspace large enough, mid-size 16-bit products split K over two workgroups
    if (ws && kernel != GEMM_KERNEL_SIMT && split_k_wins(a, h->cu_count) &&
        ws_bytes >= split_k_ws_bytes(a))
      kernel = GEMM_KERNEL_MFMA_256x128_SK2;
    else if (ws && kernel != GEMM_KERNEL_SIMT && stream_k_wins(a, h->cu_count) &&
             ws_bytes >= stream_k_ws_bytes(a, h->cu_count))
      kernel = GEMM_KERNEL_MFMA_256_SK;
  }
  // with no K tiles there is nothing to share out: the plain 256 x 256 tile runs the epilogue
  if (kernel == GEMM_KERNEL_MFMA_256_SK && a.K == 0) kernel = GEMM_KERNEL_MFMA_256;

  tgemm::GemmParams p{};
  p.A = a.A;
  p.B = a.B;
  p.C = C;
  p.bias = a.bias;
  p.lda = a.lda;
  p.ldb = a.ldb;
  p.ldc = a.ldc;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.alpha = alpha * scale_a * scale_b;
  p.beta = beta;
  p.epi = a.epi;
  if (a.mx) {
    p.sa = a.sa;
    p.sb = a.sb;
    p.ldsa = a.ldsa;
    p.ldsb = a.ldsb;
    p.kblocks = (int)(a.K / 32);
  }

  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (kernel == GEMM_KERNEL_SIMT) {
    // any M and N: the scalar kernel strides over its tiles with a bounded grid
    DeviceGuard g(h->device);
    err = tgemm::launch_simt(p, a.at, a.bt, a.transA, a.transB, s);
  } else if ((kernel >= GEMM_KERNEL_MFMA_64 && kernel <= GEMM_KERNEL_MFMA_256) ||
             kernel == GEMM_KERNEL_MFMA_32 || kernel == GEMM_KERNEL_MFMA_256x128 ||
             kernel == GEMM_KERNEL_MFMA_256x128_SK2 || kernel == GEMM_KERNEL_MFMA_256_SK) {
    if (!mfma_aligned(a)) return GEMM_ERR_UNSUPPORTED;
    if (kernel == GEMM_KERNEL_MFMA_32 && a.at != GEMM_F32 && a.at != GEMM_F16 && a.at != GEMM_BF16)
      return GEMM_ERR_UNSUPPORTED;
    const bool wide = kernel == GEMM_KERNEL_MFMA_256x128 || kernel == GEMM_KERNEL_MFMA_256x128_SK2;
    const bool stream = kernel == GEMM_KERNEL_MFMA_256_SK;
    if ((wide || stream) && !split_k_fits(a)) return GEMM_ERR_UNSUPPORTED;
    if (kernel == GEMM_KERNEL_MFMA_256x128_SK2) {
      if (!ws || ws_bytes < split_k_ws_bytes(a)) return GEMM_ERR_INVALID_VALUE;
      p.sk_ws = static_cast<uint8_t*>(ws);
    }
    const int tile = kernel == GEMM_KERNEL_MFMA_32 ? 3
                     : kernel == GEMM_KERNEL_MFMA_256x128 ? 5
                     : kernel == GEMM_KERNEL_MFMA_256x128_SK2 ? 6
                     : stream ? 7
                     : kernel - GEMM_KERNEL_MFMA_64;
    const int tmr = kernel == GEMM_KERNEL_MFMA_32 ? 32 : (wide || stream) ? 256 : 64 << tile;
    const int tnc = wide ? 128 : tmr;
    const int64_t tm = (a.M + tmr - 1) / tmr, tn = (a.N + tnc - 1) / tnc;
    if (tm * tn * 2 > kMaxDim) return GEMM_ERR_UNSUPPORTED;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    if (stream) {
      if (!ws || ws_bytes < stream_k_ws_bytes(a, h->cu_count)) return GEMM_ERR_INVALID_VALUE;
      // one persistent workgroup per compute unit (a 256 x 256 tile's stages fill most of its
      // LDS, so one runs on each at a time), and no more than K tiles (64 elements of K each),
      // so that no run is empty
      const int64_t kt = (a.K + 63) / 64;
      p.sk_ws = static_cast<uint8_t*>(ws);
      p.sk_cnt_off = stream_k_slot_region(h->cu_count);
      p.sk_grid = (int)std::min<int64_t>(h->cu_count, tm * tn * kt);
    }
    if (a.at == GEMM_E2M1) {
      // the matrix-core kernels stage packed fp4 rows as bytes: K and the leading dimensions
      // are passed in bytes (two elements each); the block count stays in elements / 32
      p.K = (int)(a.K / 2);
      p.lda = a.lda / 2;
      p.ldb = a.ldb / 2;
    } else if (is_fp6(a.at)) {
      // the same for packed 6-bit rows: three bytes per four elements
      p.K = (int)(a.K / 4 * 3);
      p.lda = a.lda / 4 * 3;
      p.ldb = a.ldb / 4 * 3;
    }
    // Storage contiguous along M (A stored K x M) or along N (B stored K x N).
    const bool a_mn = a.transA != 0, b_mn = a.transB == 0;
    const int ks = tile == 0 ? k_split(a, h->cu_count) : 1;
    DeviceGuard g(h->device);
    switch (a.at) {
      case GEMM_F32: err = tgemm::launch_mfma_f32(p, tile, a_mn, b_mn, s, ks); break;
      case GEMM_F16: err = tgemm::launch_mfma_f16(p, tile, a_mn, b_mn, s, ks); break;
      case GEMM_BF16: err = tgemm::launch_mfma_bf16(p, tile, a_mn, b_mn, s, ks); break;
      case GEMM_E4M3:
      case GEMM_E5M2:
      case GEMM_E2M1:
      case GEMM_E2M3:
      case GEMM_E3M2: err = f8_launcher(a.at, a.bt, a.mx)(p, tile, a_mn, b_mn, s); break;
      default: return GEMM_ERR_UNSUPPORTED;
    }
  } else {
    return GEMM_ERR_INVALID_VALUE;
  }
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

gemm_status_t gemm_run_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                              int64_t N, int64_t K, int transA, int transB, float alpha,
                              const void* A, int64_t lda, float scale_a, const void* B,
                              int64_t ldb, float scale_b, float beta, void* C, int64_t ldc,
                              gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                              uint32_t epilogue, const float* bias) {
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  return run_impl(h, kernel, stream, a, alpha, scale_a, scale_b, beta, C);
}

gemm_status_t gemm_run_ws_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                                 int64_t N, int64_t K, int transA, int transB, float alpha,
                                 const void* A, int64_t lda, float scale_a, const void* B,
                                 int64_t ldb, float scale_b, float beta, void* C, int64_t ldc,
                                 gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                                 uint32_t epilogue, const float* bias, void* workspace,
                                 int64_t workspace_bytes) {
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  return run_impl(h, kernel, stream, a, alpha, scale_a, scale_b, beta, C, workspace,
                  workspace_bytes);
}

gemm_status_t gemm_run_noalloc(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                               int64_t N, int64_t K, int transA, int transB, float alpha,
                               const void* A, int64_t lda, float scale_a, const void* B,
                               int64_t ldb, float scale_b, float beta, void* C, int64_t ldc,
                               gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                               uint32_t epilogue, const float* bias) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  const gemm_status_t st = check(a);
  if (st != GEMM_OK) return st;
  // the kernels that use scratch: refuse what the static array cannot hold
  if (kernel == GEMM_KERNEL_MFMA_256x128_SK2 && a.M > 0 && a.N > 0 &&
      split_k_ws_bytes(a) > h->scratch_bytes)
    return GEMM_ERR_TOO_LARGE;
  if (kernel == GEMM_KERNEL_MFMA_256_SK && a.M > 0 && a.N > 0 && a.K > 0 &&
      stream_k_ws_bytes(a, h->cu_count) > h->scratch_bytes)
    return GEMM_ERR_TOO_LARGE;
  return run_impl(h, kernel, stream, a, alpha, scale_a, scale_b, beta, C, h->scratch,
                  h->scratch_bytes);
}

gemm_status_t gemm_run_ws(gemm_handle_t h, void* stream, int64_t M, int64_t N, int64_t K,
                          int transA, int transB, float alpha, const void* A, int64_t lda,
                          float scale_a, const void* B, int64_t ldb, float scale_b, float beta,
                          void* C, int64_t ldc, gemm_dtype_t a_type, gemm_dtype_t b_type,
                          gemm_dtype_t c_type, uint32_t epilogue, const float* bias,
                          void* workspace, int64_t workspace_bytes) {
  return gemm_run_ws_kernel(h, GEMM_KERNEL_AUTO, stream, M, N, K, transA, transB, alpha, A, lda,
                            scale_a, B, ldb, scale_b, beta, C, ldc, a_type, b_type, c_type,
                            epilogue, bias, workspace, workspace_bytes);
}

int64_t gemm_workspace_bytes(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int transA,
                             int transB, const void* A, int64_t lda, const void* B, int64_t ldb,
                             const void* C, int64_t ldc, gemm_dtype_t a_type, gemm_dtype_t b_type,
                             gemm_dtype_t c_type, uint32_t epilogue, const float* bias) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias};
  const gemm_status_t st = check(a);
  if (st != GEMM_OK) return st;
  if (a.M == 0 || a.N == 0 || auto_kernel(a, h->cu_count) == GEMM_KERNEL_SIMT) return 0;
  if (split_k_wins(a, h->cu_count)) return split_k_ws_bytes(a);
  if (stream_k_wins(a, h->cu_count)) return stream_k_ws_bytes(a, h->cu_count);
  return 0;
}

int64_t gemm_kernel_workspace_bytes(gemm_handle_t h, gemm_kernel_t kernel, int64_t M, int64_t N) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return GEMM_ERR_INVALID_VALUE;
  Args a{};
  a.M = M;
  a.N = N;
  if (kernel == GEMM_KERNEL_MFMA_256x128_SK2) return split_k_ws_bytes(a);
  if (kernel == GEMM_KERNEL_MFMA_256_SK) return stream_k_ws_bytes(a, h->cu_count);
  return 0;
}

gemm_status_t gemm_run_mx_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                                 int64_t N, int64_t K, int transA, int transB, float alpha,
                                 const void* A, int64_t lda, const uint8_t* sa, int64_t ldsa,
                                 const void* B, int64_t ldb, const uint8_t* sb, int64_t ldsb,
                                 float beta, void* C, int64_t ldc, gemm_dtype_t a_type,
                                 gemm_dtype_t b_type, gemm_dtype_t c_type, uint32_t epilogue,
                                 const float* bias) {
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias, true, sa, ldsa, sb, ldsb};
  return run_impl(h, kernel, stream, a, alpha, 1.0f, 1.0f, beta, C);
}

gemm_status_t gemm_check_args_mx(int64_t M, int64_t N, int64_t K, int transA, int transB,
                                 const void* A, int64_t lda, const uint8_t* sa, int64_t ldsa,
                                 const void* B, int64_t ldb, const uint8_t* sb, int64_t ldsb,
                                 const void* C, int64_t ldc, gemm_dtype_t a_type,
                                 gemm_dtype_t b_type, gemm_dtype_t c_type, uint32_t epilogue,
                                 const float* bias) {
  const Args a{M, N, K, transA, transB, A, lda, B, ldb, C, ldc, a_type, b_type, c_type,
               epilogue, bias, true, sa, ldsa, sb, ldsb};
  return check(a);
}

gemm_status_t gemm_run_mx(gemm_handle_t h, void* stream, int64_t M, int64_t N, int64_t K,
                          int transA, int transB, float alpha, const void* A, int64_t lda,
                          const uint8_t* sa, int64_t ldsa, const void* B, int64_t ldb,
                          const uint8_t* sb, int64_t ldsb, float beta, void* C, int64_t ldc,
                          gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                          uint32_t epilogue, const float* bias) {
  return gemm_run_mx_kernel(h, GEMM_KERNEL_AUTO, stream, M, N, K, transA, transB, alpha, A, lda,
                            sa, ldsa, B, ldb, sb, ldsb, beta, C, ldc, a_type, b_type, c_type,
                            epilogue, bias);
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
      overlaps(byte_range(C, M, N, ldc, ebits(c_type)), byte_range(bias, 1, N, N, 32)))
    return GEMM_ERR_ALIAS;
  DeviceGuard g(h->device);
  const hipError_t err = tgemm::launch_bias_gelu(C, ldc, (int)M, (int)N, c_type, bias, epilogue,
                                                 h->cu_count, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

gemm_status_t gemm_probe_clock(gemm_handle_t h, void* stream, uint64_t* out, int workgroups,
                               int microseconds) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  if (!out || workgroups <= 0 || workgroups > 65536 || microseconds <= 0 || microseconds > 100000)
    return GEMM_ERR_INVALID_VALUE;
  if (h->wall_clock_khz <= 0) return GEMM_ERR_DEVICE;
  const uint64_t ticks = (uint64_t)h->wall_clock_khz * (uint64_t)microseconds / 1000u;
  DeviceGuard g(h->device);
  const hipError_t err = tgemm::launch_clock_probe(out, workgroups, ticks ? ticks : 1,
                                                   static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_wall_clock_khz(gemm_handle_t h) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  return h->wall_clock_khz;
}

gemm_status_t gemm_probe_bandwidth(gemm_handle_t h, void* stream, const void* src, void* dst,
                                   int64_t bytes, uint32_t* sink) {
  if (!valid(h)) return GEMM_ERR_INVALID_HANDLE;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!src || bytes <= 0 || bytes % 16 != 0 || !al16(src) || (dst && !al16(dst)))
    return GEMM_ERR_INVALID_VALUE;
  if (!dst && !sink) return GEMM_ERR_INVALID_VALUE;
  if (dst && overlaps(byte_range(src, 1, bytes, bytes, 8), byte_range(dst, 1, bytes, bytes, 8)))
    return GEMM_ERR_ALIAS;
  DeviceGuard g(h->device);
  const hipError_t err = tgemm::launch_bandwidth_probe(src, dst, bytes, sink, h->cu_count,
                                                       static_cast<hipStream_t>(stream));
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
    case GEMM_ERR_TOO_LARGE:
      return "GEMM_ERR_TOO_LARGE: the problem needs more scratch than the library's static buffer holds";
    default: return "GEMM_ERR_UNKNOWN";
  }
}

}  // extern "C"
