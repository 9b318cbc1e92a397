/*
 * gemm.h -- C ABI of the tiled GEMM library for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * One operation:
 *
 *     C = epi( alpha * scale_a * scale_b * op(A) * op(B)  +  beta * C  [+ bias] )
 *
 * with op(X) = X or X^T chosen by a flag, fp32 accumulation, and an epilogue that may add a
 * per-column bias and apply the erf form of GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).
 *
 * Where it comes from:
 *   - the BLAS form alpha*AB + beta*C computed in one fused store: "Case Study: The Tiled GEMM"
 *     (its epilogue paragraph);
 *   - bias / activation / scaling applied to every accumulator in registers before a single
 *     store, and transposition expressed purely through strides: "Case Study: Steel's
 *     BlockMMA" (its store_result and stride-constant paragraphs);
 *   - operands described by a base pointer plus explicit strides, with the output tile shape
 *     chosen by the library: "Rigel" (arXiv 2606.12765), section 2 (tensor_handle,
 *     matmul2d_descriptor);
 *   - the fused GEMM + bias + GELU versus the decomposed path, and fp8 E4M3 operands:
 *     "Rigel", abstract and section 1 (contribution 7);
 *   - the other low-precision formats it lists beside fp8, fp4 and block-scaled MXFP4:
 *     "Rigel", section 1 (the formats Metal 4.1 adds); the 6-bit types of the same OCP
 *     microscaling family (E2M3, E3M2) follow the OCP MX v1.0 specification, which the pages
 *     do not cover.
 *
 * Conventions shared by every entry point:
 *   - Storage is row-major.  Element (r, c) of a stored matrix X with leading dimension ldX is
 *     X[r * ldX + c].  A is stored M x K (lda >= K) or, with transA, K x M (lda >= M); B is
 *     stored K x N (ldb >= N) or, with transB, N x K (ldb >= K); C is M x N (ldc >= N).
 *     Leading dimensions and sizes are counted in elements.
 *   - Supported (A, B, C) type tuples: (F32,F32,F32), (F16,F16,F16), (BF16,BF16,BF16),
 *     (X,Y,BF16) for X, Y in {E4M3, E5M2}, (E2M1,E2M1,BF16), and (X,Y,BF16) for X, Y in
 *     {E2M3, E3M2}.  E4M3 and E5M2 are the OCP 8-bit floats (E4M3: bias 7, max 448, no
 *     infinities; E5M2: bias 15, max 57344, IEEE-style infinities and NaN).  E2M1 is the OCP
 *     4-bit float (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), stored two per byte along each
 *     stored row: element c of a row sits in byte c / 2, in the low nibble when c is even.
 *     E2M3 (bias 1, max 7.5) and E3M2 (bias 3, max 28) are the OCP 6-bit floats, without
 *     infinities or NaN, stored four per three bytes along each stored row: element c of a row
 *     occupies bits 6c .. 6c+5 of the row's bytes read as one little-endian integer.  The
 *     6-bit types need A stored M x K and B stored N x K, and K, lda and ldb multiples of 4
 *     (rows start on whole bytes).  Any other tuple returns GEMM_ERR_UNSUPPORTED.
 *   - Pointers A, B, C and bias are DEVICE pointers owned by the caller.  C is read (only when
 *     beta != 0) and written.  Nothing is allocated and nothing is retained after a call.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream).  They
 *     enqueue kernels and return; results are visible after the stream synchronises.  Device
 *     faults surface at the caller's next synchronisation, not as a return value.
 *   - Invalid arguments return a negative status and enqueue nothing.
 *   - A handle is immutable after gemm_create and may be shared by threads.
 */
#ifndef TILED_GEMM_H
#define TILED_GEMM_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GEMM_API __attribute__((visibility("default")))
#else
#define GEMM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_status {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_HANDLE = -1, /* null or destroyed handle */
  GEMM_ERR_INVALID_VALUE = -2,  /* negative size, null pointer, leading dimension too small,
                                   bias flag without bias, unknown epilogue bits, trans not 0/1 */
  GEMM_ERR_UNSUPPORTED = -3,    /* type tuple not supported, size beyond 2^31-1, or a forced
                                   kernel that cannot serve this layout/alignment */
  GEMM_ERR_ALIAS = -4,          /* C's byte range overlaps A, B or bias */
  GEMM_ERR_DEVICE = -5,         /* no such device, device is not gfx950, or a HIP error at
                                   gemm_create */
  GEMM_ERR_LAUNCH = -6,         /* the kernel launch itself failed (hipGetLastError) */
  GEMM_ERR_NO_MEMORY = -7,      /* host allocation of the handle failed */
  GEMM_ERR_TOO_LARGE = -8       /* gemm_run_noalloc: the problem needs more scratch than the
                                   library's static buffer holds */
} gemm_status_t;

typedef enum gemm_dtype {
  GEMM_F32 = 0,
  GEMM_F16 = 1,
  GEMM_BF16 = 2,
  GEMM_E4M3 = 3,
  GEMM_E5M2 = 4,
  GEMM_E2M1 = 5,
  GEMM_E2M3 = 6,
  GEMM_E3M2 = 7
} gemm_dtype_t;

/* Epilogue bits.  BIAS adds bias[j] (fp32, length N, one value per output column, broadcast
 * over rows, not scaled by alpha).  GELU applies x * Phi(x) after everything else.  Order:
 * GELU(alpha*sa*sb*acc + beta*C + bias), rounded once to C's type (round to nearest even). */
#define GEMM_EPI_NONE 0u
#define GEMM_EPI_BIAS 1u
#define GEMM_EPI_GELU 2u

/* Kernel families, for gemm_run_kernel.  AUTO picks by type, layout, alignment and size. */
typedef enum gemm_kernel {
  GEMM_KERNEL_AUTO = 0,
  GEMM_KERNEL_SIMT = 1,     /* LDS-tiled scalar FMA without matrix cores: a 64x64 tile per
                               workgroup, a 4x4 register block per thread, double-buffered K
                               slices (the shared-memory tiling of "X3: Metal GEMM", section
                               2).  Any alignment, layout and size. */
  GEMM_KERNEL_MFMA_64 = 2,  /* matrix-core kernel, 64x64 workgroup tile, 4 wavefronts */
  GEMM_KERNEL_MFMA_128 = 3, /* matrix-core kernel, 128x128 workgroup tile, 4 wavefronts */
  GEMM_KERNEL_MFMA_256 = 4, /* matrix-core kernel, 256x256 workgroup tile, 8 wavefronts */
  GEMM_KERNEL_QGEMV = 5,    /* gemm_run_q only: matrix-vector kernel for a few activation rows,
                               bound by the bandwidth of the weight codes */
  GEMM_KERNEL_QMFMA = 6,    /* gemm_run_q only: matrix-core kernel that dequantises the codes
                               in registers (prefill) */
  GEMM_KERNEL_MFMA_32 = 7,  /* matrix-core kernel, 32x32 workgroup tile, 4 wavefronts that
                               split the K loop four ways; fp32, fp16 and bf16 only (other
                               types return GEMM_ERR_UNSUPPORTED).  AUTO takes it when 64x64
                               tiles would leave three quarters of the compute units idle */
  GEMM_KERNEL_MFMA_256x128 = 8,     /* matrix-core kernel, 256x128 workgroup tile, 8 wavefronts
                                       of 64x64; fp16 and bf16 only.  AUTO takes it when
                                       128x128 tiles would need more than one round of the
                                       compute units and 256x128 tiles need at most one */
  GEMM_KERNEL_MFMA_256x128_SK2 = 9, /* the 256x128 tile with its K loop split across two
                                       workgroups that meet through a workspace: gemm_run_ws /
                                       gemm_run_ws_kernel only; fp16 and bf16 only */
  GEMM_KERNEL_MFMA_256_SK = 10      /* stream-K: the 256x256 tile on a persistent grid of
                                       one workgroup per compute unit that shares out the K
                                       tiles of all output tiles evenly; the parts of a split
                                       tile meet through a workspace: gemm_run_ws /
                                       gemm_run_ws_kernel only; fp16 and bf16 only */
} gemm_kernel_t;

typedef struct gemm_handle* gemm_handle_t;

/* Create a handle bound to HIP device `device`.  Checks that the device is a gfx950 and
 * records its compute-unit count for tile selection.  *out receives the handle (NULL on
 * failure).  Errors: GEMM_ERR_INVALID_VALUE (out == NULL), GEMM_ERR_DEVICE (no such device,
 * not gfx950, HIP error), GEMM_ERR_NO_MEMORY. */
GEMM_API gemm_status_t gemm_create(gemm_handle_t* out, int device);

/* Destroy a handle.  NULL is accepted and ignored.  Work already enqueued is unaffected. */
GEMM_API gemm_status_t gemm_destroy(gemm_handle_t h);

/* Check the arguments of gemm_run without touching any device.  Returns the status gemm_run
 * would return for them before launching (GEMM_OK when they are valid).  M == 0 or N == 0 is a
 * valid no-op; K == 0 is valid and yields C = epi(beta * C [+ bias]).  When K == 0, A and B are
 * not read and may be NULL. */
GEMM_API gemm_status_t gemm_check_args(int64_t M, int64_t N, int64_t K, int transA, int transB,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              const void* C, int64_t ldc, gemm_dtype_t a_type,
                              gemm_dtype_t b_type, gemm_dtype_t c_type, uint32_t epilogue,
                              const float* bias);

/* C = epi(alpha * scale_a * scale_b * op(A) op(B) + beta * C [+ bias]) on `stream`.
 * scale_a / scale_b are the per-tensor dequantisation scales of 8- and 4-bit operands (pass
 * 1.0f for other types; they multiply the product for every type).  beta == 0 means C is not read, so
 * NaN in C does not propagate.  The kernel is chosen automatically (GEMM_KERNEL_AUTO). */
GEMM_API gemm_status_t gemm_run(gemm_handle_t h, void* stream, int64_t M, int64_t N, int64_t K,
                       int transA, int transB, float alpha, const void* A, int64_t lda,
                       float scale_a, const void* B, int64_t ldb, float scale_b, float beta,
                       void* C, int64_t ldc, gemm_dtype_t a_type, gemm_dtype_t b_type,
                       gemm_dtype_t c_type, uint32_t epilogue, const float* bias);

/* gemm_run with an explicit kernel family.  Matrix-core kernels need 16-byte-aligned A, B and
 * C, lda * sizeof(A elem) and ldb * sizeof(B elem) multiples of 16 bytes, and ldc a multiple of
 * 4; E2M1 operands also need A stored M x K, B stored N x K and K even.  Otherwise they return
 * GEMM_ERR_UNSUPPORTED (AUTO then uses GEMM_KERNEL_SIMT). */
GEMM_API gemm_status_t gemm_run_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream, int64_t M,
                              int64_t N, int64_t K, int transA, int transB, float alpha,
                              const void* A, int64_t lda, float scale_a, const void* B,
                              int64_t ldb, float scale_b, float beta, void* C, int64_t ldc,
                              gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                              uint32_t epilogue, const float* bias);

/* gemm_run with a caller-provided device workspace, for kernels that split the K loop across
 * workgroups (the mid-size regime, fewer output tiles than compute units, where "Rigel"
 * (arXiv 2606.12765), section 3, finds small sizes clock- and latency-bound).  The split kernel,
 * GEMM_KERNEL_MFMA_256x128_SK2: each 256 x 128 tile's two workgroups multiply one half of K each;
 * the first to finish writes its fp32 partial sums into the workspace and raises a per-tile
 * flag, the second waits for that flag (a wait only ever for a workgroup already past its K
 * loop), adds the partial sums and runs the epilogue.  The result does not depend on which
 * finishes first (fp32 addition is commutative).  With GEMM_KERNEL_AUTO the library currently
 * picks the split for no argument set (it measured slower than the 128 x 128 tile with its K
 * loop split inside the workgroup at every mid size tried, 1536^3 to 2048 x 2048 x 4096), so
 * gemm_run_ws with AUTO runs exactly as gemm_run and gemm_workspace_bytes reports 0; the split
 * kernel is taken when named (gemm_run_ws_kernel).
 *   workspace: DEVICE memory owned by the caller, 256-byte aligned, workspace_bytes long
 *     (gemm_workspace_bytes gives the size a call needs; NULL with 0 bytes is allowed).  It holds
 *     one 131328-byte slot per 256 x 128 output tile, tile t in slot t whatever the size of the
 *     call: the tile's counter and flag, then its fp32 partial sums.  It must be zero-filled
 *     before its first use; every call leaves each slot it used ready for the next (counter
 *     even, flag at half the counter) and touches no other slot, so it is filled once, not per
 *     call, and calls of different sizes may share it.  Calls that share a workspace must not
 *     overlap (one stream, or synchronised); overlapping calls race on it.
 * Errors as gemm_run, plus GEMM_ERR_INVALID_VALUE for a negative workspace_bytes, a NULL
 * workspace with workspace_bytes > 0, or a workspace not aligned to 256 bytes. */
GEMM_API gemm_status_t gemm_run_ws(gemm_handle_t h, void* stream, int64_t M, int64_t N,
                                   int64_t K, int transA, int transB, float alpha,
                                   const void* A, int64_t lda, float scale_a, const void* B,
                                   int64_t ldb, float scale_b, float beta, void* C, int64_t ldc,
                                   gemm_dtype_t a_type, gemm_dtype_t b_type, gemm_dtype_t c_type,
                                   uint32_t epilogue, const float* bias, void* workspace,
                                   int64_t workspace_bytes);

/* gemm_run_ws with an explicit kernel family.  GEMM_KERNEL_MFMA_256x128_SK2 takes any M, N, K
 * of fp16 / bf16 inputs that the matrix-core kernels accept, with a workspace of at least 131328
 * bytes per 256 x 128 output tile (GEMM_ERR_INVALID_VALUE otherwise).
 * GEMM_KERNEL_MFMA_256_SK (stream-K, the work-sharing of Osama et al., "Stream-K: Work-centric
 * Parallel Decomposition for Dense Matrix-Matrix Multiplication on the GPU", PPoPP 2023) takes
 * the same arguments.  With G = min(compute units, K tiles of the whole product), where
 * the product has T output tiles of 256 x 256 and KT = ceil(K / 64) K tiles each, workgroup L
 * takes K tiles [floor(L T KT / G), floor((L+1) T KT / G)) of the sequence that lists each
 * tile's K tiles in turn, and walks them one output tile (segment) at a time.  A tile that falls
 * to several workgroups is finished by the last of them to arrive, which adds the others' fp32
 * partial sums in the order of their K ranges (the same bits on every run) and runs the
 * epilogue.  AUTO does not take this family: on the shapes measured (fewer 256 x 256 tiles than
 * compute units, or a partial last round) it was not faster than the plain tiles.  Its workspace (gemm_kernel_workspace_bytes) is two 262144-
 * byte slots of partial sums per compute unit, then an [arrive, done] pair of 32-bit counters
 * per output tile, 256-byte aligned; it must be zero-filled before its first use, and every call
 * leaves the counters it used at zero, so calls of any size may share it (but not with
 * GEMM_KERNEL_MFMA_256x128_SK2, whose slots are laid out differently, without zero-filling it
 * again).  With K = 0 it runs as GEMM_KERNEL_MFMA_256.  The other families ignore the
 * workspace. */
GEMM_API gemm_status_t gemm_run_ws_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream,
                                          int64_t M, int64_t N, int64_t K, int transA,
                                          int transB, float alpha, const void* A, int64_t lda,
                                          float scale_a, const void* B, int64_t ldb,
                                          float scale_b, float beta, void* C, int64_t ldc,
                                          gemm_dtype_t a_type, gemm_dtype_t b_type,
                                          gemm_dtype_t c_type, uint32_t epilogue,
                                          const float* bias, void* workspace,
                                          int64_t workspace_bytes);

/* gemm_run_ws_kernel without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is the library's own static device array, 16 MiB +
 * 32 KiB (128 slots) per device, held from the time the library's code object loads on that
 * device until the process ends, and addressed through the handle (gemm_create takes its
 * address).  The
 * kernel that uses it, GEMM_KERNEL_MFMA_256x128_SK2, therefore takes outputs of at most 128
 * tiles of 256 x 128 (for example 2048 x 2048); a larger one returns GEMM_ERR_TOO_LARGE and
 * enqueues nothing.  AUTO and the other kernel families use no scratch and run as
 * gemm_run_kernel.  The array needs no clearing between calls (it starts zeroed and every
 * call leaves it as the next one needs it), but it is shared by every call on its device:
 * calls that overlap on one device (different streams, unsynchronised) race on it.  Errors as
 * gemm_run_ws_kernel, plus GEMM_ERR_TOO_LARGE. */
GEMM_API gemm_status_t gemm_run_noalloc(gemm_handle_t h, gemm_kernel_t kernel, void* stream,
                                        int64_t M, int64_t N, int64_t K, int transA,
                                        int transB, float alpha, const void* A, int64_t lda,
                                        float scale_a, const void* B, int64_t ldb,
                                        float scale_b, float beta, void* C, int64_t ldc,
                                        gemm_dtype_t a_type, gemm_dtype_t b_type,
                                        gemm_dtype_t c_type, uint32_t epilogue,
                                        const float* bias);

/* Workspace bytes gemm_run_ws (AUTO) would use for these arguments: 0 when it would not split
 * the K loop across workgroups, else what gemm_kernel_workspace_bytes gives for the family it
 * takes.  Negative status for invalid arguments (as gemm_check_args) or an invalid handle. */
GEMM_API int64_t gemm_workspace_bytes(gemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                      int transA, int transB, const void* A, int64_t lda,
                                      const void* B, int64_t ldb, const void* C, int64_t ldc,
                                      gemm_dtype_t a_type, gemm_dtype_t b_type,
                                      gemm_dtype_t c_type, uint32_t epilogue, const float* bias);

/* Workspace bytes gemm_run_ws_kernel needs for an M x N output with an explicit kernel family:
 * GEMM_KERNEL_MFMA_256x128_SK2 131328 per 256 x 128 output tile; GEMM_KERNEL_MFMA_256_SK
 * 2 x 262144 per compute unit of the handle's device plus 8 per 256 x 256 output tile, the
 * latter rounded up to a multiple of 256; 0 for the families that use none.
 * GEMM_ERR_INVALID_HANDLE, or GEMM_ERR_INVALID_VALUE for a negative or too large M or N. */
GEMM_API int64_t gemm_kernel_workspace_bytes(gemm_handle_t h, gemm_kernel_t kernel, int64_t M,
                                             int64_t N);

/* Block-scaled GEMM in the OCP microscaling (MX) formats: every run of 32 consecutive k of a
 * row of op(A) and of a column of op(B) shares one E8M0 scale byte e, worth 2^(e - 127)
 * (e = 255 is NaN):
 *
 *     op(A)[i][k] = A-element * 2^(sa[i * ldsa + k / 32] - 127),  0 <= i < M, 0 <= k < K
 *     op(B)[k][j] = B-element * 2^(sb[j * ldsb + k / 32] - 127),  0 <= j < N
 *     C = epi(alpha * op(A) op(B) + beta * C [+ bias])
 *
 * sa (M rows of ldsa >= K/32 bytes) and sb (N rows of ldsb >= K/32 bytes) are DEVICE pointers
 * owned by the caller; bytes past K/32 in a row are never used.  Types: A and B in
 * {E4M3, E5M2} (MXFP8, either mix), both E2M1 (MXFP4), or A and B in {E2M3, E3M2} (MXFP6,
 * either mix); C is BF16.  K must be a multiple of 32.  Errors as gemm_run, plus GEMM_ERR_INVALID_VALUE for K % 32 != 0, a NULL scale array
 * when K > 0, or ldsa / ldsb < K / 32, and GEMM_ERR_ALIAS when C overlaps a scale array.
 * Matrix-core kernels additionally need 16-byte-aligned sa and sb, ldsa and ldsb multiples of
 * 16, and fewer than 2^32 scale bytes per array; E2M1 operands need A stored M x K and B
 * stored N x K with lda, ldb multiples of 32; E2M3 / E3M2 operands need K a multiple of 128 and
 * lda, ldb multiples of 64.  Other arguments take GEMM_KERNEL_SIMT. */
GEMM_API gemm_status_t gemm_run_mx(gemm_handle_t h, void* stream, int64_t M, int64_t N,
                                   int64_t K, int transA, int transB, float alpha,
                                   const void* A, int64_t lda, const uint8_t* sa, int64_t ldsa,
                                   const void* B, int64_t ldb, const uint8_t* sb, int64_t ldsb,
                                   float beta, void* C, int64_t ldc, gemm_dtype_t a_type,
                                   gemm_dtype_t b_type, gemm_dtype_t c_type, uint32_t epilogue,
                                   const float* bias);

/* Check the arguments of gemm_run_mx without touching any device (as gemm_check_args). */
GEMM_API gemm_status_t gemm_check_args_mx(int64_t M, int64_t N, int64_t K, int transA,
                                          int transB, const void* A, int64_t lda,
                                          const uint8_t* sa, int64_t ldsa, const void* B,
                                          int64_t ldb, const uint8_t* sb, int64_t ldsb,
                                          const void* C, int64_t ldc, gemm_dtype_t a_type,
                                          gemm_dtype_t b_type, gemm_dtype_t c_type,
                                          uint32_t epilogue, const float* bias);

/* gemm_run_mx with an explicit kernel family (as gemm_run_kernel). */
GEMM_API gemm_status_t gemm_run_mx_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream,
                                          int64_t M, int64_t N, int64_t K, int transA,
                                          int transB, float alpha, const void* A, int64_t lda,
                                          const uint8_t* sa, int64_t ldsa, const void* B,
                                          int64_t ldb, const uint8_t* sb, int64_t ldsb,
                                          float beta, void* C, int64_t ldc,
                                          gemm_dtype_t a_type, gemm_dtype_t b_type,
                                          gemm_dtype_t c_type, uint32_t epilogue,
                                          const float* bias);

/* The kernel family gemm_run would use for these arguments (a gemm_kernel_t value), or a
 * negative status when the arguments are invalid.  Touches no device. */
GEMM_API int gemm_select_kernel(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int transA,
                       int transB, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, gemm_dtype_t a_type, gemm_dtype_t b_type,
                       gemm_dtype_t c_type, uint32_t epilogue, const float* bias);

/* The decomposed second pass: C = epi(C [+ bias]) in place, elementwise, for an M x N matrix of
 * type c_type (F32, F16 or BF16) with leading dimension ldc.  With epilogue = BIAS|GELU after a
 * gemm_run with epilogue NONE this is the unfused form of the fused epilogue ("Rigel",
 * abstract: the decomposed path).  Same error conventions as gemm_run; an unsupported c_type
 * returns GEMM_ERR_UNSUPPORTED. */
GEMM_API gemm_status_t gemm_bias_gelu(gemm_handle_t h, void* stream, int64_t M, int64_t N, void* C,
                             int64_t ldc, gemm_dtype_t c_type, const float* bias,
                             uint32_t epilogue);

/* Quantized weights: the matrix-vector product of decode and the matrix product of prefill
 * with dequantisation fused into the multiply-add ("X3: Metal GEMM", section 7, which names
 * these as the main workload of LLMs on the GPU without fixing a format).  The format read
 * here is affine group quantization of the weight matrix W (N x K, one row per output):
 *
 *     w[j][k] = scales[j * ldg + k / group] * q[j][k] + offsets[j * ldg + k / group]
 *     C = epi(alpha * X W^T + beta * C [+ bias])        (C is M x N, X is M x K)
 *
 * X: DEVICE pointer, M x K activations, row-major, ldx >= K, type x_type (GEMM_F16 or
 *    GEMM_BF16).  C, scales and offsets have the same type; bias (if any) is fp32[N].
 * Wq: DEVICE pointer, N rows of codes, ldw bytes apart.  bits = 8: one unsigned code per byte
 *    (ldw >= K).  bits = 4: two codes per byte along the row, code k in byte k / 2, in the low
 *    nibble when k is even (ldw >= K / 2, K even).
 * scales, offsets: DEVICE pointers, N rows of ldg >= K / group values.  group >= 1 and
 *    K % group == 0.
 * All buffers are owned by the caller; nothing is allocated.  Asynchronous on `stream`.
 * Errors: as gemm_run (C overlapping X, Wq, scales, offsets or bias is GEMM_ERR_ALIAS), plus
 * GEMM_ERR_INVALID_VALUE for bits not 4 or 8, group < 1, K % group != 0, an odd K with 4-bit
 * codes, or ldx / ldw / ldg too small; GEMM_ERR_UNSUPPORTED for an x_type other than F16 / BF16.
 * Kernel choice (AUTO): GEMM_KERNEL_QGEMV for M <= 4 when its staged activations fit 80 KiB
 * of LDS, GEMM_KERNEL_QMFMA otherwise, each when its alignment needs hold (below), else
 * GEMM_KERNEL_SIMT (one output per thread, any alignment). */
GEMM_API gemm_status_t gemm_run_q(gemm_handle_t h, void* stream, int64_t M, int64_t N,
                                  int64_t K, float alpha, const void* X, int64_t ldx,
                                  const uint8_t* Wq, int64_t ldw, int bits, int64_t group,
                                  const void* scales, const void* offsets, int64_t ldg,
                                  float beta, void* C, int64_t ldc, gemm_dtype_t x_type,
                                  uint32_t epilogue, const float* bias);

/* gemm_run_q with an explicit kernel: GEMM_KERNEL_SIMT, GEMM_KERNEL_QGEMV (needs Wq and ldw
 * 16-byte aligned and group a multiple of 32 (4-bit) or 16 (8-bit)), or GEMM_KERNEL_QMFMA
 * (needs X, Wq, C 16-byte aligned, ldx a multiple of 8, ldw a multiple of 16, ldc a multiple of
 * 4, group a multiple of 32 and K a multiple of 64; the weights are rounded to x_type once
 * dequantised, a relative 2^-9 (bf16) or 2^-12 (f16) per weight).  Any other kernel, or one
 * whose needs do not hold, returns GEMM_ERR_UNSUPPORTED. */
GEMM_API gemm_status_t gemm_run_q_kernel(gemm_handle_t h, gemm_kernel_t kernel, void* stream,
                                         int64_t M, int64_t N, int64_t K, float alpha,
                                         const void* X, int64_t ldx, const uint8_t* Wq,
                                         int64_t ldw, int bits, int64_t group,
                                         const void* scales, const void* offsets, int64_t ldg,
                                         float beta, void* C, int64_t ldc, gemm_dtype_t x_type,
                                         uint32_t epilogue, const float* bias);

/* Check the arguments of gemm_run_q without touching any device (as gemm_check_args). */
GEMM_API gemm_status_t gemm_check_args_q(int64_t M, int64_t N, int64_t K, const void* X,
                                         int64_t ldx, const uint8_t* Wq, int64_t ldw, int bits,
                                         int64_t group, const void* scales, const void* offsets,
                                         int64_t ldg, const void* C, int64_t ldc,
                                         gemm_dtype_t x_type, uint32_t epilogue,
                                         const float* bias);

/* The kernel gemm_run_q would use for these arguments, or a negative status. */
GEMM_API int gemm_select_kernel_q(gemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                  const void* X, int64_t ldx, const uint8_t* Wq, int64_t ldw,
                                  int bits, int64_t group, const void* scales,
                                  const void* offsets, int64_t ldg, const void* C, int64_t ldc,
                                  gemm_dtype_t x_type, uint32_t epilogue, const float* bias);

/* A static, human-readable name for a status code (never NULL). */
GEMM_API const char* gemm_status_string(gemm_status_t s);

/* ---- Measurement helpers (used by the benchmark; not part of the GEMM) ----
 *
 * The fractions of peak a benchmark reports depend on the shader clock the chip ran at ("Rigel"
 * (arXiv 2606.12765), section 3: clock-state effects decide its small-size results) and, for
 * bandwidth-bound work, on the bandwidth the memory really delivers ("Case Study: The Tiled
 * GEMM": a measured bandwidth roofline beside the product's numbers). */

/* Shader clock probe.  Enqueues `workgroups` (1 .. 65536) one-wave workgroups on `stream`; each
 * reads the shader-clock cycle counter and the constant-rate counter at its start and again
 * once `microseconds` (1 .. 100000) of the constant clock have passed (at most 2^16 polls), and
 * writes four uint64 to out[4 w .. 4 w + 3]: cycles at start, ticks at start, cycles at end,
 * ticks at end.  The clock in MHz is (cycles) / (ticks) * gemm_wall_clock_khz(h) / 1000.
 * `out` is a DEVICE pointer owned by the caller.  Queued right behind a timed run, it reads the
 * clock that run left the chip at.  Errors: GEMM_ERR_INVALID_HANDLE, GEMM_ERR_INVALID_VALUE (null
 * out or a count out of range), GEMM_ERR_DEVICE (no constant-rate counter rate), GEMM_ERR_LAUNCH. */
GEMM_API gemm_status_t gemm_probe_clock(gemm_handle_t h, void* stream, uint64_t* out,
                                        int workgroups, int microseconds);

/* Rate of the constant-rate counter the clock probe reads, in kHz (100000 on MI355X), or a
 * negative status for an invalid handle. */
GEMM_API int gemm_wall_clock_khz(gemm_handle_t h);

/* Bandwidth probe: streams `bytes` (a multiple of 16) from `src` with 16-byte loads, four in
 * flight per thread, and writes them to `dst` (a copy; it must not overlap src) or, with dst
 * NULL, only reads them (`sink`, a DEVICE uint32, is written only for one improbable checksum
 * and must not be NULL then).  src and dst are 16-byte-aligned DEVICE pointers owned by the
 * caller.  Asynchronous on `stream`.  Errors: GEMM_ERR_INVALID_HANDLE, GEMM_ERR_INVALID_VALUE
 * (null src, misaligned pointers, bytes <= 0 or not a multiple of 16, no sink for a read),
 * GEMM_ERR_ALIAS (dst overlaps src), GEMM_ERR_LAUNCH. */
GEMM_API gemm_status_t gemm_probe_bandwidth(gemm_handle_t h, void* stream, const void* src,
                                            void* dst, int64_t bytes, uint32_t* sink);

#ifdef __cplusplus
}
#endif

#endif /* TILED_GEMM_H */
