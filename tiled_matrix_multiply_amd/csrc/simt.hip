// LDS-tiled scalar-FMA GEMM: the plain tiled kernel without matrix cores.
//
// "X3: Metal GEMM, from threadgroup tiling to simdgroup_matrix", section 2 (matmul_tiled):
// a 16x16 tile of threads, one output per thread, each K step stages a 16x16 slice of op(A)
// and op(B) with zeros beyond the matrix edges, then two barriers (all written before any
// read, all read before any overwrite).  Section 2 also pads the dispatch so every tile is
// complete because a barrier needs every thread; here every thread of a workgroup reaches
// both barriers and only the final store is masked.
//
// It serves as the library's fallback for any layout and alignment, and as the no-matrix-core
// baseline the matrix-core kernels are measured against.  Inputs of every type are decoded to
// fp32 while staging (with their E8M0 block scale when the call is block-scaled); products are
// accumulated with fp32 FMA.
#include "common.hpp"

namespace tgemm {

constexpr int TS = 16;

template <int AT, int BT, int CT>
__global__ __launch_bounds__(TS * TS) void gemm_simt_kernel(GemmParams p, int transA, int transB) {
  __shared__ float As[TS][TS + 1];
  __shared__ float Bs[TS][TS + 1];
  const int tx = threadIdx.x % TS, ty = threadIdx.x / TS;
  const int row = blockIdx.y * TS + ty;  // output row (M)
  const int col = blockIdx.x * TS + tx;  // output column (N)
  float acc = 0.0f;
  for (int k0 = 0; k0 < p.K; k0 += TS) {
    // op(A)[row, k0 + tx] and op(B)[k0 + ty, col], zero outside the matrices.
    const int ka = k0 + tx, kb = k0 + ty;
    float a = 0.0f, b = 0.0f;
    if (row < p.M && ka < p.K) {
      a = load_as_float<AT>(p.A, transA ? (int64_t)ka * p.lda + row : (int64_t)row * p.lda + ka);
      if (p.sa) a *= e8m0_to_float(p.sa[(int64_t)row * p.ldsa + (ka >> 5)]);
    }
    if (kb < p.K && col < p.N) {
      b = load_as_float<BT>(p.B, transB ? (int64_t)col * p.ldb + kb : (int64_t)kb * p.ldb + col);
      if (p.sb) b *= e8m0_to_float(p.sb[(int64_t)col * p.ldsb + (kb >> 5)]);
    }
    As[ty][tx] = a;
    Bs[ty][tx] = b;
    __syncthreads();  // every element written before any is read
#pragma unroll
    for (int k = 0; k < TS; ++k) acc = fmaf(As[ty][k], Bs[k][tx], acc);
    __syncthreads();  // every element read before the next step overwrites it
  }
  if (row < p.M && col < p.N) {
    const int64_t idx = (int64_t)row * p.ldc + col;
    const float cin = p.beta != 0.0f ? load_as_float<CT>(p.C, idx) : 0.0f;
    const float bj = (p.epi & EPI_BIAS) ? p.bias[col] : 0.0f;
    store_from_float<CT>(p.C, idx, epilogue_value<CT>(acc, p.alpha, p.beta, cin, bj, p.epi));
  }
}

template <int AT, int BT, int CT>
static hipError_t launch(const GemmParams& p, int transA, int transB, hipStream_t s) {
  dim3 grid((p.N + TS - 1) / TS, (p.M + TS - 1) / TS);
  hipLaunchKernelGGL((gemm_simt_kernel<AT, BT, CT>), grid, dim3(TS * TS), 0, s, p, transA, transB);
  return hipGetLastError();
}

// Launch for a supported (A type, C type) pair.  Grid: one 16x16 workgroup per output tile,
// counted in workgroups (not threads); y indexes tile rows, x tile columns.
hipError_t launch_simt(const GemmParams& p, int a_type, int b_type, int transA, int transB,
                       hipStream_t s) {
  if (p.M > 65535 * TS) return hipErrorInvalidValue;  // grid.y limit
  const int pair = a_type * 8 + b_type;
  switch (pair) {
    case F32 * 8 + F32: return launch<F32, F32, F32>(p, transA, transB, s);
    case F16 * 8 + F16: return launch<F16, F16, F16>(p, transA, transB, s);
    case BF16 * 8 + BF16: return launch<BF16, BF16, BF16>(p, transA, transB, s);
    case E4M3 * 8 + E4M3: return launch<E4M3, E4M3, BF16>(p, transA, transB, s);
    case E4M3 * 8 + E5M2: return launch<E4M3, E5M2, BF16>(p, transA, transB, s);
    case E5M2 * 8 + E4M3: return launch<E5M2, E4M3, BF16>(p, transA, transB, s);
    case E5M2 * 8 + E5M2: return launch<E5M2, E5M2, BF16>(p, transA, transB, s);
    case E2M1 * 8 + E2M1: return launch<E2M1, E2M1, BF16>(p, transA, transB, s);
    case E2M3 * 8 + E2M3: return launch<E2M3, E2M3, BF16>(p, transA, transB, s);
    case E2M3 * 8 + E3M2: return launch<E2M3, E3M2, BF16>(p, transA, transB, s);
    case E3M2 * 8 + E2M3: return launch<E3M2, E2M3, BF16>(p, transA, transB, s);
    case E3M2 * 8 + E3M2: return launch<E3M2, E3M2, BF16>(p, transA, transB, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tgemm
