// Register-blocked scalar-FMA GEMM without matrix cores: the library's fallback for any layout,
// alignment and size, and the no-matrix-core baseline the matrix-core kernels are measured
// against.
//
// It keeps the tiling idea of "X3: Metal GEMM, from threadgroup tiling to simdgroup_matrix",
// section 2: a workgroup owns a tile of C and stages the K slices of op(A) and op(B) that tile
// needs in shared memory, with zeros beyond the matrix edges.  The layout is its own:
//  * 256 threads own a 64 x 64 tile of C; thread (tx, ty) of the 16 x 16 arrangement keeps the
//    4 x 4 register block of rows ty + 16 i and columns tx + 16 j, so every value read from
//    LDS feeds four FMAs;
//  * K is walked in slices of 16, double-buffered: the next slice's global loads are issued
//    into registers before the current slice is multiplied, written to the other LDS buffer
//    afterwards, and one barrier per slice separates the two (a buffer is rewritten only after
//    every thread has passed the barrier that follows its last read);
//  * a workgroup walks tiles with a stride of the grid over a 64-bit tile index (column tiles
//    fastest, so workgroups running together share rows of op(A)), so any M and N up to
//    2^31 - 1 fit a one-dimensional grid of at most kMaxGrid workgroups;
//  * inputs of every type are decoded to fp32 as they are staged (times their E8M0 block scale
//    when the call is block-scaled) and products accumulate with fp32 FMA; the epilogue is the
//    library's, with a masked store per element.
#include "common.hpp"

namespace tgemm {

namespace {

constexpr int kTile = 64, kSlice = 16, kThreads = 256;
constexpr int kPad = kTile + 4;  // LDS row stride: the staging writes along k avoid one bank
constexpr int64_t kMaxGrid = int64_t(1) << 20;

template <int AT, int BT, int CT>
__global__ __launch_bounds__(kThreads) void gemm_simt_kernel(GemmParams p, int transA, int transB) {
  __shared__ float As[2][kSlice][kPad];  // As[buf][k][m]
  __shared__ float Bs[2][kSlice][kPad];  // Bs[buf][k][n]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t tiles_n = (p.N + kTile - 1) / kTile;
  const int64_t T = (int64_t)((p.M + kTile - 1) / kTile) * tiles_n;
  const int slices = (p.K + kSlice - 1) / kSlice;

  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int64_t m0 = (t / tiles_n) * kTile, n0 = (t % tiles_n) * kTile;

    // Element q of this thread's share of a slice: its (m or n, k) inside the slice.  The
    // mapping follows the storage order so that neighbouring lanes read neighbouring addresses.
    float ra[4], rb[4];
    auto fetch = [&](int s) {
      const int k0 = s * kSlice;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + kThreads * q;
        int m, k;
        if (transA) { m = e & 63; k = e >> 6; }   // A stored K x M: contiguous along m
        else        { m = e >> 4; k = e & 15; }   // A stored M x K: contiguous along k
        const int64_t gm = m0 + m;
        const int gk = k0 + k;
        float v = 0.0f;
        if (gm < p.M && gk < p.K) {
          v = load_as_float<AT>(p.A, transA ? (int64_t)gk * p.lda + gm : gm * p.lda + gk);
          if (p.sa) v *= e8m0_to_float(p.sa[gm * p.ldsa + (gk >> 5)]);
        }
        ra[q] = v;
        int n, kb;
        if (transB) { n = e >> 4; kb = e & 15; }  // B stored N x K: contiguous along k
        else        { n = e & 63; kb = e >> 6; }  // B stored K x N: contiguous along n
        const int64_t gn = n0 + n;
        const int gkb = k0 + kb;
        float w = 0.0f;
        if (gn < p.N && gkb < p.K) {
          w = load_as_float<BT>(p.B, transB ? gn * p.ldb + gkb : (int64_t)gkb * p.ldb + gn);
          if (p.sb) w *= e8m0_to_float(p.sb[gn * p.ldsb + (gkb >> 5)]);
        }
        rb[q] = w;
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + kThreads * q;
        if (transA) As[buf][e >> 6][e & 63] = ra[q];
        else        As[buf][e & 15][e >> 4] = ra[q];
        if (transB) Bs[buf][e & 15][e >> 4] = rb[q];
        else        Bs[buf][e >> 6][e & 63] = rb[q];
      }
    };

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    if (slices > 0) {
      fetch(0);
      stash(0);
      __syncthreads();
    }
    for (int s = 0; s < slices; ++s) {
      const int buf = s & 1;
      if (s + 1 < slices) fetch(s + 1);
      // four k per unrolled step: enough LDS reads in flight without holding a whole slice's
#pragma unroll 4
      for (int k = 0; k < kSlice; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[buf][k][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[buf][k][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      if (s + 1 < slices) stash(buf ^ 1);
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + ty + 16 * i;
      if (row >= p.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + tx + 16 * j;
        if (col >= p.N) continue;
        const int64_t idx = row * p.ldc + col;
        const float cin = p.beta != 0.0f ? load_as_float<CT>(p.C, idx) : 0.0f;
        const float bj = (p.epi & EPI_BIAS) ? p.bias[col] : 0.0f;
        store_from_float<CT>(p.C, idx, epilogue_value<CT>(acc[i][j], p.alpha, p.beta, cin, bj, p.epi));
      }
    }
  }
}

template <int AT, int BT, int CT>
hipError_t launch(const GemmParams& p, int transA, int transB, hipStream_t s) {
  const int64_t T = ((int64_t)(p.M + kTile - 1) / kTile) * ((p.N + kTile - 1) / kTile);
  const unsigned grid = (unsigned)(T < kMaxGrid ? T : kMaxGrid);
  hipLaunchKernelGGL((gemm_simt_kernel<AT, BT, CT>), dim3(grid), dim3(kThreads), 0, s, p, transA,
                     transB);
  return hipGetLastError();
}

}  // namespace

// Launch for a supported (A type, B type) pair (the output type follows: the input type for
// 16- and 32-bit inputs, bf16 for the 8-, 6- and 4-bit ones).  One-dimensional grid counted in
// workgroups (not threads), min(tiles, kMaxGrid), each workgroup striding over the tiles.
hipError_t launch_simt(const GemmParams& p, int a_type, int b_type, int transA, int transB,
                       hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
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
