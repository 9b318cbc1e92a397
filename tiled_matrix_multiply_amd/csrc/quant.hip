// Quantized-weight kernels without matrix cores: the scalar kernel (any alignment, any shape)
// and the decode matrix-vector kernel, whose time is the read of the weight codes.
#include "quant.hpp"

namespace tgemm {

// ------------------------------------------------------------------------- scalar kernel --
// One output (m, j) per thread, grid-stride: w = fma(s, q, o) per code, fp32 fma into the
// accumulator, the scale and offset of each group loaded once.
template <int XT>
__global__ __launch_bounds__(256) void qsimt_kernel(QParams p) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / p.N, j = t % p.N;
    float acc = 0.0f;
    for (int k0 = 0; k0 < p.K; k0 += p.group) {
      const int64_t g = j * p.ldg + k0 / p.group;
      const float s = load_x16<XT>(p.S, g), o = load_x16<XT>(p.O, g);
      for (int k = k0; k < k0 + p.group; ++k) {
        const float w = fmaf(s, (float)q_code(p, j, k), o);
        acc = fmaf(load_x16<XT>(p.X, m * p.ldx + k), w, acc);
      }
    }
    q_store<XT>(p, m, j, acc);
  }
}

// ------------------------------------------------------------------ matrix-vector kernel --
// Decode: few activation rows (MT at most), many weight rows.  A fixed number of workgroups per
// compute unit each stage the activations once in LDS (16-byte loads when X allows them), then
// walk blocks of weight rows: each wave takes R rows of a block, and each lane the 16-byte
// chunks c = lane + 64 u of them (32 codes at 4 bits, 16 at 8 bits; a chunk never straddles a
// group because the group is a multiple of the chunk), so that a wave's load covers 1 KiB of
// consecutive code bytes.
//  * 4-bit codes: the two codes k and k+4 of each run of eight become the 16-bit pair
//    (1 + q_k/16, 1 + q_{k+4}/16) with one shift and one and-or (the activation type's
//    encoding of 1.0 with q in the top mantissa bits, exact), and v_dot2 multiplies the pair
//    with the staged activations (x_k, x_{k+4}) into an fp32 sum T.  Over a chunk,
//    sum x q = 16 (T - sum x), so the chunk adds 16 s T + (o - 16 s) sum x, with sum x staged per
//    chunk.  1.5 VALU instructions per code.
//  * 8-bit codes: each byte converts to float in one instruction (v_cvt_f32_ubyteN) and an
//    fma accumulates x q; the chunk adds s sum(x q) + o sum x.
// Scales and offsets: when a row has at most 128 groups (and the arrays allow 4-byte loads),
// one dword load per row and array brings all of them into the wave, two per lane, and each
// lane takes the value of its chunk's group from the lane that holds it (ds_bpermute); else
// every lane loads its own.  Loads are what the kernel's time goes to: the per-lane form costs
// 16 load instructions per 8 KiB of codes, the shared form 4.
// The partial sums of the 64 lanes are reduced across the wave; lane 0 applies the epilogue.
constexpr int QGEMV_WAVES = 4;
constexpr int QGEMV_ROWS = 2;   // weight rows per wave
constexpr int QGEMV_BATCH = 4;  // chunks per lane loaded before any is used
constexpr int QGEMV_WG_PER_CU = 4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int BITS>
__host__ __device__ constexpr int qchunk() { return BITS == 4 ? 32 : 16; }

// Bytes of LDS the matrix-vector kernel stages for M activation rows of length K.
__host__ __device__ inline int64_t qgemv_lds_bytes(int M, int K, int bits) {
  const int64_t per_x = bits == 4 ? 2 : 4;  // 16-bit pairs, or fp32
  return (int64_t)M * K * per_x + (int64_t)M * (K / (bits == 4 ? 32 : 16)) * 4;
}

// Pair i (0..3) of the eight 4-bit codes in d: codes i and i+4 as 1 + q/16 in the activation
// type (bf16: mantissa bits 6..3; f16: mantissa bits 9..6).
template <int XT, int I>
__device__ __forceinline__ uint32_t code_pair(uint32_t d) {
  constexpr int SH = XT == BF16 ? 3 : 6;  // position of q in each half
  constexpr uint32_t ONE = XT == BF16 ? 0x3F803F80u : 0x3C003C00u;
  constexpr uint32_t MASK = 0x000F000Fu << SH;
  constexpr int MOVE = 4 * I - SH;  // right shift taking nibble I to bit SH
  const uint32_t v = MOVE >= 0 ? (d >> MOVE) : (d << -MOVE);
  return (v & MASK) | ONE;
}

template <int XT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (XT == BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
}

template <int XT, int BITS, int MT, bool SHARED_SO>
__global__ __launch_bounds__(64 * QGEMV_WAVES) void qgemv_kernel(QParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t qsm[];
  constexpr int CH = qchunk<BITS>();
  const int M = p.M, K = p.K, NCH = K / CH;
  constexpr int XB = BITS == 4 ? 2 : 4;
  uint8_t* const xs = qsm;
  float* const csum = reinterpret_cast<float*>(qsm + (size_t)M * K * XB);

  // Stage: one chunk of one activation row per thread and step; the chunk's sum in k order.
  const bool xvec = ((reinterpret_cast<uintptr_t>(p.X) | (uintptr_t)(p.ldx * 2)) & 15u) == 0;
  for (int u = threadIdx.x; u < M * NCH; u += 64 * QGEMV_WAVES) {
    const int m = u / NCH, c = u % NCH;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(p.X) + (int64_t)m * p.ldx + c * CH;
    float sum = 0.0f;
#pragma unroll
    for (int e8 = 0; e8 < CH; e8 += 8) {
      uint32_t h[8];
      if (xvec) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + e8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = v[e] & 0xffffu;
          h[2 * e + 1] = v[e] >> 16;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = src[e8 + e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += x16_to_float<XT>(h[e]);
      if constexpr (BITS == 4) {
        *reinterpret_cast<u32x4_t*>(xs + ((size_t)m * K + c * CH + e8) * 2) =
            u32x4_t{h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16)};
      } else {
        float* d = reinterpret_cast<float*>(xs + ((size_t)m * K + c * CH + e8) * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = x16_to_float<XT>(h[e]);
      }
    }
    csum[m * NCH + c] = sum;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int ROWS_PER_BLOCK = QGEMV_WAVES * QGEMV_ROWS;
  const int ngroups = K / p.group;
  for (int64_t jb = blockIdx.x; jb * ROWS_PER_BLOCK < p.N; jb += gridDim.x) {
    const int64_t j0 = (jb * QGEMV_WAVES + wave) * QGEMV_ROWS;
    float acc[QGEMV_ROWS][MT];
#pragma unroll
    for (int r = 0; r < QGEMV_ROWS; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    // Every load below is unconditional (lanes past the end read a valid clamped address and
    // mask the value), so that the compiler issues them back to back: a load under a branch is
    // followed by a full wait, which would leave one load in flight per wave.
    // The group words of each row, two 16-bit values per lane (shared form).
    uint32_t sw[QGEMV_ROWS], ow[QGEMV_ROWS];
    if constexpr (SHARED_SO) {
#pragma unroll
      for (int r = 0; r < QGEMV_ROWS; ++r) {
        const bool ok = j0 + r < p.N && 2 * lane < ngroups;
        const int64_t w = ok ? ((j0 + r) * p.ldg) / 2 + lane : 0;
        const uint32_t s2 = reinterpret_cast<const uint32_t*>(p.S)[w];
        const uint32_t o2 = reinterpret_cast<const uint32_t*>(p.O)[w];
        sw[r] = ok ? s2 : 0u;
        ow[r] = ok ? o2 : 0u;
      }
    }
    for (int cb = lane; cb < NCH; cb += 64 * QGEMV_BATCH) {
      u32x4_t wv[QGEMV_ROWS][QGEMV_BATCH];
      float sv[QGEMV_ROWS][QGEMV_BATCH], ov[QGEMV_ROWS][QGEMV_BATCH];
#pragma unroll
      for (int r = 0; r < QGEMV_ROWS; ++r)
#pragma unroll
        for (int b = 0; b < QGEMV_BATCH; ++b) {
          const int c = cb + 64 * b;
          const int64_t j = j0 + r;
          const bool ok = c < NCH && j < p.N;
          const int64_t jc = ok ? j : 0, cc = ok ? c : 0;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p.W + jc * p.ldw + cc * 16);
          wv[r][b] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
          const int gi = (int)(cc * CH / p.group);  // group of the chunk
          float sf, of;
          if constexpr (SHARED_SO) {
            const int src = (gi >> 1) & 63, sh = 16 * (gi & 1);
            sf = x16_to_float<XT>(((uint32_t)__shfl((int)sw[r], src, 64) >> sh) & 0xffffu);
            of = x16_to_float<XT>(((uint32_t)__shfl((int)ow[r], src, 64) >> sh) & 0xffffu);
          } else {
            const int64_t g = jc * p.ldg + gi;
            sf = load_x16<XT>(p.S, g);
            of = load_x16<XT>(p.O, g);
          }
          sv[r][b] = ok ? sf : 0.0f;
          ov[r][b] = ok ? of : 0.0f;
        }
#pragma unroll
      for (int b = 0; b < QGEMV_BATCH; ++b) {
        const int c = cb + 64 * b;
        const int cc = c < NCH ? c : 0;  // masked chunks carry zero scale and offset
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m >= M) break;  // uniform
          const float xsum = csum[m * NCH + cc];
          if constexpr (BITS == 4) {
            u32x4_t xv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              xv[i] = *reinterpret_cast<const u32x4_t*>(xs + ((size_t)m * K + cc * CH + 8 * i) * 2);
#pragma unroll
            for (int r = 0; r < QGEMV_ROWS; ++r) {
              float t = 0.0f;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t d = wv[r][b][i];
                t = dot2<XT>(code_pair<XT, 0>(d), xv[i][0], t);
                t = dot2<XT>(code_pair<XT, 1>(d), xv[i][1], t);
                t = dot2<XT>(code_pair<XT, 2>(d), xv[i][2], t);
                t = dot2<XT>(code_pair<XT, 3>(d), xv[i][3], t);
              }
              const float s16 = 16.0f * sv[r][b];
              acc[r][m] = fmaf(s16, t, acc[r][m]);
              acc[r][m] = fmaf(ov[r][b] - s16, xsum, acc[r][m]);
            }
          } else {
            float xv[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 f = *reinterpret_cast<const float4*>(xs + ((size_t)m * K + cc * CH + 4 * i) * 4);
              xv[4 * i] = f.x; xv[4 * i + 1] = f.y; xv[4 * i + 2] = f.z; xv[4 * i + 3] = f.w;
            }
#pragma unroll
            for (int r = 0; r < QGEMV_ROWS; ++r) {
              float t = 0.0f;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t d = wv[r][b][i];
#pragma unroll
                for (int e = 0; e < 4; ++e) t = fmaf(xv[4 * i + e], (float)((d >> (8 * e)) & 255u), t);
              }
              acc[r][m] = fmaf(sv[r][b], t, acc[r][m]);
              acc[r][m] = fmaf(ov[r][b], xsum, acc[r][m]);
            }
          }
        }
      }
    }
    // Reduce over the wave, then lane 0 stores.
#pragma unroll
    for (int r = 0; r < QGEMV_ROWS; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[r][m] += __shfl_xor(acc[r][m], off, 64);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < QGEMV_ROWS; ++r) {
        const int64_t j = j0 + r;
        if (j >= p.N) break;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m >= M) break;
          q_store<XT>(p, m, j, acc[r][m]);
        }
      }
    }
  }  // row blocks
}

template <int XT>
hipError_t launch_qsimt_t(const QParams& p, int cu_count, hipStream_t s) {
  const int64_t total = (int64_t)p.M * p.N;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < (int64_t)cu_count * 32 ? blocks : (int64_t)cu_count * 32);
  hipLaunchKernelGGL((qsimt_kernel<XT>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_qsimt(const QParams& p, int x_type, int cu_count, hipStream_t s) {
  return x_type == BF16 ? launch_qsimt_t<BF16>(p, cu_count, s) : launch_qsimt_t<F16>(p, cu_count, s);
}

// Scales and offsets can be shared across the wave (see the kernel) when a row has at most 128
// groups and both arrays allow 4-byte loads.
inline bool qgemv_shared_so(const QParams& p) {
  return p.K / p.group <= 128 && (p.ldg & 1) == 0 &&
         ((reinterpret_cast<uintptr_t>(p.S) | reinterpret_cast<uintptr_t>(p.O)) & 3u) == 0;
}

template <int XT, int BITS, int MT>
hipError_t launch_qgemv_t(const QParams& p, int cu_count, hipStream_t s) {
  const int64_t rows_per_wg = (int64_t)QGEMV_WAVES * QGEMV_ROWS;
  const int64_t blocks = (p.N + rows_per_wg - 1) / rows_per_wg;
  const int64_t cap = (int64_t)cu_count * QGEMV_WG_PER_CU;
  const unsigned grid = (unsigned)(blocks < cap ? blocks : cap);
  const size_t lds = (size_t)qgemv_lds_bytes(p.M, p.K, BITS);
  if (qgemv_shared_so(p))
    hipLaunchKernelGGL((qgemv_kernel<XT, BITS, MT, true>), dim3(grid), dim3(64 * QGEMV_WAVES), lds, s, p);
  else
    hipLaunchKernelGGL((qgemv_kernel<XT, BITS, MT, false>), dim3(grid), dim3(64 * QGEMV_WAVES), lds, s, p);
  return hipGetLastError();
}

template <int XT, int BITS>
hipError_t launch_qgemv_b(const QParams& p, int cu_count, hipStream_t s) {
  if (p.M <= 1) return launch_qgemv_t<XT, BITS, 1>(p, cu_count, s);
  if (p.M <= 2) return launch_qgemv_t<XT, BITS, 2>(p, cu_count, s);
  return launch_qgemv_t<XT, BITS, 4>(p, cu_count, s);
}

// The host has checked: 1 <= M <= 4, LDS need <= 64 KiB, alignment and group divisibility.
hipError_t launch_qgemv(const QParams& p, int x_type, int cu_count, hipStream_t s) {
  if (x_type == BF16)
    return p.bits == 4 ? launch_qgemv_b<BF16, 4>(p, cu_count, s) : launch_qgemv_b<BF16, 8>(p, cu_count, s);
  return p.bits == 4 ? launch_qgemv_b<F16, 4>(p, cu_count, s) : launch_qgemv_b<F16, 8>(p, cu_count, s);
}

}  // namespace tgemm
