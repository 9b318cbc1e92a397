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
// walk blocks of weight rows: each wave takes R rows of a block, in ncb units of B 16-byte
// chunks per lane and row (unit t takes chunks c = lane + 64 (t + ncb b), b < B: each load
// instruction of a wave covers 1 KiB of consecutive code bytes, and a unit spreads over the
// whole row; a chunk holds 32 codes at 4 bits, 16 at 8 bits, and never straddles a group
// because the group is a multiple of the chunk).
//  * 4-bit codes: the two codes k and k+4 of each run of eight become one 16-bit pair in the
//    activation type, each half an exact value e(q) = B0 + q / Q (see code_pairs), and v_dot2
//    multiplies the pair with the staged activations (x_k, x_{k+4}) into an fp32 sum T.  Over a
//    chunk, sum x q = Q (T - B0 sum x), so the chunk adds Q s T + (o - Q B0 s) sum x, with sum x
//    staged per chunk.  Per 32-bit word of eight codes: three instructions split the even and
//    the odd nibbles into bytes, four byte permutes build the pairs, four v_dot2 (11 VALU
//    instructions, 1.375 per code).
//  * 8-bit codes: each byte converts to float in one instruction (v_cvt_f32_ubyteN) and an
//    fma accumulates x q; the chunk adds s sum(x q) + o sum x.
// Scales and offsets: when a row has at most 128 groups (an even number, and the arrays allow
// 4-byte loads), one dword load per row and array brings all of them into the wave, two per
// lane, and each lane takes the value of its chunk's group from the lane that holds it
// (ds_bpermute); else every lane loads its own.
// Software pipeline: a wave requests its next unit (codes, scales and offsets, and the
// epilogue's operands) before it converts the current one, into the other of two register sets,
// and its first unit before the activations are staged.  Nothing between two units waits for
// all loads: the conversion work overlaps the wave's own reads, not only other waves'.
// The partial sums of the 64 lanes are reduced across the wave (DPP); lane 0 applies the
// epilogue.
constexpr int QGEMV_WAVES = 4;
constexpr int QGEMV_ROWS = 2;   // weight rows per wave
constexpr int QGEMV_BATCH = 2;  // chunks per lane and row in one unit
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

// The eight 4-bit codes of d (code i in bits 4i..4i+3) as four 16-bit pairs in the activation
// type: out[i] holds codes i and i+4.  Each half is one code byte under a constant exponent byte
// (one v_perm_b32 per pair, after the nibbles are spread over bytes):
//   bf16: 0x3F00 | q         = 1/2 + q/256   (q in mantissa bits 3..0)
//   f16:  0x3C00 | (q << 4)  = 1 + q/64      (q in mantissa bits 7..4)
// so e(q) = B0 + q/Q with (B0, Q) = (1/2, 256) or (1, 64), both exact.
template <int XT>
struct QPair {
  static constexpr float Q = XT == BF16 ? 256.0f : 64.0f;
  static constexpr float QB0 = XT == BF16 ? 128.0f : 64.0f;  // Q * B0
};

template <int XT>
__device__ __forceinline__ void code_pairs(uint32_t d, uint32_t hi, uint32_t (&out)[4]) {
  uint32_t ev, od;  // codes 0, 2, 4, 6 and codes 1, 3, 5, 7, one per byte
  if constexpr (XT == BF16) {
    ev = d & 0x0F0F0F0Fu;
    od = (d >> 4) & 0x0F0F0F0Fu;
  } else {
    ev = (d << 4) & 0xF0F0F0F0u;
    od = d & 0xF0F0F0F0u;
  }
  // v_perm_b32(s0, s1, sel): selector bytes 4..7 take bytes 0..3 of s0, 0..3 those of s1.
  // hi holds the exponent byte in every byte.
  out[0] = __builtin_amdgcn_perm(ev, hi, 0x00060004u);  // codes 0, 4
  out[1] = __builtin_amdgcn_perm(od, hi, 0x00060004u);  // codes 1, 5
  out[2] = __builtin_amdgcn_perm(ev, hi, 0x00070005u);  // codes 2, 6
  out[3] = __builtin_amdgcn_perm(od, hi, 0x00070005u);  // codes 3, 7
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

// Sum over the 64 lanes of a wave (all active), the result in every lane: lane pairs, quads,
// rows of 8 and of 16 through DPP moves (no LDS round trip), then the four row sums read as
// scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

template <int XT, int BITS, int MT, bool SHARED_SO>
__global__ __launch_bounds__(64 * QGEMV_WAVES, MT == 1 ? QGEMV_WG_PER_CU : 1) void qgemv_kernel(QParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t qsm[];
  constexpr int CH = qchunk<BITS>();
  constexpr int R = QGEMV_ROWS, B = QGEMV_BATCH;
  const int M = p.M, K = p.K, NCH = K / CH;
  constexpr int XB = BITS == 4 ? 2 : 4;
  uint8_t* const xs = qsm;
  float* const csum = reinterpret_cast<float*>(qsm + (size_t)M * K * XB);
  // The wave index is uniform: kept scalar, so that row addresses are too.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ngroups = K / p.group;
  // The exponent byte of the code pairs, kept in a vector register: v_perm_b32 takes one scalar
  // operand, and its selector is the other.
  uint32_t hi = XT == BF16 ? 0x3F3F3F3Fu : 0x3C3C3C3Cu;
  asm volatile("" : "+v"(hi));

  // A wave's work is a sequence of units (jb, t): batch t < ncb of the chunks of row block jb,
  // for jb = blockIdx.x, blockIdx.x + gridDim.x, ... < nblk (the host launches at most one
  // workgroup per block).
  const int ncb = (NCH + 64 * B - 1) / (64 * B);
  constexpr int ROWS_PER_BLOCK = QGEMV_WAVES * R;
  const int64_t nblk = (p.N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  const int64_t grid = gridDim.x;
  const int64_t nunits = ((nblk - blockIdx.x + grid - 1) / grid) * ncb;  // per wave
  struct Cursor {
    int64_t jb;
    int t;
  };
  auto advance = [&](Cursor c) {
    return c.t + 1 < ncb ? Cursor{c.jb, c.t + 1} : Cursor{c.jb + grid, 0};
  };

  // The raw data of one unit: B 16-byte chunks of each of the wave's R rows and, in the shared
  // form, the scale and offset words of those rows.
  struct Unit {
    u32x4_t w[R][B];
    uint32_t sw[R], ow[R];        // shared form: two groups' values per lane
    uint32_t so[R][B];            // else: the chunk's own scale (low half) and offset
    uint32_t cin[R][MT];          // the 16-bit C_in words of the rows' outputs
    float bias[R];
  };
  // Every load is unconditional: lanes past the end read a valid clamped address and the value
  // is masked at use, so that the compiler issues the loads back to back (a load under a branch
  // is followed by a full wait, which would leave one load in flight per wave).
  // The epilogue's operands come with the unit (the same address in every lane), so that the
  // store needs no load and no wait: a wait there would also wait for the next unit's codes.
  // When there is no bias, the bias load reads the codes instead (4 N bytes of them at least);
  // C_in is read even when beta = 0 (C is the output, so the address is valid) and not used.
  const float* const biasp = (p.epi & EPI_BIAS) ? p.bias : reinterpret_cast<const float*>(p.W);
  auto load = [&](Cursor u, Unit& d) {
    const int cb = lane + 64 * u.t;
    const int64_t j0 = (u.jb * QGEMV_WAVES + wave) * R;
    // The small operands first: a wait for them is then a wait for the oldest loads only.
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t jc = j0 + r < p.N ? j0 + r : p.N - 1;
      d.bias[r] = biasp[jc];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        d.cin[r][m] = reinterpret_cast<const uint16_t*>(p.C)[(int64_t)(m < M ? m : 0) * p.ldc + jc];
      if constexpr (SHARED_SO) {
        const int64_t wi = (jc * p.ldg) / 2 + (2 * lane < ngroups ? lane : 0);
        d.sw[r] = reinterpret_cast<const uint32_t*>(p.S)[wi];
        d.ow[r] = reinterpret_cast<const uint32_t*>(p.O)[wi];
      } else {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int c = cb + 64 * ncb * b;
          const int64_t gi = jc * p.ldg + (int64_t)(c < NCH ? c : NCH - 1) * CH / p.group;
          d.so[r][b] = (uint32_t)reinterpret_cast<const uint16_t*>(p.S)[gi] |
                       ((uint32_t)reinterpret_cast<const uint16_t*>(p.O)[gi] << 16);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t jc = j0 + r < p.N ? j0 + r : p.N - 1;
      const uint8_t* const row = p.W + jc * p.ldw;  // uniform
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int c = cb + 64 * ncb * b;
        const uint32_t off = (uint32_t)(c < NCH ? c : NCH - 1) * 16u;
        d.w[r][b] = *reinterpret_cast<const u32x4_t*>(row + off);
      }
    }
  };

  float acc[R][MT];
  auto compute = [&](Cursor u, const Unit& d) {
    const int t = u.t;
    const int cb = lane + 64 * t;
    const int64_t j0 = (u.jb * QGEMV_WAVES + wave) * R;
    if (t == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = cb + 64 * ncb * b;
      const bool cok = c < NCH;
      const int cc = cok ? c : NCH - 1;
      const int gi = (int)((int64_t)cc * CH / p.group);  // group of the chunk
      float sv[R], ov[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool ok = cok && j0 + r < p.N;  // masked chunks carry zero scale and offset
        float sf, of;
        if constexpr (SHARED_SO) {
          const int src = (gi >> 1) & 63, sh = 16 * (gi & 1);
          sf = x16_to_float<XT>(((uint32_t)__shfl((int)d.sw[r], src, 64) >> sh) & 0xffffu);
          of = x16_to_float<XT>(((uint32_t)__shfl((int)d.ow[r], src, 64) >> sh) & 0xffffu);
        } else {
          sf = x16_to_float<XT>(d.so[r][b] & 0xffffu);
          of = x16_to_float<XT>(d.so[r][b] >> 16);
        }
        sv[r] = ok ? sf : 0.0f;
        ov[r] = ok ? of : 0.0f;
      }
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
          for (int r = 0; r < R; ++r) {
            float tt = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t pr[4];
              code_pairs<XT>(d.w[r][b][i], hi, pr);
#pragma unroll
              for (int e = 0; e < 4; ++e) tt = dot2<XT>(pr[e], xv[i][e], tt);
            }
            acc[r][m] = fmaf(QPair<XT>::Q * sv[r], tt, acc[r][m]);
            acc[r][m] = fmaf(fmaf(-QPair<XT>::QB0, sv[r], ov[r]), xsum, acc[r][m]);
          }
        } else {
          float xv[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 f = *reinterpret_cast<const float4*>(xs + ((size_t)m * K + cc * CH + 4 * i) * 4);
            xv[4 * i] = f.x; xv[4 * i + 1] = f.y; xv[4 * i + 2] = f.z; xv[4 * i + 3] = f.w;
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float tt = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t w = d.w[r][b][i];
#pragma unroll
              for (int e = 0; e < 4; ++e) tt = fmaf(xv[4 * i + e], (float)((w >> (8 * e)) & 255u), tt);
            }
            acc[r][m] = fmaf(sv[r], tt, acc[r][m]);
            acc[r][m] = fmaf(ov[r], xsum, acc[r][m]);
          }
        }
      }
    }
    if (t == ncb - 1) {
      // Reduce over the wave, then lane 0 stores.
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t j = j0 + r;
          if (j >= p.N) break;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m >= M) break;
            const float cin = x16_to_float<XT>(d.cin[r][m]);
            store_from_float<XT>(p.C, (int64_t)m * p.ldc + j,
                                 epilogue_value<XT>(acc[r][m], p.alpha, p.beta, cin, d.bias[r], p.epi));
          }
        }
      }
    }
  };

  // The first unit's codes are requested before the activations are staged, and every later
  // unit's before the previous one is computed (two register sets, used in turn).
  Unit ua, ub;
  load(Cursor{blockIdx.x, 0}, ua);

  // Stage: one chunk of one activation row per thread and step; the chunk's sum in k order.
  const bool xvec = ((reinterpret_cast<uintptr_t>(p.X) | (uintptr_t)(p.ldx * 2)) & 15u) == 0;
  for (int u = threadIdx.x; u < M * NCH; u += 64 * QGEMV_WAVES) {
    const int m = u / NCH, c = u % NCH;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(p.X) + (int64_t)m * p.ldx + c * CH;
    // Every load of the chunk is issued before any value is used.
    uint32_t hv[CH];
    if (xvec) {
#pragma unroll
      for (int e8 = 0; e8 < CH; e8 += 8) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + e8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[e8 + 2 * e] = v[e] & 0xffffu;
          hv[e8 + 2 * e + 1] = v[e] >> 16;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < CH; ++e) hv[e] = src[e];
    }
    float sum = 0.0f;
#pragma unroll
    for (int e8 = 0; e8 < CH; e8 += 8) {
      const uint32_t* h = hv + e8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += x16_to_float<XT>(h[e]);
      if constexpr (BITS == 4) {
        *reinterpret_cast<u32x4_t*>(xs + ((size_t)m * K + c * CH + e8) * 2) =
            u32x4_t{h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16)};
      } else {
        float* dst = reinterpret_cast<float*>(xs + ((size_t)m * K + c * CH + e8) * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = x16_to_float<XT>(h[e]);
      }
    }
    csum[m * NCH + c] = sum;
  }
  __syncthreads();

  // The request past the end repeats the current unit (cache-resident), so that no load is
  // conditional.
  // Units are taken in pairs; the loop's only exit is its test, so that the compiler's wait at
  // the loop head does not count loads that only a mid-loop exit leaves in flight (it would
  // wait for all of them).  When two units are left, the request for the unit after them
  // repeats the second (cache-resident), so that no load is conditional.  The scheduling
  // barriers keep every load of the next unit ahead of the current unit's first use of its data.
  Cursor u0{blockIdx.x, 0};
  for (int64_t left = nunits; left >= 2; left -= 2) {
    const Cursor u1 = advance(u0);
    load(u1, ub);
    __builtin_amdgcn_sched_barrier(0);
    compute(u0, ua);
    const Cursor u2 = left >= 3 ? advance(u1) : u1;
    load(u2, ua);
    __builtin_amdgcn_sched_barrier(0);
    compute(u1, ub);
    u0 = u2;
  }
  if (nunits & 1) compute(u0, ua);
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
// groups, an even number of them (a dword load never reaches past a row's last group), and both
// arrays allow 4-byte loads.
inline bool qgemv_shared_so(const QParams& p) {
  return p.K / p.group <= 128 && ((p.K / p.group) & 1) == 0 && (p.ldg & 1) == 0 &&
         ((reinterpret_cast<uintptr_t>(p.S) | reinterpret_cast<uintptr_t>(p.O)) & 3u) == 0;
}

// One launch of the persistent matrix-vector kernel: as many workgroups per compute unit as
// are resident at once (registers and LDS decide it: the runtime's occupancy query, at most
// QGEMV_WG_PER_CU), so that no workgroup waits for a slot and the row blocks are shared evenly.
// More than 64 KiB of dynamic LDS (four activation rows of K = 8192) is declared first.
template <class Kernel>
hipError_t launch_qgemv_kernel(Kernel kernel, const QParams& p, int cu_count, size_t lds,
                               hipStream_t s) {
  if (lds > 64 * 1024) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 64 * QGEMV_WAVES, lds) !=
          hipSuccess || occ < 1)
    occ = 1;
  if (occ > QGEMV_WG_PER_CU) occ = QGEMV_WG_PER_CU;
  const int64_t rows_per_wg = (int64_t)QGEMV_WAVES * QGEMV_ROWS;
  const int64_t blocks = (p.N + rows_per_wg - 1) / rows_per_wg;
  const int64_t cap = (int64_t)cu_count * occ;
  const unsigned grid = (unsigned)(blocks < cap ? blocks : cap);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * QGEMV_WAVES), lds, s, p);
  return hipGetLastError();
}

template <int XT, int BITS, int MT>
hipError_t launch_qgemv_t(const QParams& p, int cu_count, hipStream_t s) {
  const size_t lds = (size_t)qgemv_lds_bytes(p.M, p.K, BITS);
  if (qgemv_shared_so(p)) return launch_qgemv_kernel(qgemv_kernel<XT, BITS, MT, true>, p, cu_count, lds, s);
  return launch_qgemv_kernel(qgemv_kernel<XT, BITS, MT, false>, p, cu_count, lds, s);
}

template <int XT, int BITS>
hipError_t launch_qgemv_b(const QParams& p, int cu_count, hipStream_t s) {
  if (p.M <= 1) return launch_qgemv_t<XT, BITS, 1>(p, cu_count, s);
  if (p.M <= 2) return launch_qgemv_t<XT, BITS, 2>(p, cu_count, s);
  return launch_qgemv_t<XT, BITS, 4>(p, cu_count, s);
}

// The host has checked: 1 <= M <= 4, LDS need <= 80 KiB, alignment and group divisibility.
hipError_t launch_qgemv(const QParams& p, int x_type, int cu_count, hipStream_t s) {
  if (x_type == BF16)
    return p.bits == 4 ? launch_qgemv_b<BF16, 4>(p, cu_count, s) : launch_qgemv_b<BF16, 8>(p, cu_count, s);
  return p.bits == 4 ? launch_qgemv_b<F16, 4>(p, cu_count, s) : launch_qgemv_b<F16, 8>(p, cu_count, s);
}

}  // namespace tgemm
