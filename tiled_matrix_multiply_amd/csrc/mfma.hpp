// Matrix-core (MFMA) tiled GEMM for gfx950.
//
// Structure (each piece restated from the pages, rebuilt for CDNA4):
//  * One workgroup per BM x BN output tile; the grid counts workgroups ("X3: Metal GEMM",
//    section 6 and its first pitfall: the dispatch unit must be the tile, not the thread).
//  * Cooperative global -> LDS staging of a BM x BK slice of op(A) and a BK x BN slice of
//    op(B), zero outside the matrix ("X3", sections 2 and 4), with 16-byte vector loads per
//    thread (the vectorised loader of "X3", section 7).
//  * A register-blocked accumulator grid per wavefront: each wave keeps FM x FN 32x32 fp32
//    accumulator tiles for the whole kernel and marches K in MFMA-sized steps ("Case Study:
//    Steel's BlockMMA", the TM x TN fragment grid and its K-march; "X3", section 4 on why more
//    accumulators per wave means more reuse).
//  * Transposition handled by layout, never by branching in the inner loop ("Steel's
//    BlockMMA", stride constants): both operands are staged K-contiguous in LDS; an operand
//    whose storage is contiguous along M or N is transposed in registers while staging.
//  * The epilogue applies alpha, beta*C, bias and GELU to the accumulators in registers and
//    stores once ("Steel's BlockMMA", store_result; "Case Study: The Tiled GEMM", fused
//    alpha*AB + beta*C), with an unmasked store for interior tiles and a masked store at the
//    edges ("X3", section 5: store_result versus store_result_safe).
// What differs from the pages' Metal kernels: MFMA 32x32 tiles instead of 8x8 simdgroup
// fragments, a double-buffered K loop with a single barrier per step instead of two
// barriers, an XOR-swizzled LDS layout instead of padding, and an XCD-aware tile order.
#pragma once

#include "common.hpp"

namespace tgemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------- LDS layout --
// Each operand tile row (one m of op(A), or one n of op(B)) holds 128 bytes of K as eight
// 16-byte chunks.  Chunk c of row r sits at byte r*128 + 16*lds_swizzle(r, c).  The XOR with
// (r ^ r/8) keeps both access patterns free of bank conflicts: 8 consecutive rows read at the
// same logical chunk (fragment reads), and rows 8 apart written at the same chunk (the
// transposing stager).
constexpr int ROW_BYTES = 128;

__device__ __forceinline__ int lds_swizzle(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// ------------------------------------------------------------------------- MFMA ops --
// Each op consumes, per lane, CPL 16-byte chunks of the first operand (32 rows of D) and of
// the second operand (32 columns of D) for one "k-group" of KG_CHUNKS chunks per row.  Lanes
// 0-31 supply the first CPL chunks of the group for rows/columns 0-31, lanes 32-63 the next CPL
// chunks.  Any fixed assignment of k to (lane half, byte) is correct as long as both operands
// use the same one, which the symmetric operand layouts of these instructions guarantee.
// Result layout of every 32x32 op: lane l holds column l%32 of D; register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
template <int DT> struct MmaOp;

template <> struct MmaOp<BF16> {
  static constexpr int KG_CHUNKS = 2, CPL = 1;
  __device__ static __forceinline__ f32x16 run(const u32x4* x, const u32x4* y, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x[0]),
                                                   __builtin_bit_cast(bf16x8, y[0]), c, 0, 0, 0);
  }
};

template <> struct MmaOp<F16> {
  static constexpr int KG_CHUNKS = 2, CPL = 1;
  __device__ static __forceinline__ f32x16 run(const u32x4* x, const u32x4* y, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x[0]),
                                                  __builtin_bit_cast(f16x8, y[0]), c, 0, 0, 0);
  }
};

// fp32: the 32x32x2 op takes one value per lane; a 16-byte chunk feeds four ops.
template <> struct MmaOp<F32> {
  static constexpr int KG_CHUNKS = 2, CPL = 1;
  __device__ static __forceinline__ f32x16 run(const u32x4* x, const u32x4* y, f32x16 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(x[0][s]), __uint_as_float(y[0][s]),
                                               c, 0, 0, 0);
    return c;
  }
};

// fp8 E4M3 (OCP): the 32x32x64 f8f6f4 op, format code 0 (E4M3) for both operands, unit block
// scales (E8M0 exponent 127 = 2^0); the per-tensor scales are folded into alpha instead.
template <> struct MmaOp<E4M3> {
  static constexpr int KG_CHUNKS = 4, CPL = 2;
  __device__ static __forceinline__ f32x16 run(const u32x4* x, const u32x4* y, f32x16 c) {
    const i32x8 xa = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                      (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]};
    const i32x8 ya = {(int)y[0][0], (int)y[0][1], (int)y[0][2], (int)y[0][3],
                      (int)y[1][0], (int)y[1][1], (int)y[1][2], (int)y[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, ya, c, 0, 0, 0, 127, 0, 127);
  }
};

// ----------------------------------------------------------------------------- staging --

// Load the first `n` elements (n < 16/ES) of a 16-byte chunk, zero the rest.
template <int ES>
__device__ __forceinline__ u32x4 load_partial(const uint8_t* src, int n) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < n; ++e) {
    uint32_t v;
    if constexpr (ES == 4) v = reinterpret_cast<const uint32_t*>(src)[e];
    else if constexpr (ES == 2) v = reinterpret_cast<const uint16_t*>(src)[e];
    else v = src[e];
    const int bit = e * ES * 8;
    w[bit >> 5] |= v << (bit & 31);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Global -> register -> LDS staging of one operand tile (ROWS rows of 128 bytes of K) by NTH
// threads.  K-contiguous storage (row r at X + r*ld): each thread moves LOADS whole chunks.
// MN-contiguous storage (k-row k at X + k*ld): each thread loads KR k-rows of one 16-byte
// run along M/N and transposes them into CE row pieces of KR elements.
template <int ES, int ROWS, int NTH, bool MN>
struct Stage {
  static constexpr int CE = 16 / ES;               // elements per 16-byte chunk
  static constexpr int LOADS = ROWS * 8 / NTH;     // 16-byte loads per thread per tile
  static constexpr int KR = MN ? (LOADS < CE ? LOADS : CE) : 1;
  static constexpr int UNITS = LOADS / KR;
  static constexpr int MNC = ROWS / CE;            // 16-byte runs along M/N per k-row
  static_assert(ROWS * 8 % NTH == 0 && LOADS % KR == 0, "staging split");

  __device__ static __forceinline__ void load(u32x4 (&r)[LOADS], const uint8_t* X, int64_t ld,
                                              int row0, int rows, int k0, int K, int t) {
    if constexpr (!MN) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int e = t + u * NTH, row = e >> 3, c = e & 7;
        const int grow = row0 + row, gk = k0 + c * CE;
        const uint8_t* src = X + ((int64_t)grow * ld + gk) * ES;
        if (grow < rows && gk + CE <= K) r[u] = *reinterpret_cast<const u32x4*>(src);
        else if (grow < rows && gk < K) r[u] = load_partial<ES>(src, K - gk);
        else r[u] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        const int e = t + u * NTH, mc = e % MNC, kb = e / MNC;
        const int gmn = row0 + mc * CE;
#pragma unroll
        for (int q = 0; q < KR; ++q) {
          const int gk = k0 + kb * KR + q;
          const uint8_t* src = X + ((int64_t)gk * ld + gmn) * ES;
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (gk < K && gmn + CE <= rows) v = *reinterpret_cast<const u32x4*>(src);
          else if (gk < K && gmn < rows) v = load_partial<ES>(src, rows - gmn);
          r[u * KR + q] = v;
        }
      }
    }
  }

  // Dword w of the piece for M/N position j: the elements of k-rows w*(4/ES) .. at column j.
  __device__ static __forceinline__ uint32_t piece_dword(const u32x4* r, int j, int w) {
    if constexpr (ES == 4) {
      return r[w][j];
    } else if constexpr (ES == 2) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      return __builtin_amdgcn_perm(r[2 * w + 1][j >> 1], r[2 * w][j >> 1], sel);
    } else {
      const int b = j & 3, d = j >> 2;
      const uint32_t sel = (uint32_t)b | ((uint32_t)(4 + b) << 8) | 0x0c0c0000u;
      const uint32_t lo = __builtin_amdgcn_perm(r[4 * w + 1][d], r[4 * w][d], sel);
      const uint32_t hi = __builtin_amdgcn_perm(r[4 * w + 3][d], r[4 * w + 2][d], sel);
      return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }

  __device__ static __forceinline__ void store(const u32x4 (&r)[LOADS], uint8_t* lds, int t) {
    if constexpr (!MN) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int e = t + u * NTH, row = e >> 3, c = e & 7;
        *reinterpret_cast<u32x4*>(lds + row * ROW_BYTES + lds_swizzle(row, c) * 16) = r[u];
      }
    } else {
      constexpr int PIECE = KR * ES;  // bytes per row piece: 4, 8 or 16
#pragma unroll
      for (int u = 0; u < UNITS; ++u) {
        const int e = t + u * NTH, mc = e % MNC, kb = e / MNC;
        const int kbyte = kb * PIECE, c = kbyte >> 4, off = kbyte & 15;
        const u32x4* src = &r[u * KR];
#pragma unroll
        for (int j = 0; j < CE; ++j) {
          const int row = mc * CE + j;
          uint8_t* dst = lds + row * ROW_BYTES + lds_swizzle(row, c) * 16 + off;
          if constexpr (PIECE == 16) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{piece_dword(src, j, 0), piece_dword(src, j, 1),
                                                   piece_dword(src, j, 2), piece_dword(src, j, 3)};
          } else if constexpr (PIECE == 8) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{piece_dword(src, j, 0), piece_dword(src, j, 1)};
          } else {
            *reinterpret_cast<uint32_t*>(dst) = piece_dword(src, j, 0);
          }
        }
      }
    }
  }
};

// ----------------------------------------------------------------------- configuration --

template <int DT_, int TILE_, int WM_, int WN_, bool A_MN_, bool B_MN_>
struct MfmaCfg {
  static constexpr int DT = DT_;
  static constexpr int CT = (DT_ == E4M3) ? BF16 : DT_;
  static constexpr int BM = TILE_, BN = TILE_;
  static constexpr int WM = WM_, WN = WN_, NW = WM_ * WN_, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 accumulators per wave
  static constexpr int ES = DTypeInfo<DT_>::bytes;
  static constexpr int BKE = ROW_BYTES / ES;           // K elements per staged tile
  static constexpr bool A_MN = A_MN_, B_MN = B_MN_;    // operand stored contiguous along M/N
  static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
  static constexpr int NTH = NT / 2;                   // stager threads per operand
  using SA = Stage<ES, BM, NTH, A_MN_>;
  using SB = Stage<ES, BN, NTH, B_MN_>;
  static_assert(SA::LOADS == SB::LOADS, "both operands share the prefetch registers");
  static constexpr int LOADS = SA::LOADS;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is a whole number of 32x32 tiles");
};

// Group of tile rows walked together so that concurrently running tiles share A panels.
constexpr int TILE_GROUP_M = 4;

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_mfma_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE_BYTES];
  using Op = MmaOp<C::DT>;
  constexpr int G = 8 / Op::KG_CHUNKS;  // k-groups per staged tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Tile order.  Workgroups are dealt to the 8 XCDs round-robin by id; renumber so each XCD
  // receives a contiguous range, then walk tiles in groups of TILE_GROUP_M tile rows so the
  // tiles on one XCD share A and B panels in that XCD's L2.
  int bid = blockIdx.x;
  const int T = p.tiles_m * p.tiles_n;
  if ((T & 7) == 0) bid = (bid & 7) * (T >> 3) + (bid >> 3);
  const int per_group = TILE_GROUP_M * p.tiles_n;
  const int first_m = (bid / per_group) * TILE_GROUP_M;
  const int gsz = min(p.tiles_m - first_m, TILE_GROUP_M);
  const int tm = first_m + (bid % per_group) % gsz;
  const int tn = (bid % per_group) / gsz;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // The first half of the threads stages op(A), the second half op(B) (wave-uniform split).
  const bool stages_a = tid < C::NTH;
  const int st = stages_a ? tid : tid - C::NTH;
  const uint8_t* Ag = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* Bg = reinterpret_cast<const uint8_t*>(p.B);

  u32x4 pre[C::LOADS];
  auto gload = [&](int kt) {
    const int k0 = kt * C::BKE;
    if (stages_a) C::SA::load(pre, Ag, p.lda, m0, p.M, k0, p.K, st);
    else C::SB::load(pre, Bg, p.ldb, n0, p.N, k0, p.K, st);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * C::STAGE_BYTES;
    if (stages_a) C::SA::store(pre, base, st);
    else C::SB::store(pre, base + C::BM * ROW_BYTES, st);
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  auto compute = [&](int buf) {
    const uint8_t* As = smem + buf * C::STAGE_BYTES;
    const uint8_t* Bs = As + C::BM * ROW_BYTES;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      u32x4 af[C::FM][Op::CPL], bf[C::FN][Op::CPL];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WTM + i * 32 + lrow;
#pragma unroll
        for (int x = 0; x < Op::CPL; ++x) {
          const int c = g * Op::KG_CHUNKS + lhalf * Op::CPL + x;
          af[i][x] = *reinterpret_cast<const u32x4*>(As + row * ROW_BYTES + lds_swizzle(row, c) * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WTN + j * 32 + lrow;
#pragma unroll
        for (int x = 0; x < Op::CPL; ++x) {
          const int c = g * Op::KG_CHUNKS + lhalf * Op::CPL + x;
          bf[j][x] = *reinterpret_cast<const u32x4*>(Bs + row * ROW_BYTES + lds_swizzle(row, c) * 16);
        }
      }
      // D = op(B)^T-fragment x op(A)^T-fragment: rows of D are n, columns are m, so each lane
      // ends up holding 4 consecutive n of one m (vector stores along the C row).
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = Op::run(bf[j], af[i], acc[i][j]);
    }
  };

  // Double-buffered K loop: tile kt+1 travels global -> registers while tile kt is multiplied
  // from LDS; one barrier per step separates "stage kt+1 written" from "stage kt+1 read" and
  // "stage kt read" from "stage kt overwritten two steps later".
  const int KT = (p.K + C::BKE - 1) / C::BKE;
  if (KT > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kt + 1);
    compute(kt & 1);
    if (kt + 1 < KT) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue in registers, then one store per element.
  const bool full = (m0 + C::BM <= p.M) && (n0 + C::BN <= p.N);
  const float alpha = p.alpha, beta = p.beta;
  const uint32_t epi = p.epi;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int m = m0 + wm * C::WTM + i * 32 + lrow;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n0 + wn * C::WTN + j * 32 + rg * 8 + lhalf * 4;
        const int64_t idx = (int64_t)m * p.ldc + n;
        float v[4];
        if (full) {
          float cin[4] = {0.f, 0.f, 0.f, 0.f}, bj[4] = {0.f, 0.f, 0.f, 0.f};
          if (beta != 0.0f) {
            if constexpr (C::CT == F32) {
              const float4 c4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.C) + idx);
              cin[0] = c4.x; cin[1] = c4.y; cin[2] = c4.z; cin[3] = c4.w;
            } else {
              const u32x2 c2 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(p.C) + idx);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t h = (c2[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                cin[e] = (C::CT == F16) ? f16_bits_to_float(h) : bf16_bits_to_float(h);
              }
            }
          }
          if (epi & EPI_BIAS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) bj[e] = p.bias[n + e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = epilogue_value(acc[i][j][rg * 4 + e], alpha, beta, cin[e], bj[e], epi);
          if constexpr (C::CT == F32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + idx) = float4{v[0], v[1], v[2], v[3]};
          } else {
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (C::CT == F16) ? float_to_f16_bits(v[e]) : float_to_bf16_bits(v[e]);
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.C) + idx) =
                u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          }
        } else if (m < p.M) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e < p.N) {
              const float cin = beta != 0.0f ? load_as_float<C::CT>(p.C, idx + e) : 0.0f;
              const float bj = (epi & EPI_BIAS) ? p.bias[n + e] : 0.0f;
              store_from_float<C::CT>(p.C, idx + e,
                                      epilogue_value(acc[i][j][rg * 4 + e], alpha, beta, cin, bj, epi));
            }
          }
        }
      }
    }
  }
}

template <class C>
hipError_t launch_mfma_cfg(const GemmParams& p, hipStream_t s) {
  const int64_t T = (int64_t)p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((gemm_mfma_kernel<C>), dim3((unsigned)T), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// Tile families: 0 -> 64x64 (2x2 waves of 32x32), 1 -> 128x128 (2x2 waves of 64x64),
// 2 -> 256x256 (2x4 waves of 128x64).
constexpr int TILE_SIZE[3] = {64, 128, 256};

template <int DT, int TILE, int WM, int WN>
hipError_t launch_mfma_layout(const GemmParams& p, bool a_mn, bool b_mn, hipStream_t s) {
  if (!a_mn && !b_mn) return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, false, false>>(p, s);
  if (!a_mn && b_mn) return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, false, true>>(p, s);
  if (a_mn && !b_mn) return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, true, false>>(p, s);
  return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, true, true>>(p, s);
}

template <int DT>
hipError_t launch_mfma_dtype(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s) {
  switch (tile) {
    case 0: return launch_mfma_layout<DT, 64, 2, 2>(p, a_mn, b_mn, s);
    case 1: return launch_mfma_layout<DT, 128, 2, 2>(p, a_mn, b_mn, s);
    case 2: return launch_mfma_layout<DT, 256, 2, 4>(p, a_mn, b_mn, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tgemm
