// Matrix-core (MFMA) tiled GEMM for gfx950.
//
// Structure (each piece restated from the pages, rebuilt for CDNA4):
//  * One workgroup per BM x BN output tile; the grid counts workgroups ("X3: Metal GEMM",
//    section 6 and its first pitfall: the dispatch unit is the tile, not the thread).
//  * Cooperative global -> LDS staging of a BM x BK slice of op(A) and a BK x BN slice of
//    op(B) per K step ("X3", sections 2 and 4), 16 contiguous bytes per lane (the vectorised
//    loader of "X3", section 7).  Here the copy goes straight from global memory into LDS
//    (buffer loads with the LDS-destination bit), so staging costs no registers.
//  * A register-blocked accumulator grid per wavefront: each wave keeps FM x FN 32x32 fp32
//    accumulator tiles for the whole kernel and marches K in MFMA-sized steps ("Case Study:
//    Steel's BlockMMA", the TM x TN fragment grid and its K-march; "X3", section 4 on why more
//    accumulators per wave means more reuse).
//  * Transposition by layout, never by branching in the inner loop ("Steel's BlockMMA",
//    stride constants).  Each operand is copied into LDS in its storage order; an operand stored
//    contiguous along K is read with 16-byte LDS loads, one stored contiguous along M or N with
//    the CDNA4 transposing LDS loads (ds_read_b64_tr_b16 / _tr_b8), which hand each lane K-runs
//    of one column.
//  * The epilogue applies alpha, beta*C, bias and GELU to the accumulators in registers and
//    stores once ("Steel's BlockMMA", store_result; "Case Study: The Tiled GEMM", fused
//    alpha*AB + beta*C), with an unmasked store for interior tiles and a masked store at the
//    edges ("X3", section 5: store_result versus store_result_safe).
// Zero fill at the edges ("X3", sections 2 and 4): each operand's buffer descriptor spans
// exactly the bytes the matrix occupies, so loads past its end read zero without touching
// memory.  Rows past M (or columns past N) that still fall inside the matrix feed only output
// rows (columns) that are never stored.  The one case that needs care is K: in the last K
// tile, chunks that reach past K are rewritten in LDS with zeros beyond K.
// What differs from the pages' Metal kernels: 32x32 MFMA tiles instead of 8x8 simdgroup
// fragments, a multi-buffered K loop (2 or 3 LDS stages) with a single barrier per step
// instead of two, an XOR-swizzled LDS layout instead of padding, an XCD-aware tile order, and
// interior-tile stores staged per wave through LDS (the pages' Cs buffer) so that every store
// instruction writes whole cache lines.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace tgemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor word 3 for raw (unformatted, unswizzled) buffers on gfx9-family parts.
constexpr int BUFFER_FLAGS = 0x00020000;

// Raw buffer descriptor over [base, base + bytes): reads past the end return zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, BUFFER_FLAGS};
}

// Wait until at most N of this wave's vector-memory loads are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most n loads are outstanding, LO <= n <= HI (n is uniform; the count must be
// an immediate, so the possible values are split by a binary search of uniform branches).
template <int LO, int HI>
__device__ __forceinline__ void wait_vm(int n) {
  if constexpr (LO >= HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vm<MID, HI>(n);
    else wait_vm<LO, MID - 1>(n);
  }
}

// 16 bytes per lane from the buffer at byte offset voffset straight into LDS at
// lds_base + 16 * lane (lds_base is wave-uniform).  Written as inline assembly so that the
// compiler does not treat the in-flight LDS writes as aliasing every LDS read that follows:
// the kernel itself waits (vmcnt 0) and barriers before any wave reads the stage written.
// m0 holds the LDS base for the instruction and is restored afterwards.
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voffset), "s"(rsrc)
      : "memory");
}

// ------------------------------------------------------------------------- MFMA ops --
// Each op consumes, per lane, CPL 16-byte "chunks" of the first operand (32 rows of D) and of
// the second operand (32 columns of D) for one k-group of 2*CPL chunks.  Lane half h (lanes
// 32h .. 32h+31, one row/column each) holds chunk 2x + h of the group in its x-th 16 bytes,
// K running in order through each chunk.  Any assignment shared by both operands gives the dot
// product; this one is the hardware's for the scaled 8-bit op, where the K block of a byte is
// fixed by its position in the operand (bytes 16x .. 16x+15 of both lane halves form block x,
// scaled by lane half x's scale: measured with a one-wave probe), so that block x of the
// k-group is chunks 2x and 2x+1.  With one chunk per lane (CPL = 1) lane half h holds chunk h.
// Result layout of every 32x32 op: lane l holds column l%32 of D; register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
template <int DT> struct MmaOp;

template <> struct MmaOp<BF16> {
  static constexpr int KG = 16, CPL = 1;  // K per k-group, 16-byte chunks per lane
  using Frag = u32x4;
  __device__ static __forceinline__ f32x16 run(const Frag& x, const Frag& y, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
  }
};

template <> struct MmaOp<F16> {
  static constexpr int KG = 16, CPL = 1;
  using Frag = u32x4;
  __device__ static __forceinline__ f32x16 run(const Frag& x, const Frag& y, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
  }
};

// fp32: the 32x32x2 op takes one value per lane; one 4-value chunk feeds four ops.
template <> struct MmaOp<F32> {
  static constexpr int KG = 8, CPL = 1;
  using Frag = u32x4;
  __device__ static __forceinline__ f32x16 run(const Frag& x, const Frag& y, f32x16 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(x[s]), __uint_as_float(y[s]), c, 0, 0, 0);
    return c;
  }
};

// 8-, 6- and 4-bit inputs (OCP E4M3, E5M2, E2M3, E3M2, E2M1): the 32x32x64 f8f6f4 op with a
// format code per operand and one E8M0 scale per lane half and operand: lanes 32h .. 32h+31
// give the scale of the k-group's block h (its k 32h .. 32h+31), which with per-tensor scaling
// is 2^0 (code 127, the scales folded into alpha).  XT is the type of the first operand (the B
// fragment), YT of the second.  KG counts staged bytes per k-group of 64 elements: 64 (8-bit),
// 48 (packed 6-bit), 32 (packed 4-bit).  Where each element sits in a lane differs by width (an
// in-bounds one-instruction probe): an 8-bit lane half h holds k 16h .. 16h+15 and
// 32+16h .. 32+16h+15 (bytes 0-15 and 16-31), a 6- or 4-bit lane half h holds k 32h .. 32h+31 in
// order, element i at bits 6i (4i) of its 6 (4) registers.  So 6-bit pairs only with 6-bit and
// 4-bit with 4-bit.
template <int DT>
constexpr int f8f6f4_format() {
  return DT == E4M3 ? 0 : DT == E5M2 ? 1 : DT == E2M3 ? 2 : DT == E3M2 ? 3 : 4;
}
template <int DT>
constexpr bool is_fp6() { return DT == E2M3 || DT == E3M2; }

template <int XT, int YT>
struct MmaScaled {
  static_assert((XT == E2M1) == (YT == E2M1), "fp4 pairs only with fp4");
  static_assert(is_fp6<XT>() == is_fp6<YT>(), "6-bit pairs only with 6-bit");
  static constexpr bool FP4 = XT == E2M1, FP6 = is_fp6<XT>();
  static constexpr int KG = FP4 ? 32 : (FP6 ? 48 : 64), CPL = FP4 ? 1 : 2;
  using Frag = typename std::conditional<FP4, u32x4, u32x8>::type;
  __device__ static __forceinline__ i32x8 widen(const Frag& x) {
    if constexpr (FP4) return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
    else return __builtin_bit_cast(i32x8, x);
  }
  // OS: which byte of the scale registers sx and sy the op reads (its op_sel field)
  template <int OS = 0>
  __device__ static __forceinline__ f32x16 run(const Frag& x, const Frag& y, f32x16 c, int sx,
                                               int sy) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        widen(x), widen(y), c, f8f6f4_format<XT>(), f8f6f4_format<YT>(), OS, sx, OS, sy);
  }
};

template <int DT>
constexpr bool is_f8f6f4() { return DT == E4M3 || DT == E5M2 || DT == E2M1 || is_fp6<DT>(); }

// ----------------------------------------------------------------------- configuration --

// LDS stages (K tiles resident or in flight per operand) by tile size, from a sweep over
// n = 512 .. 2048 (fp16, random operands): the 128 x 128 tile with one group of four waves
// gains 12% at 2048 from a third stage (its four waves cannot hide one copy's latency; the 16-
// and 32-bit types now split its K loop between two groups of two stages instead, which is
// faster still); the 64 x 64 tile loses from any more (fewer workgroups fit a compute unit);
// the 256 x 256 tile fills 128 of the 160 KB with two.
template <int TILE>
constexpr int default_stages() { return TILE == 128 ? 3 : 2; }

// DT_ / BT_: types of A and B (they differ only within the 8-bit or the 6-bit family); MX_: OCP
// microscaling, one E8M0 scale per 32 k of each row of op(A) and column of op(B).
// QB_: B is given as affine group-quantized codes of QB_ bits (4 or 8; 0 = B is plain data),
// dequantised into the 16-bit type of A as it is staged (the B tile then looks exactly like a
// K-contiguous 16-bit B).  KS_: K split inside the workgroup: KS_ groups of WM_ x WN_ waves
// each walk every KS_-th K tile with their own LDS stages and add their accumulators at the
// end (small problems, whose time is the chain of K tiles rather than the multiplies).
// BN_: tile width along N (0: square, BN = TILE_).  SK_: the K loop split across workgroups,
// 1, 2 or 0: with 2, two workgroups share a tile, each multiplying one half of its K tiles; the
// first to finish hands its fp32 accumulators to the other through a workspace in device memory
// (a pair protocol, below), and the other adds them and runs the epilogue.  With 0 (stream-K)
// a persistent grid shares out the K tiles of all output tiles evenly, in contiguous runs that
// may start and end inside a tile; the parts of a split tile meet through the workspace.
template <int DT_, int TILE_, int WM_, int WN_, bool A_MN_, bool B_MN_,
          int S_ = default_stages<TILE_>(), int BT_ = DT_, bool MX_ = false, int QB_ = 0,
          int KS_ = 1, int BN_ = 0, int SK_ = 1>
struct MfmaCfg {
  static constexpr int DT = DT_, BT = BT_;
  static constexpr bool F8 = is_f8f6f4<DT_>(), MX = MX_;
  static_assert(DT_ == BT_ || (F8 && is_f8f6f4<BT_>()), "mixed types only in the 8-bit family");
  static_assert(!MX_ || F8, "block scales only with 8- and 4-bit inputs");
  using Op = typename std::conditional<F8, MmaScaled<BT_, DT_>, MmaOp<DT_>>::type;
  static constexpr int CT = F8 ? BF16 : DT_;
  static constexpr int BM = TILE_, BN = BN_ ? BN_ : TILE_;
  static constexpr int KS = KS_, SK = SK_;
  static_assert(SK_ == 1 || ((SK_ == 2 || SK_ == 0) && KS_ == 1 && !MX_ && QB_ == 0),
                "K split across workgroups: plain inputs, no split inside");
  static_assert(SK_ != 0 || (TILE_ == 256 && BN_ == 0), "stream-K runs the 256 x 256 tile");
  static constexpr int WM = WM_, WN = WN_, NW = WM_ * WN_, NT = NW * 64 * KS_;  // NW waves per K group
  // Waves that issue the K loop's copies.  The 256 x 256 tile runs two waves per SIMD; right
  // after each barrier every wave would issue its copies at once, the address unit's queue
  // fills, and both waves of a SIMD stall on it together while the matrix core idles.  So one
  // wave per SIMD issues all of them (data and block scales), and the other keeps multiplying
  // meanwhile: the dispatcher deals a workgroup's waves to the four SIMDs in turn, so waves
  // 0 .. 3 sit on four different SIMDs and wave w + 4 shares wave w's (read from the hardware-ID
  // register).  Measured at 4096 x 4096 x 8192: bf16 -1.8%, fp8 -3%, MXFP4 -3.5%, fused bf16
  // + bias + GELU 4096^3 -2.5%; with quantized B (whose codes every thread still loads) the
  // 4-bit prefill 4096^3 -1.6%; 6-bit inputs, whose copies skip the unused quarter of each row
  // (below), about -1%.
  static constexpr int NCW = (TILE_ == 256 && BN_ == 0 && NW == 8 && KS_ == 1) ? 4 : NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 accumulators per wave
  static constexpr int ES = DTypeInfo<DT_>::bytes;
  static constexpr bool FP6 = is_fp6<DT_>();
  // K elements per staged tile: 128 bytes of each row, or for packed 6-bit rows 96 bytes (128
  // elements, two k-groups) in the 128-byte LDS row; the copies move the row's 128 bytes from
  // the tile start (on the 256 tile only the first 96), and the fragment reads never touch the
  // last 32.
  static constexpr int BKE = FP6 ? 96 : 128 / ES;
  static constexpr bool A_MN = A_MN_, B_MN = B_MN_;    // operand stored contiguous along M/N
  static_assert(!FP6 || (!A_MN_ && !B_MN_), "packed 6-bit operands are staged K-contiguous");
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;  // one staged K tile
  static constexpr int S = S_;  // LDS buffers per operand: K tiles kt .. kt+S-1 are resident or in flight
  static constexpr int QB = QB_;
  static_assert(QB_ == 0 || ((QB_ == 4 || QB_ == 8) && !B_MN_ && !MX_ && S_ == 2 &&
                             (DT_ == BF16 || DT_ == F16)),
                "quantized B: K-contiguous codes, 16-bit A, two stages");
  // MX scales: a staged K tile covers BPT 32-element blocks (4 for 8- and 6-bit elements, 8
  // for packed fp4); each row's 16 consecutive scale bytes (TPC = 16 / BPT tiles) are copied as one
  // piece into a double-buffered region of (BM + BN) rows x 16 bytes after the data stages.
  static constexpr int BPT = (DT_ == E2M1) ? 8 : 4, TPC = 16 / BPT;
  static constexpr int GS = S * (A_BYTES + B_BYTES);  // one K group's stages
  static constexpr int SC_OFF = KS_ * GS, SC_BUF = (BM + BN) * 16;
  static constexpr int LDS_BYTES = SC_OFF + (MX_ ? 2 * SC_BUF : 0);
  // K split: the partial accumulators of groups 1 .. KS-1 (fp32, wave by wave), then the
  // epilogue's output staging
  static constexpr int ACC_BYTES = (BM / WM) * (BN / WN) * 4 * NW;  // one group's accumulators
  static constexpr int STG_OFF = (KS_ - 1) * ACC_BYTES;
  static_assert(KS_ == 1 || ((KS_ == 2 || KS_ == 4) && !MX_ && QB_ == 0),
                "K split: 2 or 4 groups, plain inputs");
  static_assert(S >= 2 && LDS_BYTES <= 160 * 1024, "LDS holds at most 160 KB");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is a whole number of 32x32 tiles");
};

constexpr int gcd8(int x) { return (x & 7) == 0 ? 8 : (x & 3) == 0 ? 4 : (x & 1) == 0 ? 2 : 1; }

// One operand's staged tile.  LDS holds it in storage order:
//  * K-contiguous (A not transposed, B transposed): BX rows of 128 bytes (one row per m or n),
//    eight 16-byte chunks per row, chunk c of row r at position c ^ kswz(r);
//  * M/N-contiguous (A transposed, B not transposed): BKE rows of BX*ES bytes (one row per k),
//    chunk c of row k at position c ^ mswz(k).
// The XOR patterns keep the fragment reads free of bank conflicts: eight consecutive rows at
// one chunk (16-byte reads), or 4 (16-bit) / 8 (8-bit) consecutive k-rows at the same columns
// (transposing reads).
template <class C, bool IS_A>
struct Operand {
  static constexpr bool MN = IS_A ? C::A_MN : C::B_MN;
  static constexpr int BX = IS_A ? C::BM : C::BN;   // tile extent along M (A) or N (B)
  static constexpr int ES = C::ES, CE = 16 / ES;    // elements per chunk
  static constexpr int RB = MN ? BX * ES : 128;     // LDS row bytes
  static constexpr int CPR = RB / 16;               // chunks per LDS row
  static constexpr int WLOADS = BX / 8;             // 1 KB wave-loads per tile (BX*128 bytes)
  static constexpr int PER_WAVE = WLOADS / C::NCW;  // copies per copying wave
  static constexpr int RPU = MN ? 1024 / RB : 8;     // rows (k-rows when MN) per wave-load
  // A K-contiguous chunk's position in its row depends only on its wave-load modulo 8 (see
  // chunk_of), so a copying wave's wave-loads i and i % VP differ by a whole number of rows, the
  // same for every lane: the per-lane offsets of the first VP can serve them all, plus a
  // uniform row step folded into the buffer descriptor (scalar work per copy).  Only the
  // block-scaled fp4 kernel does so: on the 256 tile it would spill otherwise, while for the
  // others the descriptor arithmetic costs scalar registers they are short of; they keep one
  // offset register per copy.
  static constexpr int SWZ_STEP = C::NCW;
  static constexpr int VP =
      (MN || !C::MX || C::DT != E2M1 || PER_WAVE < 8 / gcd8(SWZ_STEP)) ? PER_WAVE : 8 / gcd8(SWZ_STEP);
  static_assert(PER_WAVE % VP == 0, "whole periods of per-lane offsets");
  static constexpr int LDS_OFF = IS_A ? 0 : C::S * C::A_BYTES;  // first buffer of the operand
  static constexpr int BUF_BYTES = IS_A ? C::A_BYTES : C::B_BYTES;
  static_assert(WLOADS % C::NCW == 0, "every copying wave issues the same number of loads");
  static_assert(!MN || (RB <= 1024 && 1024 % RB == 0), "whole k-rows per wave-load");

  __device__ static __forceinline__ int kswz(int r) { return (r ^ (r >> 3)) & 7; }
  __device__ static __forceinline__ int mswz(int k) {
    if constexpr (ES == 4) return 0;  // 32 lanes read one k-row: never conflicts
    else if constexpr (ES == 2) return CPR >= 16 ? (k & 3) << 2 : CPR >= 8 ? (k & 3) << 1 : 0;
    else if constexpr (CPR >= 16) return (k & 7) << 1;
    else if constexpr (CPR == 8) return k & 7;
    else return (k >> 1) & 3;
  }

  // The chunk this lane copies in wave-load u: its row in the tile and its logical chunk.
  __device__ static __forceinline__ void chunk_of(int u, int lane, int& row, int& c) {
    if constexpr (!MN) {
      row = 8 * u + (lane >> 3);
      c = (lane & 7) ^ kswz(row);
    } else {
      constexpr int RPW = 1024 / RB;  // k-rows per wave-load
      row = RPW * u + lane / CPR;
      c = (lane % CPR) ^ mswz(row);
    }
  }
};

// Group of tile rows walked together so that concurrently running tiles share A panels.
constexpr int TILE_GROUP_M = 4;

// Byte extent of a stored rows x cols matrix from element (r0, c0) to its last element,
// rounded down to whole 16-byte chunks (so that no 16-byte load straddles the end: a chunk is
// either entirely inside the matrix or reads as zero; the last-K-tile fix-up restores the
// valid part of a chunk cut off here), clamped to what a buffer descriptor holds, and 0 when
// (r0, c0) is past the end.
__device__ __forceinline__ uint32_t extent_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t r0,
                                                 int64_t c0, int es) {
  const int64_t e = (((rows - 1 - r0) * ld + cols - c0) * es) & ~int64_t(15);
  return e <= 0 ? 0u : (e >= 0xfffffff0LL ? 0xfffffff0u : (uint32_t)e);
}

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

// Flags computed on the host: which operands need the last-K-tile fix-up.
enum : uint32_t { FIX_A = 1u << 8, FIX_B = 1u << 9 };

// One stream-K segment: K tiles [kb, ke) of output tile `tile`, taken by contributor `part`
// of the tile's `parts` (consecutive workgroups in the renumbered order, the first of them
// `first_w`; parts == 1: the whole tile).
struct SkSeg {
  int tile, kb, ke, part, parts, first_w;
};

// Workspace slot of stream-K contributor `part` of a tile whose first contributor is workgroup
// w0: each workgroup has two slots, 2 w for the segment its run starts with (the end of a
// tile) and 2 w + 1 for the one its run ends with (the start of a tile, part 0).
__device__ __forceinline__ int64_t sk_slot(int w0, int part) {
  return 2 * (int64_t)(w0 + part) + (part == 0 ? 1 : 0);
}

// The work of one workgroup on one output tile (or, with stream-K, one segment of its K tiles),
// from the copies of its first K tile to the stores of its epilogue.
template <class C>
__device__ __forceinline__ void mfma_tile(const GemmParams p, const SkSeg sg) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
  using Op = typename C::Op;
  using OA = Operand<C, true>;
  using OB = Operand<C, false>;
  constexpr int ES = C::ES;
  constexpr int G = C::BKE / Op::KG;  // k-groups per staged tile

  // (stream-K: the lane index from an instruction the compiler cannot hoist out of the loop
  // over segments; the wave's base index is scalar)
  int tid_l = threadIdx.x;
  if constexpr (C::SK == 0) {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    tid_l = (int)(__builtin_amdgcn_readfirstlane(threadIdx.x) & ~63u) | ln;
  }
  const int tid = tid_l, lane = tid & 63, lane_id = lane;
  // K group (0 unless the K loop is split), wave-uniform so that tile addresses stay scalar
  const int kg = __builtin_amdgcn_readfirstlane((tid >> 6) / C::NW);
  const int wave = (tid >> 6) % C::NW;  // wave within the group
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index, in a scalar register
  uint8_t* const gsm = smem + kg * C::GS;  // the group's stages

  // Tile order.  Workgroups are dealt to the 8 XCDs round-robin by id; renumber so each XCD
  // receives a contiguous range, then walk tiles in groups of TILE_GROUP_M tile rows so the
  // tiles on one XCD share A and B panels in that XCD's L2.
  // With the K loop split across workgroups, the SK workgroups of a tile get consecutive ids
  // after the renumbering, so that both halves of a tile run on one XCD and meet in its L2.
  // With stream-K the segment names the tile (its grid is renumbered the same way, below).
  int bid = blockIdx.x;
  int khalf = 0;  // which part of the K tiles this workgroup takes (K split across workgroups)
  if constexpr (C::SK == 0) {
    bid = sg.tile;
  } else {
    const int T = p.tiles_m * p.tiles_n;
    const int U = T * C::SK;  // workgroups
    if ((U & 7) == 0) bid = (bid & 7) * (U >> 3) + (bid >> 3);
    if constexpr (C::SK > 1) {
      khalf = bid % C::SK;
      bid /= C::SK;
    }
  }
  const int tile_id = bid;
  const int per_group = TILE_GROUP_M * p.tiles_n;
  const int first_m = (bid / per_group) * TILE_GROUP_M;
  const int gsz = min(p.tiles_m - first_m, TILE_GROUP_M);
  const int tm = first_m + (bid % per_group) % gsz;
  const int tn = (bid % per_group) / gsz;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const uint8_t* Ag = reinterpret_cast<const uint8_t*>(p.A);
  const uint8_t* Bg = reinterpret_cast<const uint8_t*>(p.B);

  // Copying waves (all, or one per SIMD; see MfmaCfg::NCW) and this one's index among them.
  const bool copier = C::NCW == C::NW || wave_u < (uint32_t)C::NCW;
  const int cw = wave % C::NCW;
  const uint32_t cw_u = wave_u % C::NCW;
  // Per-lane byte offsets of the chunks this lane copies in its first VP wave-loads (loop
  // invariant); wave-load i uses those of i % VP with the buffer moved on by a row step.
  uint32_t voA[OA::VP], voB[OB::VP];
#pragma unroll
  for (int i = 0; i < OA::VP; ++i) {
    int r, c;
    OA::chunk_of(cw + C::NCW * i, lane, r, c);
    voA[i] = (uint32_t)((int64_t)r * p.lda * ES + c * 16);
  }
#pragma unroll
  for (int i = 0; i < OB::VP; ++i) {
    int r, c;
    OB::chunk_of(cw + C::NCW * i, lane, r, c);
    voB[i] = (uint32_t)((int64_t)r * p.ldb * ES + c * 16);
  }
  // Wave-load i of a copying wave: the buffer [base, base + ext) moved on by the uniform row
  // step between wave-loads i and i % VP (a multiple of 16 bytes, since the row stride is),
  // its extent shortened to match, so that a chunk reads zero exactly where it did before.
  auto copy_wave_loads = [&](auto opnd, const uint8_t* base, uint32_t ext, uint32_t row_bytes,
                             uint32_t l, const uint32_t* vo) {
    using O = decltype(opnd);
#pragma unroll
    for (int i = 0; i < O::PER_WAVE; ++i) {
      const uint32_t step = (uint32_t)((i - i % O::VP) * C::NCW * O::RPU) * row_bytes;
      // an opaque difference: written plainly, the compiler turns the clamp into a saturating
      // subtract that only the vector unit has, and the descriptor leaves the scalar registers
      uint32_t rest = ext - step;
      asm volatile("" : "+s"(rest));
      const i32x4 r = make_rsrc(base + step, ext > step ? rest : 0u);
      if constexpr (C::FP6 && !O::MN && C::BM == 256) {
        // a 6-bit K tile is the first 96 bytes of each 128-byte row: the lanes of the last two
        // chunks copy nothing (their LDS slots are never read).  On the 256 tile that takes a
        // quarter off the copies' address work: MXFP6 4096^3 -4.5%, per-tensor fp6 -5.5%; on
        // the 128 tile the masked loads measured 2% slower, so it copies whole rows
        int row, c;
        O::chunk_of(cw + C::NCW * i, lane, row, c);
        if (c < 6) buffer_load_lds16(r, l + C::NCW * i * 1024, vo[i % O::VP]);
      } else {
        buffer_load_lds16(r, l + C::NCW * i * 1024, vo[i % O::VP]);
      }
    }
  };

  // Issue the direct copies of K tile kt of A (into A buffer buf) or of B (into B buffer buf).
  auto issue_a = [&](int kt, int buf) {
    if (!copier) return;
    const int k0 = kt * C::BKE;
    const uint8_t* base;
    uint32_t ext;
    if constexpr (!OA::MN) {  // A stored M x K
      base = Ag + ((int64_t)m0 * p.lda + k0) * ES;
      ext = extent_bytes(p.M, p.K, p.lda, m0, k0, ES);
    } else {                  // A stored K x M
      base = Ag + ((int64_t)k0 * p.lda + m0) * ES;
      ext = extent_bytes(p.K, p.M, p.lda, k0, m0, ES);
    }
    const uint32_t l = (uint32_t)reinterpret_cast<uintptr_t>(gsm + OA::LDS_OFF + buf * C::A_BYTES) + cw_u * 1024;
    copy_wave_loads(OA{}, base, ext, (uint32_t)(p.lda * ES), l, voA);
  };
  auto issue_b = [&](int kt, int buf) {
    if (!copier) return;
    const int k0 = kt * C::BKE;
    const uint8_t* base;
    uint32_t ext;
    if constexpr (OB::MN) {   // B stored K x N
      base = Bg + ((int64_t)k0 * p.ldb + n0) * ES;
      ext = extent_bytes(p.K, p.N, p.ldb, k0, n0, ES);
    } else {                  // B stored N x K
      base = Bg + ((int64_t)n0 * p.ldb + k0) * ES;
      ext = extent_bytes(p.N, p.K, p.ldb, n0, k0, ES);
    }
    const uint32_t l = (uint32_t)reinterpret_cast<uintptr_t>(gsm + OB::LDS_OFF + buf * C::B_BYTES) + cw_u * 1024;
    copy_wave_loads(OB{}, base, ext, (uint32_t)(p.ldb * ES), l, voB);
  };

  // Last K tile: rewrite every chunk that reaches past K (K-contiguous operand) or past the
  // matrix edge in the final k-row (M/N-contiguous operand) with its valid elements and zeros.
  // Runs after the tile's copies have landed and before the barrier; each copying wave fixes
  // the chunks it copied.
  auto fixup = [&](int kt, int abuf, int bbuf) {
    if (!copier) return;
    // An opaque copy of the lane index keeps the compiler from hoisting this rarely run code's
    // address arithmetic out of the K loop, where it would hold registers for every iteration.
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int k0 = kt * C::BKE;
    if (p.epi & FIX_A) {
#pragma unroll
      for (int i = 0; i < OA::PER_WAVE; ++i) {
        const int u = cw + C::NCW * i;
        int r, c;
        OA::chunk_of(u, lane, r, c);
        uint8_t* dst = gsm + OA::LDS_OFF + abuf * C::A_BYTES + u * 1024 + lane * 16;
        if constexpr (!OA::MN) {
          const int gm = m0 + r, gk = k0 + c * OA::CE;
          if (gk + OA::CE > p.K) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (gm < p.M && gk < p.K) v = load_partial<ES>(Ag + ((int64_t)gm * p.lda + gk) * ES, p.K - gk);
            *reinterpret_cast<u32x4*>(dst) = v;
          }
        } else {
          const int gk = k0 + r, gm = m0 + c * OA::CE;
          if (gk == p.K - 1 && gm < p.M && gm + OA::CE > p.M)
            *reinterpret_cast<u32x4*>(dst) = load_partial<ES>(Ag + ((int64_t)gk * p.lda + gm) * ES, p.M - gm);
        }
      }
    }
    if (p.epi & FIX_B) {
#pragma unroll
      for (int i = 0; i < OB::PER_WAVE; ++i) {
        const int u = cw + C::NCW * i;
        int r, c;
        OB::chunk_of(u, lane, r, c);
        uint8_t* dst = gsm + OB::LDS_OFF + bbuf * C::B_BYTES + u * 1024 + lane * 16;
        if constexpr (!OB::MN) {
          const int gn = n0 + r, gk = k0 + c * OB::CE;
          if (gk + OB::CE > p.K) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (gn < p.N && gk < p.K) v = load_partial<ES>(Bg + ((int64_t)gn * p.ldb + gk) * ES, p.K - gk);
            *reinterpret_cast<u32x4*>(dst) = v;
          }
        } else {
          const int gk = k0 + r, gn = n0 + c * OB::CE;
          if (gk == p.K - 1 && gn < p.N && gn + OB::CE > p.N)
            *reinterpret_cast<u32x4*>(dst) = load_partial<ES>(Bg + ((int64_t)gk * p.ldb + gn) * ES, p.N - gn);
        }
      }
    }
  };

  // Fragment reads.  K-contiguous: one or two 16-byte reads per lane.  M/N-contiguous:
  // transposing reads, each giving a lane 4 (16-bit) or 8 (8-bit) consecutive k of its column;
  // fp32 reads one value per k-row.
  const int lrow = lane & 31, lhalf = lane >> 5;
  using Frag = typename Op::Frag;
  // Per-lane LDS byte offsets of the fragment reads, computed once and kept opaque so that the
  // compiler holds exactly these few registers instead of materialising one address per
  // (fragment, k-group, chunk).
  //  * K-contiguous tile: row = wbase + 32 f + lrow and chunk c = KGC g + 2 x + lhalf sit at
  //    byte row*128 + 16 (c ^ kswz(row)), and kswz(row) = s_lane ^ 4 ((wbase/32 + f) & 1) with
  //    s_lane = (lrow & 7) ^ (lrow >> 3).  So the offset is
  //      (wbase + 32 f) * 128 + (kbase[par] ^ 16 (KGC g + 2 x)),  par = (wbase/32 + f) & 1,
  //    kbase[par] = lrow*128 + 16 (lhalf ^ s_lane ^ 4 par).
  //  * M/N-contiguous tile: the swizzle depends only on k % 4 (16-bit) or k % 8 (8-bit), which is
  //    fixed per lane, so each fragment f has one base and every k-group / k-row step is a
  //    plain offset.
  constexpr int KGC = Op::KG * ES / 16;  // chunks per k-group
  const int s_lane = (lrow & 7) ^ (lrow >> 3);
  auto kbase = [&](int par) {
    int v = lrow * 128 + 16 * (lhalf ^ s_lane ^ (4 * par));
    asm volatile("" : "+v"(v));
    return v;
  };
  auto mbase = [&](auto opnd, int wbase, int f) {
    using O = decltype(opnd);
    int v;
    if constexpr (ES == 2) {
      const int q = lane >> 4, sl = lane & 15;
      const int n = wbase + f * 32 + 16 * (q & 1) + 4 * (sl & 3);
      const int k = 8 * (q >> 1) + (sl >> 2);
      v = k * O::RB + (((n >> 3) ^ O::mswz(k)) << 4) + ((n & 7) << 1);
    } else if constexpr (ES == 1) {
      const int q = lane >> 4, sl = lane & 15;
      const int n = wbase + f * 32 + 16 * (q & 1) + 8 * (sl & 1);
      const int k = 16 * (q >> 1) + (sl >> 1);  // lane half h: k 16h .. (see the op layout)
      v = k * O::RB + (((n >> 4) ^ O::mswz(k)) << 4) + (n & 15);
    } else {
      const int n = wbase + f * 32 + lrow;
      v = 4 * lhalf * O::RB + n * 4;
    }
    asm volatile("" : "+v"(v));
    return v;
  };
  // Packed 6-bit K-contiguous tiles: piece t of k-group g is the 8 bytes at row byte
  // 48 g + 24 lhalf + 8 t, i.e. logical chunk c = that / 16 at byte (that % 16) of it, held at
  // position c ^ kswz(row); for even-parity fragment rows kswz(row) = s_lane, and odd ones flip
  // bit 2 of the position (offset ^ 64), as for the other widths.
  int k6[C::FP6 ? 6 : 1];
  if constexpr (C::FP6) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rb = 48 * g + 24 * lhalf + 8 * t;
        int v = lrow * 128 + (((rb >> 4) ^ s_lane) << 4) + (rb & 15);
        asm volatile("" : "+v"(v));
        k6[3 * g + t] = v;
      }
  }
  // Fragment f of an operand for k-group g, from the operand buffer at byte offset `boff`
  // (uniform) past the operand's first buffer.
  auto read_frag = [&](uint32_t boff, auto opnd, int wbase, int f, int g, const int* kb,
                       const int* mb, Frag& out) {
    using O = decltype(opnd);
    const uint8_t* s = gsm + O::LDS_OFF + boff;
    if constexpr (!O::MN && C::FP6) {
      // the lane half's 32 elements: bytes 48 g + 24 h .. + 23 of the row, three 8-byte pieces
      // (each inside one 16-byte chunk) into registers 0..5; registers 6 and 7 stay zero
      const int par = ((wbase >> 5) + f) & 1;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int off = (wbase + f * 32) * 128 + (k6[3 * g + t] ^ (64 * par));
        const u32x2 v = *reinterpret_cast<const u32x2*>(s + off);
        out[2 * t] = v[0];
        out[2 * t + 1] = v[1];
      }
    } else if constexpr (!O::MN) {
      const int par = ((wbase >> 5) + f) & 1;
#pragma unroll
      for (int x = 0; x < Op::CPL; ++x) {
        const int off = (wbase + f * 32) * 128 + (kb[par] ^ (16 * (KGC * g + 2 * x)));
        const u32x4 v = *reinterpret_cast<const u32x4*>(s + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * x + e] = v[e];
      }
    } else if constexpr (ES == 2) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint8_t* a = s + mb[f] + (g * 16 + 4 * t) * O::RB;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
        const u32x2 d = __builtin_bit_cast(u32x2, v);
        out[2 * t] = d[0];
        out[2 * t + 1] = d[1];
      }
    } else if constexpr (ES == 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // bytes 8t .. 8t+7: k 32 (t / 2) + 16 h + 8 (t % 2) + 0..7 of the k-group
        const uint8_t* a = s + mb[f] + (g * 64 + 32 * (t >> 1) + 8 * (t & 1)) * O::RB;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)a);
        out[2 * t] = (uint32_t)v[0];
        out[2 * t + 1] = (uint32_t)v[1];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        out[t] = *reinterpret_cast<const uint32_t*>(s + mb[f] + (g * 8 + t) * O::RB);
    }
  };
  int kbA[2] = {0, 0}, kbB[2] = {0, 0}, mbA[C::FM], mbB[C::FN];
  if constexpr (!OA::MN) {
    kbA[0] = kbase(0);
    kbA[1] = kbase(1);
  } else {
#pragma unroll
    for (int f = 0; f < C::FM; ++f) mbA[f] = mbase(OA{}, wm * C::WTM, f);
  }
  if constexpr (!OB::MN) {
    kbB[0] = kbase(0);
    kbB[1] = kbase(1);
  } else {
#pragma unroll
    for (int f = 0; f < C::FN; ++f) mbB[f] = mbase(OB{}, wn * C::WTN, f);
  }

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment schedules.  A tile is multiplied in G k-groups; in each, every wave issues the
  // FM x FN multiplies of its accumulator grid.
  //  * 16- and 32-bit inputs (GROUPED): all fragments of k-group g+1 are read while k-group g
  //    is multiplied (two register sets, set g & 1).
  //  * 8-bit inputs (streamed): the 64-cycle multiplies and twice-as-large fragments favour
  //    fewer registers: the tile is walked in S = G * FM steps, step s = g * FM + i issuing the
  //    FN multiplies of row i; the A fragment of step s+1 (slot (s+1) & 1) is read during step
  //    s, and one set of B fragments is read at the start of each k-group.
  // G, FM and S are even, so the register-set parities carry over from tile to tile.
  constexpr bool GROUPED = Op::CPL == 1;
  constexpr int AS = GROUPED ? C::FM : 1;   // A fragments per register set
  constexpr int BS = GROUPED ? 2 : 1;       // B register sets
  Frag af[2][AS], bf[BS][C::FN];
  if constexpr (C::FP6) {  // registers 6 and 7 of a 6-bit fragment are never loaded
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < AS; ++j) af[i][j] = Frag{};
#pragma unroll
    for (int i = 0; i < BS; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) bf[i][j] = Frag{};
  }
  // MX: the E8M0 scales of a fragment lane for every k-group of a K tile, read once per tile
  // and fragment (one 8- or 4-byte read of the staged scale row): lane half h's scale for
  // k-group g is block 2g + h of the tile, held at byte OPS(g) of one register, and the
  // multiply of k-group g selects that byte with its op_sel field.  The words read with the
  // next tile's first fragments (rAn / rBn) are only rearranged into scAc / scBc at the top of
  // that tile: any arithmetic on them before the current tile's last multiplies would make
  // those multiplies wait for the reads.  Blocks past K (the last tile's zero-filled tail)
  // take 2^0 (code 127) whatever the padding holds.
  auto OPS = [](int g) { return C::BPT == 8 ? g : 2 * g; };
  constexpr int RW = C::MX ? C::BPT / 4 : 1;  // words read per fragment and tile
  uint32_t scAc[C::FM], scBc[C::FN], rAn[C::FM][RW] = {}, rBn[C::FN][RW] = {};
#pragma unroll
  for (int i = 0; i < C::FM; ++i) scAc[i] = 0x7F7F7F7Fu;
#pragma unroll
  for (int j = 0; j < C::FN; ++j) scBc[j] = 0x7F7F7F7Fu;
  int scrow = lrow * 16;  // this lane's 16-byte scale row within a fragment's 32 rows
  asm volatile("" : "+v"(scrow));
  auto read_scales = [&](auto opnd, int wbase, int f, int kt, uint32_t (&dst)[RW]) {
    using O = decltype(opnd);
    constexpr int ROW0 = std::is_same<O, OA>::value ? 0 : C::BM;  // A rows, then B rows
    const uint8_t* row = smem + C::SC_OFF + ((kt / C::TPC) & 1) * C::SC_BUF + (ROW0 + wbase + 32 * f) * 16 +
                         (kt % C::TPC) * C::BPT + scrow;
    if constexpr (RW == 2) {
      const u32x2 d = *reinterpret_cast<const u32x2*>(row);
      dst[0] = d[0];
      dst[RW - 1] = d[1];
    } else {
      dst[0] = *reinterpret_cast<const uint32_t*>(row);
    }
  };
  auto read_tile_scales = [&](int kt) {
    if constexpr (C::MX) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) read_scales(OA{}, wm * C::WTM, i, kt, rAn[i]);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) read_scales(OB{}, wn * C::WTN, j, kt, rBn[j]);
    }
  };
  // the scales of tile kt (read by read_tile_scales(kt)) into the registers the multiplies use
  auto next_tile_scales = [&](int kt) {
    if constexpr (C::MX) {
      auto pack = [&](const uint32_t (&w)[RW]) {
        // 8 blocks: this lane half's four (bytes h, 2+h, 4+h, 6+h); 4 blocks: its two, to
        // bytes 0 and 2
        return RW == 2 ? __builtin_amdgcn_perm(w[RW - 1], w[0], lhalf ? 0x07050301u : 0x06040200u)
                       : w[0] >> (8 * lhalf);
      };
#pragma unroll
      for (int i = 0; i < C::FM; ++i) scAc[i] = pack(rAn[i]);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) scBc[j] = pack(rBn[j]);
      // Only a tile that reaches past K (the last, when K is not a whole number of tiles) has
      // blocks to force to 2^0: a uniform branch, so that the other tiles' first multiplies
      // wait on nothing but the byte permutes.
      // (block-scaled kernels never split K, so iteration kt is K tile kt)
      if (kt * C::BPT + C::BPT > p.kblocks) {
        uint32_t fix = 0;  // bytes of blocks past K
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (kt * C::BPT + 2 * g + lhalf >= p.kblocks) fix |= 0xFFu << (8 * OPS(g));
#pragma unroll
        for (int i = 0; i < C::FM; ++i) scAc[i] = (scAc[i] & ~fix) | (0x7F7F7F7Fu & fix);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) scBc[j] = (scBc[j] & ~fix) | (0x7F7F7F7Fu & fix);
      }
    }
  };
  auto load_a = [&](uint32_t aoff, int g, int i, Frag& dst) {
    read_frag(aoff, OA{}, wm * C::WTM, i, g, kbA, mbA, dst);
  };
  auto load_b = [&](uint32_t boff, int g, int set) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) read_frag(boff, OB{}, wn * C::WTN, j, g, kbB, mbB, bf[set][j]);
  };
  // k-group g of tile kt; with g = 0 also the tile's scales
  auto load_group = [&](int kt, uint32_t aoff, uint32_t boff, int g, int set) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) load_a(aoff, g, i, af[set][i]);
    load_b(boff, g, set);
    if (g == 0) read_tile_scales(kt);
  };
  // D = op(B)-fragment x op(A)-fragment: rows of D are n, columns are m, so each lane ends up
  // holding 4 consecutive n of one m (vector stores along the C row).  With the 256 x 256 tile
  // (128 accumulator registers, held in VGPRs) an empty asm after each multiply pins it in
  // place: the multiplies touch no memory, so the compiler would otherwise sink them past the
  // barrier and read every fragment of the tile up front, which costs the registers these
  // schedules are built to save.  Smaller grids keep their accumulators in AccVGPRs, which a
  // VGPR operand constraint would force out and back on every step, so they are not pinned.
  constexpr bool PIN = C::FM * C::FN >= 8;
  // multiplies of A fragment a (row i of the accumulator grid) in k-group g
  auto mma = [&](int i, const Frag& a, int g, int bset) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      if constexpr (C::MX) {
        const int sb = (int)scBc[j], sa = (int)scAc[i];
        switch (OPS(g)) {  // g is a constant once the loops are unrolled
          case 0: acc[i][j] = Op::template run<0>(bf[bset][j], a, acc[i][j], sb, sa); break;
          case 1: acc[i][j] = Op::template run<1>(bf[bset][j], a, acc[i][j], sb, sa); break;
          case 2: acc[i][j] = Op::template run<2>(bf[bset][j], a, acc[i][j], sb, sa); break;
          default: acc[i][j] = Op::template run<3>(bf[bset][j], a, acc[i][j], sb, sa); break;
        }
      } else if constexpr (C::F8) {
        acc[i][j] = Op::run(bf[bset][j], a, acc[i][j], 127, 127);
      } else {
        acc[i][j] = Op::run(bf[bset][j], a, acc[i][j]);
      }
      if constexpr (PIN) asm volatile("" : "+v"(acc[i][j]));
    }
  };
  auto mma_group = [&](int g) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) mma(i, af[g & 1][i], g, g & 1);
  };
  constexpr int S = G * C::FM;
  static_assert(G % 2 == 0 && S % 2 == 0, "register-set parities carry across tiles");

  // Multi-buffered K loop with one barrier per K tile.  While tile kt is multiplied, the copies
  // of tiles kt+1 .. kt+S-1 are in flight.  The barrier sits before the tile's last multiplies:
  // by then every wave holds their fragments and has finished reading tile kt's buffers, so
  // right after the barrier those buffers are refilled (tile kt+S) and the first fragments of
  // tile kt+1 are read while the last multiplies of tile kt keep the matrix cores busy.  A wave's
  // copies land in the order they were issued, so "tile kt+1 has landed" is a bound on the
  // number of its copies still outstanding (vmcnt): those of the tiles issued after it.
  //
  // MX scales: the piece of scale rows covering tiles c*TPC .. c*TPC+TPC-1 ("chunk" c, buffer
  // c & 1) is copied just before the data of tile c*TPC, so waiting for that tile covers it.
  // Its buffer last served tiles up to (c-1)*TPC - 1, whose scale reads precede the barrier of
  // boundary (c-1)*TPC - 1, and chunk c is issued at boundary c*TPC - S >= (c-1)*TPC - 1.
  // K tiles.  With the K loop split, group kg takes tiles kg, kg + KS, ... (KT of them) in NI
  // iterations that every group runs, so that all reach the same barriers; the loop below
  // counts iterations, which are tiles when KS = 1.
  // With the K loop split across workgroups (SK = 2), part h takes the K tiles
  // [h KH, min((h+1) KH, KT_ALL)), KH = ceil(KT_ALL / 2).
  // With stream-K the segment's K tiles [sg.kb, sg.ke).
  const int KT_ALL = (p.K + C::BKE - 1) / C::BKE;
  const int KH = C::SK > 1 ? (KT_ALL + C::SK - 1) / C::SK : KT_ALL;
  const int kbeg = C::SK == 0 ? sg.kb : khalf * KH;
  const int KT_SK = C::SK == 0 ? sg.ke - sg.kb : C::SK > 1 ? max(0, min(KH, KT_ALL - kbeg)) : KT_ALL;
  const int NI = C::KS == 1 ? KT_SK : (KT_ALL + C::KS - 1) / C::KS;
  const int KT = C::KS == 1 ? KT_SK : (KT_ALL - kg + C::KS - 1) / C::KS;
  auto tile_of = [&](int i) { return C::KS == 1 ? kbeg + i : i * C::KS + kg; };
  const bool need_fix = (p.epi & (FIX_A | FIX_B)) != 0;
  constexpr int NL = OA::PER_WAVE + (C::QB ? 0 : OB::PER_WAVE);  // data copies per copying wave per K tile
  const int nl = copier ? NL : 0;                                 // ... by this wave
  constexpr int NWL = (C::BM + C::BN) / 64;         // 64-row scale wave-loads per chunk
  constexpr int SPW = NWL > C::NCW ? NWL / C::NCW : 1;  // ... issued by each copying wave
  static_assert(!C::MX || ((NWL % C::NCW == 0 || C::NCW % NWL == 0) && C::TPC + 1 >= C::S),
                "the scale copies share evenly among the copying waves; chunk buffers free in time");
  const int nsc = copier ? SPW : 0;                 // scale copies per chunk by this wave
  auto issue_scales = [&](int c) {
    // copying wave w copies 64 rows per wave-load (w, w + NCW, ...; mod NWL, so extra waves
    // repeat a copy, writing the same bytes): row r of op(A) (then of op(B)) gives its 16 scale
    // bytes from block 16 c on
    if (!copier) return;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int u = (int)((cw_u + C::NCW * j) % NWL);
      const uint32_t l = (uint32_t)reinterpret_cast<uintptr_t>(smem + C::SC_OFF + (c & 1) * C::SC_BUF) + u * 1024;
      if (64 * u < C::BM) {
        const int64_t bytes = (int64_t)p.M * p.ldsa;
        const i32x4 r = make_rsrc(p.sa, (uint32_t)(bytes < 0xfffffff0LL ? bytes : 0xfffffff0LL) & ~15u);
        buffer_load_lds16(r, l, (uint32_t)((int64_t)(m0 + 64 * u + lane) * p.ldsa + 16 * c));
      } else {
        const int64_t bytes = (int64_t)p.N * p.ldsb;
        const i32x4 r = make_rsrc(p.sb, (uint32_t)(bytes < 0xfffffff0LL ? bytes : 0xfffffff0LL) & ~15u);
        buffer_load_lds16(r, l, (uint32_t)((int64_t)(n0 + 64 * u - C::BM + lane) * p.ldsb + 16 * c));
      }
    }
  };
  auto issue = [&](int it, int buf) {  // the tile of iteration it
    const int kt = tile_of(it);
    if constexpr (C::MX)
      if (kt % C::TPC == 0) issue_scales(kt / C::TPC);
    if constexpr (!C::QB) issue_b(kt, buf);
    issue_a(kt, buf);
  };
  // Copies a wave issues for tiles t0 .. t1 (each tile's data, and its chunk of scales first).
  auto copies = [&](int t0, int t1) {
    int n = 0;
    for (int t = t0; t <= t1; ++t) n += nl + ((C::MX && t % C::TPC == 0) ? nsc : 0);
    return n;
  };
  constexpr int MAXC = (C::S - 1) * (NL + (C::MX ? SPW : 0));
  static_assert(MAXC < 64, "outstanding-copy counts fit the 6-bit vmcnt");
  // With copying waves and the grouped schedule (16- and 32-bit inputs, two stages), a copying
  // wave issues a tile's A copies at the boundary and its B copies only after the next tile's
  // first k-group: the 16 copies at once kept it at the address unit for about 1060 cycles per
  // tile (about 60 B per clock per compute unit), during which its partner was the only wave
  // on the SIMD with multiplies to issue and could not hide its own fragment reads.  The B
  // copies still land a good half tile before the boundary that waits for them.
  constexpr bool DEFER_B = C::NCW < C::NW && GROUPED && !C::MX && C::QB == 0 && C::S == 2;
#ifdef GEMM_DEBUG_POISON_LDS
  // Race check (a debug build of the library): a stage about to be refilled is first
  // overwritten with all-ones words, a NaN in every floating-point type staged here (a wrong
  // value in the 4- and 6-bit ones), between two barriers.  A fragment read of a stage before
  // its copies have landed, or of a tile's stage after its refill began, then reads the poison
  // instead of stale data that may happen to be right, and the result differs from the
  // library's own.  Only the data stages are poisoned (not the MX scale rows).
  auto poison_stage = [&](int buf) {
    const int gt = tid % (C::NW * 64);
    uint8_t* const a = gsm + OA::LDS_OFF + buf * C::A_BYTES;
    uint8_t* const b = gsm + OB::LDS_OFF + buf * C::B_BYTES;
    for (int o = gt * 16; o < C::A_BYTES; o += C::NW * 64 * 16)
      *reinterpret_cast<u32x4*>(a + o) = u32x4{~0u, ~0u, ~0u, ~0u};
    for (int o = gt * 16; o < C::B_BYTES; o += C::NW * 64 * 16)
      *reinterpret_cast<u32x4*>(b + o) = u32x4{~0u, ~0u, ~0u, ~0u};
  };
#endif
  auto tile_boundary = [&](int kt, int abuf, int anext) {
    // tiles kt+2 .. min(kt+S-1, KT-1) may stay in flight
    wait_vm<0, MAXC>(copies(kt + 2, min(kt + C::S - 1, KT - 1)));
    if (kt + 2 == KT && need_fix && tile_of(kt + 1) == KT_ALL - 1) fixup(tile_of(kt + 1), anext, anext);
    __syncthreads();
#ifdef GEMM_DEBUG_POISON_LDS
    if (kt + C::S < KT) poison_stage(abuf);
    __syncthreads();  // outside the condition: the groups of a split K loop count tiles apart
#endif
    if (kt + C::S < KT) {  // into the buffers tile kt has released
      if constexpr (DEFER_B) issue_a(tile_of(kt + C::S), abuf);
      else issue(kt + C::S, abuf);
    }
  };
  // Quantized B.  Thread t dequantises the 32 codes k0 + 32 (t % 2) .. +31 of row t / 2 of the
  // B tile (one 16-byte code chunk at 4 bits, two at 8), one group (group % 32 == 0): w =
  // fma(s, q, o) in fp32, rounded once to the 16-bit type, written as four 16-byte chunks of
  // the K-contiguous B layout above.  The codes of K tile u are loaded into registers at the
  // boundary after tile u-3 and dequantised during tile u-1 (part i, 8 codes, after k-group i),
  // into the buffer tile u-2 released: their load has a whole tile to land, and the stores
  // are published by the barrier ending tile u-1.
  struct QCodes {
    u32x4 w[C::QB == 8 ? 2 : 1];
    uint32_t s, o;
  };
  const int qrow = tid >> 1, qh = tid & 1;
  auto qload = [&](int u) {
    QCodes q{};
    if constexpr (C::QB != 0) {
      // rows past N feed only columns that are not stored: read any valid row instead
      const int64_t n = min(n0 + qrow, p.N - 1);
      const bool ok = qrow < C::BN && u < KT;
      const int64_t k = ok ? (int64_t)u * C::BKE + 32 * qh : 0;
      const uint8_t* src = Bg + n * p.ldb + k * C::QB / 8;
#pragma unroll
      for (int i = 0; i < (C::QB == 8 ? 2 : 1); ++i) q.w[i] = *reinterpret_cast<const u32x4*>(src + 16 * i);
      const int64_t g = n * p.ldg + k / p.group;
      q.s = reinterpret_cast<const uint16_t*>(p.qs)[g];
      q.o = reinterpret_cast<const uint16_t*>(p.qo)[g];
    }
    return q;
  };
  auto qstore_part = [&](const QCodes& q, int buf, int i) {
    if constexpr (C::QB != 0) {
      if (qrow >= C::BN) return;
      const float sc = C::DT == BF16 ? bf16_bits_to_float(q.s) : f16_bits_to_float(q.s);
      const float of = C::DT == BF16 ? bf16_bits_to_float(q.o) : f16_bits_to_float(q.o);
      float w[8];
      if constexpr (C::QB == 4) {
        const uint32_t d = q.w[0][i];
        const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;  // even / odd codes
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[2 * e] = fmaf(sc, (float)((lo >> (8 * e)) & 255u), of);
          w[2 * e + 1] = fmaf(sc, (float)((hi >> (8 * e)) & 255u), of);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dw = 2 * i + e / 4;
          w[e] = fmaf(sc, (float)((q.w[dw / 4][dw % 4] >> (8 * (e % 4))) & 255u), of);
        }
      }
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (C::DT == BF16) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          typedef float f32x2_t __attribute__((ext_vector_type(2)));
          h[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{w[2 * e], w[2 * e + 1]}), bf16x2_t));
        } else {
          h[e] = float_to_f16_bits(w[2 * e]) | (float_to_f16_bits(w[2 * e + 1]) << 16);
        }
      }
      const int c = 4 * qh + i;  // 8-element chunk of the 64-element K tile
      *reinterpret_cast<u32x4*>(smem + OB::LDS_OFF + buf * C::B_BYTES + qrow * 128 +
                                ((c ^ OB::kswz(qrow)) << 4)) = u32x4{h[0], h[1], h[2], h[3]};
    }
  };
  QCodes qcur{}, qnext{};  // codes of tiles kt+1 and kt+2 during tile kt
  // Makes the codes' registers ready at this point (the compiler waits for their loads here).
  auto qpin = [&](QCodes& q) {
#pragma unroll
    for (int i = 0; i < (C::QB == 8 ? 2 : 1); ++i) asm volatile("" : "+v"(q.w[i]));
    asm volatile("" : "+v"(q.s), "+v"(q.o));
  };
  // Prologue: copies of tiles 0 .. S-1, then wait for tile 0.
#ifdef GEMM_DEBUG_POISON_LDS
#pragma unroll
  for (int t = 0; t < C::S; ++t) poison_stage(t);
  __syncthreads();
#endif
  if constexpr (C::QB != 0) {
    const QCodes q0 = qload(0);
    qcur = qload(1);
    qnext = qload(2);
#pragma unroll
    for (int i = 0; i < 4; ++i) qstore_part(q0, 0, i);
  }
#pragma unroll
  for (int t = 0; t < C::S; ++t)
    if (t < KT) issue(t, t);
  wait_vm<0, MAXC>(copies(1, min(C::S - 1, KT - 1)));
  if (KT == 1 && need_fix && tile_of(0) == KT_ALL - 1) fixup(tile_of(0), 0, 0);
  __syncthreads();
  int abuf = 0;  // buffer of tile kt (kt % S)
  if constexpr (GROUPED) {
    if (KT > 0) load_group(0, 0, 0, 0, 0);
    for (int kt = 0; kt < NI; ++kt) {
      next_tile_scales(kt);
      const bool work = C::KS == 1 || kt < KT;  // a split group may have one tile fewer
      const uint32_t aoff = abuf * C::A_BYTES, boff = abuf * C::B_BYTES;
      const int anext = abuf + 1 == C::S ? 0 : abuf + 1;
#pragma unroll
      for (int g = 0; g + 1 < G; ++g) {
        // Ask the scheduler to interleave this k-group's multiplies with the next group's LDS
        // reads (LLVM's MFMA / DS-read interleaving strategy 1).  At 4096^3 this is 4% faster
        // while the clock holds (constant operands) and neutral on random operands, where the
        // chip runs near 2.1 GHz.
        if (work) {
          // (not with the K split: the compiler's interleaving search runs out of memory on
          // those instantiations)
          if constexpr (C::KS == 1) __builtin_amdgcn_iglp_opt(1);
          load_group(kt, aoff, boff, g + 1, (g + 1) & 1);
          mma_group(g);
        }
        // the deferred B copies of tile kt + 1, into the buffer tile kt - 1 released
        if constexpr (DEFER_B)
          if (g == 0 && kt >= 1 && kt + 1 < KT) issue_b(tile_of(kt + 1), anext);
        if constexpr (C::QB != 0)
          if (kt + 1 < KT) qstore_part(qcur, anext, g);
      }
      if constexpr (C::QB != 0) {
        static_assert(!C::QB || G == 4, "four 8-code parts per K tile");
        if (kt + 1 < KT) qstore_part(qcur, anext, G - 1);
        // Rotate before the boundary's own wait for every outstanding copy.  The compiler
        // cannot count the inline-assembly copies, so a wait for the codes placed after the
        // boundary would also wait for the copies the boundary has just issued.
        qcur = qnext;
        qpin(qcur);
      }
      tile_boundary(kt, abuf, anext);
      if constexpr (C::QB != 0) qnext = qload(kt + 3);
      if (kt + 1 < KT) load_group(kt + 1, anext * C::A_BYTES, anext * C::B_BYTES, 0, 0);
      if (work) mma_group(G - 1);
      abuf = anext;
    }
  } else {
    static_assert(C::KS == 1, "K split with the grouped schedule only");
    if (KT > 0) {
      load_b(0, 0, 0);
      load_a(0, 0, 0, af[0][0]);
      read_tile_scales(0);
    }
    for (int kt = 0; kt < KT; ++kt) {
      next_tile_scales(kt);
      const uint32_t aoff = abuf * C::A_BYTES, boff = abuf * C::B_BYTES;
      const int anext = abuf + 1 == C::S ? 0 : abuf + 1;
#pragma unroll
      for (int st = 0; st < S; ++st) {
        const int g = st / C::FM, i = st % C::FM;
        if (i == 0 && g > 0) load_b(boff, g, 0);
        if (st + 1 < S) {
          load_a(aoff, (st + 1) / C::FM, (st + 1) % C::FM, af[(st + 1) & 1][0]);
          mma(i, af[st & 1][0], g, 0);
        } else {
          tile_boundary(kt, abuf, anext);
          if (kt + 1 < KT) {
            load_a(anext * C::A_BYTES, 0, 0, af[0][0]);
            read_tile_scales(kt + 1);
          }
          mma(i, af[st & 1][0], g, 0);
          // the single B set is still read by the last step: refill it only afterwards
          if (kt + 1 < KT) load_b(anext * C::B_BYTES, 0, 0);
        }
      }
      abuf = anext;
    }
  }

  if constexpr (C::KS > 1) {
    // K split: groups 1 .. KS-1 hand their accumulators to group 0 through LDS (wave by wave,
    // float4 by float4, consecutive lanes 16 bytes apart), which adds them and stores.
    constexpr int NF = C::FM * C::FN * 4;  // float4 pieces per lane
    float4* const part = reinterpret_cast<float4*>(smem);
    __syncthreads();  // every group is done with its stages
    if (kg > 0) {
      float4* dst = part + ((kg - 1) * C::NW + wave) * NF * 64 + lane;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[((i * C::FN + j) * 4 + q) * 64] =
                float4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int h = 1; h < C::KS; ++h) {
      const float4* src = part + ((h - 1) * C::NW + wave) * NF * 64 + lane;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = src[((i * C::FN + j) * 4 + q) * 64];
            acc[i][j][4 * q] += v.x;
            acc[i][j][4 * q + 1] += v.y;
            acc[i][j][4 * q + 2] += v.z;
            acc[i][j][4 * q + 3] += v.w;
          }
    }
  }

  if constexpr (C::SK > 1) {
    // K split across two workgroups: the pair protocol.  Per tile, a counter and a flag in the
    // workspace (both zero before the first call; every call leaves the counter even and the
    // flag at counter / 2).  The counter's old value decides the roles: even, this workgroup is
    // first and publishes its fp32 accumulators; odd, it is second, waits for the first one's
    // flag, adds them and runs the epilogue.  The wait is only ever for a workgroup that has
    // already left its K loop (it took the counter first), whose remaining work is its stores
    // and its flag, so it needs nothing else to run and the wait ends: no co-residency of the
    // grid is assumed.  The spin is bounded all the same.  fp32 addition is commutative, so the
    // result is the same whichever workgroup arrives first.
    // Coherence across the compute units (and the XCDs, whose L2 caches are not coherent with
    // one another) comes from the accesses themselves: the partial sums are stored and loaded
    // at device scope (the sc1 cache policy: no stale line in a per-CU or per-XCD cache serves
    // them), the stores are complete (vmcnt 0) before the flag is raised, and the flag and the
    // counter are device-scope atomics.  That avoids a release / acquire fence, which here would
    // write the whole L2 back and invalidate it under every workgroup still at work on the XCD.
    __shared__ uint32_t sk_old;
    static_assert(256 + C::BM * C::BN * 4 == kSplitSlotBytes, "one workspace slot per tile");
    uint8_t* const slot = p.sk_ws + (int64_t)tile_id * kSplitSlotBytes;
    uint32_t* const sync = reinterpret_cast<uint32_t*>(slot);  // [counter, flag]
    constexpr int NF = C::FM * C::FN * 4;                      // float4 pieces per lane
    constexpr int DEVICE_SCOPE = 16;                           // sc1 cache-policy bit
    const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
        slot + 256, (short)0, C::BM * C::BN * 4, BUFFER_FLAGS);
    const int pbase = (wave * NF * 64 + lane) * 16;            // this lane's first piece, bytes
    __syncthreads();  // every wave has left the K loop
    if (tid == 0) sk_old = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t old = sk_old, round = (old >> 1) + 1u;
    if ((old & 1u) == 0u) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), part,
                                                   pbase + ((i * C::FN + j) * 4 + q) * 64 * 16, 0, DEVICE_SCOPE);
          }
      wait_vmcnt<0>();  // this wave's stores are complete
      __syncthreads();
      if (tid == 0) __hip_atomic_store(sync + 1, round, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (tid == 0) {
      for (uint32_t n = 0; n < (1u << 22); ++n) {
        if (__hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == round) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();  // the loads below are issued after the flag was seen
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(part, pbase + ((i * C::FN + j) * 4 + q) * 64 * 16, 0,
                                                          DEVICE_SCOPE));
          acc[i][j][4 * q] += v[0];
          acc[i][j][4 * q + 1] += v[1];
          acc[i][j][4 * q + 2] += v[2];
          acc[i][j][4 * q + 3] += v[3];
        }
  }

  if constexpr (C::SK == 0) {
    // Stream-K: the parts of a split tile meet through the workspace.  Per tile, an [arrive,
    // done] pair of counters (both zero between calls).  Each part takes a ticket from
    // `arrive` when it leaves its K loop.  Every part but the last to arrive publishes its fp32
    // accumulators in its own slot and counts itself in `done`; the last one waits until
    // `done` shows all the others, adds their sums and runs the epilogue.  So the wait is only
    // ever for parts that have already left their K loops and have only their stores and one
    // atomic left: no co-residency of the grid is assumed, and the spin is bounded all the
    // same.  The sum runs in part order whichever part arrives last (((p0 + p1) + p2) + ...;
    // a last arriver that is not part 0 publishes its own sums too and reads them back), so the
    // result is the same bits on every run.  The last arriver then sets both counters back to
    // zero: every part has already counted itself in both.  Coherence as in the pair protocol
    // above: device-scope (sc1) stores and loads of the sums, stores complete before `done`
    // moves, device-scope atomics for the counters.
    if (sg.parts > 1) {
      __shared__ uint32_t sk_ticket;
      constexpr int64_t SLOT = (int64_t)C::BM * C::BN * 4;
      static_assert(SLOT == kStreamSlotBytes, "one workspace slot holds a tile's fp32 sums");
      // The segment's numbers and the ticket are workgroup-uniform: read them into scalar
      // registers, so that the slots' buffer descriptors are scalar and every load and store
      // below is issued back to back (the compiler otherwise wrapped each in a loop over the
      // lanes' descriptors, one access in flight at a time).
      const int part = __builtin_amdgcn_readfirstlane(sg.part);
      const int parts = __builtin_amdgcn_readfirstlane(sg.parts);
      const int first_w = __builtin_amdgcn_readfirstlane(sg.first_w);
      const int tile = __builtin_amdgcn_readfirstlane(sg.tile);
      uint32_t* const cnt = reinterpret_cast<uint32_t*>(p.sk_ws + p.sk_cnt_off) + 2 * (int64_t)tile;
      constexpr int NF = C::FM * C::FN * 4;  // float4 pieces per lane
      constexpr int DEVICE_SCOPE = 16;       // sc1 cache-policy bit
      const int pbase = (wave * NF * 64 + lane) * 16;
      auto slot_rsrc = [&](int q) {
        return __builtin_amdgcn_make_buffer_rsrc(p.sk_ws + sk_slot(first_w, q) * SLOT, (short)0,
                                                 (int)SLOT, BUFFER_FLAGS);
      };
      __syncthreads();  // every wave has left the K loop
      if (tid == 0) sk_ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const bool last = __builtin_amdgcn_readfirstlane(sk_ticket) == (uint32_t)(parts - 1);
      if (!last || part != 0) {
        const __amdgpu_buffer_rsrc_t own = slot_rsrc(part);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 v = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), own,
                                                     pbase + ((i * C::FN + j) * 4 + q) * 64 * 16, 0, DEVICE_SCOPE);
            }
        wait_vmcnt<0>();  // this wave's stores are complete
        __syncthreads();
        if (!last) {
          if (tid == 0) __hip_atomic_fetch_add(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
      }
      if (tid == 0) {
        for (uint32_t n = 0; n < (1u << 22); ++n) {
          if (__hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(parts - 1)) break;
          __builtin_amdgcn_s_sleep(2);
        }
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();  // the loads below are issued after the count was seen
      // one accumulator row (FN x 4 pieces) of loads in flight before its adds
      for (int k = part == 0 ? 1 : 0; k < parts; ++k) {
        const __amdgpu_buffer_rsrc_t src = slot_rsrc(k);
#pragma unroll
        for (int i0 = 0; i0 < C::FM; i0 += 2) {
          f32x4 v[2][C::FN][4];
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              v[ii][j][q] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(src, pbase + (((i0 + ii) * C::FN + j) * 4 + q) * 64 * 16, 0,
                                                              DEVICE_SCOPE));
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[i0 + ii][j][4 * q + e] = k == 0 ? v[ii][j][q][e] : acc[i0 + ii][j][4 * q + e] + v[ii][j][q][e];
        }
      }
    }
  }

  // Epilogue in registers.  Lane (lrow, lhalf) of accumulator (i, j) holds rows
  // m = m0 + wm*WTM + 32 i + lrow and, in register group rg, the 4 consecutive columns
  // n = n0 + wn*WTN + 32 j + 8 rg + 4 lhalf (+0..3).
  const bool full = (m0 + C::BM <= p.M) && (n0 + C::BN <= p.N);
  const float alpha = p.alpha, beta = p.beta;
  const uint32_t epi = p.epi & (EPI_BIAS | EPI_GELU);
  const int mw = m0 + wm * C::WTM + lrow;
  const int nw = n0 + wn * C::WTN + lhalf * 4;
  {
    // Interior tiles carry no masks.  The bias values of the lane's columns are fetched in one
    // batch (a single wait), each row's C values (beta != 0) likewise, and the element loop is
    // specialised on (beta != 0, GELU, edge) so that it carries no branches: this loop runs on
    // the vector ALUs after the last multiply, so every instruction in it is paid in full.
    // Edge tiles (past M or N) take the same path with masked bias and C loads and masked
    // stores, so that their stores are full granules too wherever the granule lies inside.
    // With GELU and a 16-bit output the element loop computes y = x / 2 (alpha, beta and the
    // bias halved, an exact scaling) and gelu16_half(y).
    const bool half = C::CT != F32 && (epi & EPI_GELU);
    const float hs = half ? 0.5f : 1.0f;
    float bj[C::FN][4][4];
    if (full) {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          // four scalar loads (the bias need only be 4-byte aligned); they merge into one
#pragma unroll
          for (int e = 0; e < 4; ++e) bj[j][rg][e] = (epi & EPI_BIAS) ? hs * p.bias[nw + 32 * j + 8 * rg + e] : 0.0f;
        }
    } else {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = nw + 32 * j + 8 * rg + e;
            bj[j][rg][e] = ((epi & EPI_BIAS) && n < p.N) ? hs * p.bias[n] : 0.0f;
          }
    }
    const float alpha_e = hs * alpha, beta_e = hs * beta;
    // Output staging.  In the accumulator layout one store instruction would write 32 rows x
    // 16 bytes, 32 partial cache lines that L2 merges one request at a time.  Instead each wave
    // writes one row of accumulator tiles (32 x WTN outputs) into a private LDS region in that
    // layout, reads it back as whole 16-byte granules along the rows and stores full lines.
    // The K loop's buffers are free here: every wave has passed the last tile's barrier, after
    // which LDS is not read, and no copy is in flight.  Granule g of staged row r sits at
    // position g ^ (r % GPR), which keeps the row-wise read-back free of bank conflicts.
    constexpr int OES = C::CT == F32 ? 4 : 2;           // output element bytes
    constexpr int EPG = 16 / OES;                        // elements per granule
    constexpr int ROWB = C::WTN * OES, GPR = ROWB / 16;  // staged row bytes, granules per row
    constexpr int CHUNK = 32 * ROWB;                      // one wave's region
    static_assert(C::STG_OFF + C::NW * CHUNK <= C::LDS_BYTES, "output staging fits the K loop's LDS");
    uint8_t* const ostage = smem + C::STG_OFF + wave_u * CHUNK;
    const int m_w0 = m0 + wm * C::WTM, n_w0 = n0 + wn * C::WTN;
    typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
    auto store_tile = [&](auto has_beta, auto has_gelu, auto is_edge) {
      constexpr bool HB = decltype(has_beta)::value, HG = decltype(has_gelu)::value;
      constexpr bool EDGE = decltype(is_edge)::value;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int m = mw + 32 * i;                     // this lane's row (beta != 0 loads)
        const int64_t row = (int64_t)m * p.ldc;
        float cin[C::FN][4][4];
        if constexpr (HB) {
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int n = nw + 32 * j + 8 * rg;
              const int64_t idx = row + n;
              if (EDGE && !(m < p.M && n + 3 < p.N)) {
                // a run of four that leaves the matrix: element by element
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  cin[j][rg][e] = (m < p.M && n + e < p.N) ? load_as_float<C::CT>(p.C, idx + e) : 0.0f;
              } else if constexpr (C::CT == F32) {
                const float4 c4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.C) + idx);
                cin[j][rg][0] = c4.x; cin[j][rg][1] = c4.y; cin[j][rg][2] = c4.z; cin[j][rg][3] = c4.w;
              } else {
                const u32x2 c2 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(p.C) + idx);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const uint32_t h = (c2[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                  cin[j][rg][e] = (C::CT == F16) ? f16_bits_to_float(h) : bf16_bits_to_float(h);
                }
              }
            }
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = fmaf(alpha_e, acc[i][j][rg * 4 + e], bj[j][rg][e]);
              if constexpr (HB) x = fmaf(beta_e, cin[j][rg][e], x);
              if constexpr (HG) {
                if constexpr (C::CT == F32) x = gelu_out<C::CT>(x);
                else x = gelu16_half(x);
              }
              v[e] = x;
            }
            const int gb = (32 * j + 8 * rg + 4 * lhalf) * OES;  // byte offset in the row
            stage4<C::CT>(ostage + lrow * ROWB + 16 * ((gb >> 4) ^ (lrow % GPR)) + (gb & 15), v);
          }
        // read back whole granules: linear granule L = 64 q + lane is row L / GPR, granule L % GPR
#pragma unroll
        for (int q = 0; q < GPR / 2; ++q) {
          const int L = 64 * q + lane, r = L / GPR, g = L % GPR;
          const u32x4 val = *reinterpret_cast<const u32x4*>(ostage + r * ROWB + 16 * (g ^ (r % GPR)));
          const int gm = m_w0 + 32 * i + r, gn = n_w0 + g * EPG;
          uint8_t* dst = reinterpret_cast<uint8_t*>(p.C) + ((int64_t)gm * p.ldc + gn) * OES;
          if (!EDGE || (gm < p.M && gn + EPG <= p.N)) {
            // non-temporal: C is not read again here, and lines the L2 does not keep dirty
            // need no write-back when the kernel ends (1.3 us less per 4096^3 launch)
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4_a4*>(dst));
          } else if (gm < p.M && gn < p.N) {
            // the granule that straddles column N: its elements up to N one by one
            for (int e = 0; e < p.N - gn; ++e) {
              if constexpr (OES == 4) reinterpret_cast<uint32_t*>(dst)[e] = val[e];
              else reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(val[e >> 1] >> ((e & 1) * 16));
            }
          }
        }
      }
    };
    auto store_any = [&](auto is_edge) {
      if (beta != 0.0f) {
        if (epi & EPI_GELU) store_tile(std::true_type{}, std::true_type{}, is_edge);
        else store_tile(std::true_type{}, std::false_type{}, is_edge);
      } else {
        if (epi & EPI_GELU) store_tile(std::false_type{}, std::true_type{}, is_edge);
        else store_tile(std::false_type{}, std::false_type{}, is_edge);
      }
    };
    if (full) store_any(std::false_type{});
    else store_any(std::true_type{});
  }
}

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_mfma_kernel(GemmParams p) {
  if constexpr (C::SK != 0) {
    mfma_tile<C>(p, SkSeg{});
  } else {
    // Stream-K: a persistent grid of G workgroups shares out the I = tiles x KT K tiles of the
    // product, workgroup L taking the run [floor(L I / G), floor((L+1) I / G)) of the tile-major
    // sequence (output tile t owns K tiles [t KT, (t+1) KT)) and walking it segment by segment,
    // one output tile at a time.  K tile x belongs to workgroup floor(((x+1) G - 1) / I), which
    // gives every segment its tile's contributors.  Workgroups are renumbered as for the other
    // kernels, so that each XCD takes a contiguous range of runs: the parts of a tile mostly
    // meet in one XCD's L2.
    // Registers: held across segments, the run's bounds and the body's loop-invariant offsets
    // made the kernel spill inside its K loop.  So the run's state lives in LDS (read again
    // after each segment, whose barriers order it), and each segment recomputes its lane index
    // (an opaque instruction, below), so that what derives from it is not kept from one segment
    // to the next.  What still spills (a few scalars and three words per lane) is read once per
    // segment, outside the K loop.
    // (One workgroup per segment instead, in rounds, needs no loop and spills nothing, but the
    // dispatcher then hands the later segments out unevenly: measured 3072 x 4096 x 4096 150 us
    // against 117 us persistent.)
    __shared__ int64_t run[4];  // [next K tile, end of the run, I, G | L << 32]
    if (threadIdx.x == 0) {
      const int G = (int)gridDim.x;
      int L = (int)blockIdx.x;
      if ((G & 7) == 0) L = (L & 7) * (G >> 3) + (L >> 3);
      const int64_t I = (int64_t)p.tiles_m * p.tiles_n * ((p.K + C::BKE - 1) / C::BKE);
      run[0] = (int64_t)L * I / G;
      run[1] = (int64_t)(L + 1) * I / G;
      run[2] = I;
      run[3] = (int64_t)G | ((int64_t)L << 32);
    }
    __syncthreads();
    for (;;) {
      const int64_t it = run[0], end = run[1], I = run[2];
      const int G = (int)(run[3] & 0xffffffff), L = (int)(run[3] >> 32);
      if (it >= end) break;
      const int KT = (p.K + C::BKE - 1) / C::BKE;
      const int t = (int)(it / KT);
      const int64_t t0 = (int64_t)t * KT;
      const int kb = (int)(it - t0), ke = (int)min((int64_t)KT, end - t0);
      const int w0 = (int)(((t0 + 1) * G - 1) / I), w1 = (int)(((t0 + KT) * G - 1) / I);
      // Every thread has read the position (so that all walk the same segment and meet the
      // same barriers), and the previous segment is done with LDS.
      __syncthreads();
      if (threadIdx.x == 0) run[0] = t0 + ke;  // published by the segment's own barriers
      mfma_tile<C>(p, SkSeg{t, kb, ke, L - w0, w1 - w0 + 1, w0});
    }
  }
}

template <class C>
hipError_t launch_mfma_cfg(GemmParams p, hipStream_t s) {
  const int64_t T = (int64_t)p.tiles_m * p.tiles_n;
  // Last-K-tile fix-ups: a K-contiguous operand whose K is not a whole number of tiles, or an
  // M/N-contiguous operand whose row length is not a whole number of 16-byte chunks.
  constexpr int CE = 16 / C::ES;
  const bool fix_a = C::A_MN ? (p.M % CE != 0) : (p.K % C::BKE != 0);
  const bool fix_b = C::B_MN ? (p.N % CE != 0) : (p.K % C::BKE != 0);
  p.epi |= (fix_a ? FIX_A : 0u) | (fix_b ? FIX_B : 0u);
  // stream-K: a persistent grid of p.sk_grid workgroups (at most one per K tile)
  const int64_t grid = C::SK == 0 ? p.sk_grid : T * C::SK;
  hipLaunchKernelGGL((gemm_mfma_kernel<C>), dim3((unsigned)grid), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// Tile families: 0 -> 64x64 (2x2 waves of 32x32), 1 -> 128x128 (2x2 waves of 64x64; two such
// groups splitting K for 16- and 32-bit inputs), 2 -> 256x256 (2x4 waves of 128x64), 3 -> 32x32
// (four one-wave groups splitting K; 16- and 32-bit inputs).  BT: type of B (differs from A only in the 8-bit
// family); MX: block-scaled.  Packed fp4 and 6-bit operands are staged K-contiguous only (A
// stored M x K, B stored N x K): the other layouts return an error (the host never routes them
// here).
template <int DT, int TILE, int WM, int WN, int BT, bool MX, int KS = 1, int BN = 0, int SK = 1>
hipError_t launch_mfma_layout(const GemmParams& p, bool a_mn, bool b_mn, hipStream_t s) {
  // a K split gives each group its own stages: two each; the 256-row tiles keep two as well
  constexpr int S = (KS > 1 || BN) ? 2 : default_stages<TILE>();
  if (!a_mn && !b_mn) return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, false, false, S, BT, MX, 0, KS, BN, SK>>(p, s);
  if constexpr (DT == E2M1 || is_fp6<DT>()) {
    return hipErrorInvalidValue;
  } else {
    if (!a_mn && b_mn) return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, false, true, S, BT, MX, 0, KS, BN, SK>>(p, s);
    if (a_mn && !b_mn) return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, true, false, S, BT, MX, 0, KS, BN, SK>>(p, s);
    return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, true, true, S, BT, MX, 0, KS, BN, SK>>(p, s);
  }
}

// ks (64 x 64 tile only, 16- and 32-bit inputs): the K split, 1 or 2 groups of four waves (four
// groups measured no faster than two at 512^3 and 1024^3).
template <int DT, int BT = DT, bool MX = false>
hipError_t launch_mfma_dtype(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s,
                             int ks = 1) {
  if constexpr (DT == F32 || DT == F16 || DT == BF16) {
    if (tile == 0 && ks == 2) return launch_mfma_layout<DT, 64, 2, 2, BT, MX, 2>(p, a_mn, b_mn, s);
  }
  if (tile == 3) {  // 32 x 32, one wave per K group, four groups (small products)
    if constexpr ((DT == F32 || DT == F16 || DT == BF16) && !MX)
      return launch_mfma_layout<DT, 32, 1, 1, BT, MX, 4>(p, a_mn, b_mn, s);
    else
      return hipErrorInvalidValue;
  }
  if (tile == 5 || tile == 6) {  // 256 x 128, 4 x 2 waves of 64 x 64; 6: K split over two workgroups
    if constexpr ((DT == F16 || DT == BF16) && !MX) {
      if (ks != 1) return hipErrorInvalidValue;
      if (tile == 6) return launch_mfma_layout<DT, 256, 4, 2, BT, MX, 1, 128, 2>(p, a_mn, b_mn, s);
      return launch_mfma_layout<DT, 256, 4, 2, BT, MX, 1, 128, 1>(p, a_mn, b_mn, s);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (tile == 7) {  // 256 x 256, stream-K over a persistent grid
    if constexpr ((DT == F16 || DT == BF16) && !MX) {
      if (ks != 1) return hipErrorInvalidValue;
      return launch_mfma_layout<DT, 256, 2, 4, BT, MX, 1, 0, 0>(p, a_mn, b_mn, s);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (ks != 1) return hipErrorInvalidValue;
  switch (tile) {
    case 0: return launch_mfma_layout<DT, 64, 2, 2, BT, MX>(p, a_mn, b_mn, s);
    case 1:
      // 16- and 32-bit inputs: two groups of four waves split the K loop (two waves per SIMD,
      // so that one covers the other's waits)
      if constexpr ((DT == F32 || DT == F16 || DT == BF16) && !MX)
        return launch_mfma_layout<DT, 128, 2, 2, BT, MX, 2>(p, a_mn, b_mn, s);
      else
        return launch_mfma_layout<DT, 128, 2, 2, BT, MX>(p, a_mn, b_mn, s);
    case 2: return launch_mfma_layout<DT, 256, 2, 4, BT, MX>(p, a_mn, b_mn, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tgemm
