// GEMMs on gfx950's 8/6/4-bit MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) for
// the two formats the pages compare NVFP4 with: MXFP4 and FP8 (E4M3, one
// scale per tensor). C [M][N] = A [M][K] * B [N][K]^T, both operands
// K-contiguous.
//
// Sources: gist.science summary of "Pretraining Large Language Models with
// NVFP4", Resumen técnico §1 (FP8 as the baseline; MXFP4's coarser scales)
// and §2 "Formato NVFP4" (MXFP4 blocks of 32 elements); deultimominuto.info,
// "Cómo funciona NVFP4" (E4M3: 4 exponent, 3 mantissa bits).
//
// The instruction multiplies a 32 x 64 slice of A by a 32 x 64 slice of B:
// lane l supplies row l % 32 and the 32 K values of half l / 32 (16 bytes of
// FP4 codes, 32 bytes of FP8 bytes). With FP4 operands it also takes one
// E8M0 scale per row and 32 K, which is MXFP4's own definition, so codes and
// scale bytes go to the MFMA as stored. FP8 operands take the scale byte 127
// (2^0) and the per-tensor scales multiply C in the epilogue.
//
// Staging: a 256 x 256 C tile per workgroup, 4 waves of 128 x 128 (16
// accumulator tiles of 32 x 32 each). A step moves one whole 128-byte line of
// every A and B row (K = 256 FP4 codes or K = 128 FP8 bytes) into one of two
// LDS stages with direct-to-LDS loads. Whole lines keep the L1-to-L2
// requests at one per line: 64-byte half lines cost a whole line's request
// each, which kept the address and load units busy. The 8 16-byte chunks of
// a 128-byte LDS row are XOR-swizzled by (row >> 1) & 7, so that both the
// DMA (lane j fills slot j % 8 of row j / 8) and the fragment reads of 16
// consecutive rows hit distinct banks. A step holds 4 (FP4) or 2 (FP8) MFMA
// sub-steps of K = 64; a sub-step's MFMAs run while the next sub-step's
// fragments are read from LDS. One barrier per step, before its last
// sub-step, hands the step's stage back to the DMA for the step after next.
//
// K mapping: in a step, lane half h takes K [128 h, 128 h + 128) (FP4) or
// [64 h, 64 h + 64) (FP8) and each sub-step a quarter (FP4) or half (FP8) of
// it, so an FP4 lane's four scale bytes of the step are adjacent: one 32-bit
// LDS read serves the step and op_sel picks the byte. A and B use the same
// mapping, so every MFMA sums matching K. K % 256 == 128 (FP4) or
// K % 128 == 64 (FP8) leaves a last half step (64 bytes per row) whose K is
// mapped in the same way over half the length.
#include <type_traits>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

using namespace gemm_common;

enum class Fmt { kMxFp4, kFp8 };

constexpr int kThreads = 256;
constexpr int kTile = 256;                     // C rows and columns per workgroup
constexpr int kWave = 128;                     // C rows and columns per wave
constexpr int kRowBytes = 128;                 // code bytes per row and step
constexpr int kCodeBytes = kTile * kRowBytes;  // per operand and stage
constexpr int kMxBlock = 32;
constexpr int kDmaLoads = 8;                   // code loads per wave, operand and step (8 rows each)

template <Fmt F>
struct Traits;

template <>
struct Traits<Fmt::kMxFp4> {
  static constexpr int kBK = 256;                   // K elements per step
  static constexpr int kSub = 4;                    // MFMA sub-steps (K = 64) per step
  static constexpr int kChunks = 1;                 // 16-byte chunks per lane and fragment
  static constexpr int kScaleRow = kBK / kMxBlock;  // scale bytes per row and step
  static constexpr int kChunkSteps = 4;             // steps per scale chunk
  static constexpr int kChunkRow = kChunkSteps * kScaleRow;
  static constexpr int kChunkBytes = kTile * kChunkRow;  // per operand
  static __device__ __forceinline__ int64_t row_bytes(int64_t K) { return K >> 1; }
};

template <>
struct Traits<Fmt::kFp8> {
  static constexpr int kBK = 128;
  static constexpr int kSub = 2;
  static constexpr int kChunks = 2;
  static constexpr int kScaleRow = 0;
  static constexpr int kChunkSteps = 1;
  static constexpr int kChunkRow = 0;
  static constexpr int kChunkBytes = 0;
  static __device__ __forceinline__ int64_t row_bytes(int64_t K) { return K; }
};

// LDS: [A codes, stages 0 and 1][B codes][scale buffer 0: A, B][buffer 1]
// (160 KiB for MXFP4). A scale buffer holds a chunk of 4 steps' scale bytes
// (32 per row): loading 8 rows' 32 bytes per instruction instead of 32
// rows' 8 bytes per step touches a quarter as many lines per step.
template <Fmt F>
struct Lds {
  static constexpr int kA = 0;
  static constexpr int kB = 2 * kCodeBytes;
  static constexpr int kSa = 4 * kCodeBytes;
  static constexpr int kSb = kSa + Traits<F>::kChunkBytes;
  static constexpr int kScaleBuf = 2 * Traits<F>::kChunkBytes;  // between the two buffers
  static constexpr int kBytes = kSa + 2 * kScaleBuf;
};

typedef int int8v_t __attribute__((ext_vector_type(8)));

struct BlockGemmParams {
  const uint8_t *qa, *sa, *qb, *sb;  // scales: MXFP4 only
  const float *ta, *tb;              // per-tensor scales: FP8 only
  void* c;
  int64_t M, N, K, ldc;
};

// One operand's loads for this wave: 8 code loads of 8 rows each (lane j of
// load k: tile row 64 w + 8 k + j / 8, the chunk whose swizzled slot is
// j % 8) and, for MXFP4, scale loads of 8 rows each (lane j: the same row,
// 4 bytes of the row's scale chunk). (row >> 1) & 7 = (4 k + j / 16) & 7 for
// these rows. Rows past the matrix read its last row instead (they only feed
// C outside M x N). Addresses are formed with integer minimums, not
// selects: a select on a pointer can become a branch, and a branch in the
// loop let the compiler sink the MFMAs behind the loads.
struct Dma {
  const uint8_t* q;  // operand codes (uniform)
  const uint8_t* s;  // operand scales (uniform; MXFP4)
  int row;          // this lane's row of load 0
  int last;         // the operand's last row
  int64_t rb, srb;   // code and scale bytes per row (uniform)
};

__device__ __forceinline__ int dma_chunk(int k, int lane) { return (lane & 7) ^ ((4 * k + (lane >> 4)) & 7); }

template <Fmt F>
__device__ __forceinline__ Dma dma_setup(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                         int64_t row0, int64_t rows, int64_t K, int wave, int lane) {
  Dma d;
  d.q = q;
  d.s = s;
  d.rb = Traits<F>::row_bytes(K);
  d.srb = K / kMxBlock;
  d.row = static_cast<int>(row0) + 64 * wave + (lane >> 3);
  d.last = static_cast<int>(rows) - 1;
  return d;
}

// Requests step `step` of one operand's codes (this wave's 64 rows) into the
// LDS stage at byte address codes. A half step (64 bytes per row, the last
// step of some K) reads chunk c & 3 for chunk c: the slots of chunks 4-7
// then hold copies that are never read.
template <Fmt F>
__device__ __forceinline__ void dma_step(const Dma& d, uint32_t codes, int step, bool half, int wave,
                                         int lane) {
  const int64_t off = static_cast<int64_t>(step) * kRowBytes;
  const uint32_t c0 = codes + 64 * wave * kRowBytes;
  const int cmask = half ? 3 : 7;
#pragma unroll
  for (int k = 0; k < kDmaLoads; ++k) {
    const int row = min(d.row + 8 * k, d.last);
    const int c = dma_chunk(k, lane) & cmask;
    lds_dma<16>(d.q + static_cast<int64_t>(row) * d.rb + off + 16 * c, c0 + k * (8 * kRowBytes));
  }
}

// Step `step` of A's and B's codes into stage step % 2; a half step when
// step is the last and K leaves half a step.
template <Fmt F>
__device__ __forceinline__ void dma_both(const Dma& da, const Dma& db, uint32_t lds, int step, bool half,
                                         int wave, int lane) {
  using L = Lds<F>;
  const int st = step & 1;
  dma_step<F>(da, lds + L::kA + st * kCodeBytes, step, half, wave, lane);
  dma_step<F>(db, lds + L::kB + st * kCodeBytes, step, half, wave, lane);
}

// Scale words in LDS: a row's 32-byte chunk holds its eight 4-byte words
// (two per step) with word w at position w ^ scale_swizzle(row), so that the
// 64 lanes of a scale read (32 rows, two words each) fall in 64 distinct
// banks instead of eight rows sharing each bank.
__device__ __forceinline__ int scale_swizzle(int row) { return 2 * ((row >> 3) & 3); }
static_assert(Traits<Fmt::kMxFp4>::kChunkRow == 32 && Traits<Fmt::kMxFp4>::kScaleRow == 8,
              "eight 4-byte words per row chunk, two per step: the swizzle stays inside the chunk");

// Load k (k = 2 q + e) of a wave's scale chunk fills rows 64 w + 8 k .. + 7;
// lane j lands in position j % 8 of row 64 w + 8 k + j / 8 and so fetches
// word (j % 8) ^ scale_swizzle(8 k) of the chunk. A word past the row's K / 32
// (the last chunk of a K that is not a multiple of 1024) reads the row's
// first bytes instead: no step reads it.
__device__ __forceinline__ int64_t scale_src(const Dma& d, int chunk, int k, int lane) {
  constexpr int kRow = Traits<Fmt::kMxFp4>::kChunkRow;
  const int64_t want = static_cast<int64_t>(chunk) * kRow + 4 * ((lane & 7) ^ scale_swizzle(8 * k));
  return want + 4 <= d.srb ? want : 0;
}

// Quarter q (loads 2q and 2q + 1, 16 rows of this wave's 64) of scale chunk
// `chunk` (MXFP4) of one operand into the LDS buffer at byte address buf.
__device__ __forceinline__ void dma_scale_quarter(const Dma& d, uint32_t buf, int chunk, int q, int wave,
                                                  int lane) {
  constexpr int kRow = Traits<Fmt::kMxFp4>::kChunkRow;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 16 * q + 8 * e;  // load 2 q + e: rows r .. r + 7 of the wave's 64
    const int row = min(d.row + r, d.last);
    lds_dma<4>(d.s + static_cast<int64_t>(row) * d.srb + scale_src(d, chunk, 2 * q + e, lane),
               buf + (64 * wave + r) * kRow);
  }
}

__device__ __forceinline__ void dma_scales(const Dma& da, const Dma& db, uint32_t lds, int chunk, int q,
                                           int wave, int lane) {
  using L = Lds<Fmt::kMxFp4>;
  const uint32_t buf = (chunk & 1) * L::kScaleBuf;
  dma_scale_quarter(da, lds + L::kSa + buf, chunk, q, wave, lane);
  dma_scale_quarter(db, lds + L::kSb + buf, chunk, q, wave, lane);
}

// Single loads, for interleaving with the MFMAs. A step's loads of one
// operand are the 8 code loads k and, for MXFP4, the two loads e of one
// quarter of a scale chunk; "part 0" of a step's loads is A's codes 0-3,
// B's codes 0-3 and A's scale loads, "part 1" the rest (B's scale loads).
template <Fmt F>
__device__ __forceinline__ void dma_code(const Dma& d, uint32_t operand, int step, bool half, int k, int wave,
                                         int lane) {
  const int st = step & 1;
  const int row = min(d.row + 8 * k, d.last);
  const int c = dma_chunk(k, lane) & (half ? 3 : 7);
  lds_dma<16>(d.q + static_cast<int64_t>(row) * d.rb + static_cast<int64_t>(step) * kRowBytes + 16 * c,
              operand + st * kCodeBytes + (64 * wave + 8 * k) * kRowBytes);
}

__device__ __forceinline__ void dma_scale(const Dma& d, uint32_t operand, int chunk, int q, int e, int wave,
                                          int lane) {
  using L = Lds<Fmt::kMxFp4>;
  constexpr int kRow = Traits<Fmt::kMxFp4>::kChunkRow;
  const int r = 16 * q + 8 * e;
  const int row = min(d.row + r, d.last);
  lds_dma<4>(d.s + static_cast<int64_t>(row) * d.srb + scale_src(d, chunk, 2 * q + e, lane),
             operand + (chunk & 1) * L::kScaleBuf + (64 * wave + r) * kRow);
}

template <int kN>
using IC = std::integral_constant<int, kN>;

template <typename Fn, int... kI>
__device__ __forceinline__ void unroll_impl(Fn&& fn, std::integer_sequence<int, kI...>) {
  (fn(IC<kI>{}), ...);
}

// fn(IC<0>{}), ..., fn(IC<kN - 1>{}) in order.
template <int kN, typename Fn>
__device__ __forceinline__ void unroll(Fn&& fn) {
  unroll_impl(fn, std::make_integer_sequence<int, kN>{});
}

// One sub-step's fragments, each the MFMA operand of one row (column)
// block: 16 bytes per lane for FP4, 32 for FP8 (two chunks read into one
// register tuple).
template <Fmt F>
struct Frags {
  using Frag = typename std::conditional<F == Fmt::kMxFp4, uint4, int8v_t>::type;
  Frag a[4], b[4];
};

// Lane offsets (bytes from the LDS base) of the 4 chunk positions a lane
// reads in a step: q = sub-step (FP4) or 2 sub-step + chunk (FP8), chunk
// 4 h + q of a full step and 2 h + q of a half step, in row block 0 of
// stage 0 of this wave's A (B) rows.
struct FragOffsets {
  int a[4], b[4];
  int sa, sb;  // the lane's scale word (full step) or 16-bit half (half step)
  int sx;      // XOR on a step's byte offset within the row's chunk: 4 scale_swizzle(row)
};

template <Fmt F>
__device__ __forceinline__ FragOffsets frag_offsets(int wm, int wn, int lane, bool half) {
  using L = Lds<F>;
  FragOffsets o;
  const int rl = lane & 31, h = lane >> 5;
  const int swz = (rl >> 1) & 7;  // (row >> 1) & 7 of every row this lane reads
  const int ra = wm * kWave + rl, rb = wn * kWave + rl;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = half ? (2 * h + (q & 1)) : (4 * h + q);
    o.a[q] = L::kA + ra * kRowBytes + 16 * (c ^ swz);
    o.b[q] = L::kB + rb * kRowBytes + 16 * (c ^ swz);
  }
  o.sa = L::kSa + ra * Traits<F>::kChunkRow + (half ? 2 * h : 4 * h);
  o.sb = L::kSb + rb * Traits<F>::kChunkRow + (half ? 2 * h : 4 * h);
  o.sx = 4 * scale_swizzle(rl);  // rows ra and rb (and + 32 i) share it
  return o;
}

template <Fmt F, int kSubStep>
__device__ __forceinline__ void read_frags(Frags<F>& f, const uint8_t* __restrict__ lds, const FragOffsets& o,
                                           int st) {
  constexpr int kC = Traits<F>::kChunks;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* pa = lds + st * kCodeBytes + i * 32 * kRowBytes;
    const uint4 a0 = *reinterpret_cast<const uint4*>(pa + o.a[kSubStep * kC]);
    const uint4 b0 = *reinterpret_cast<const uint4*>(pa + o.b[kSubStep * kC]);
    if constexpr (kC == 2) {
      const uint4 a1 = *reinterpret_cast<const uint4*>(pa + o.a[kSubStep * kC + 1]);
      const uint4 b1 = *reinterpret_cast<const uint4*>(pa + o.b[kSubStep * kC + 1]);
      f.a[i] = int8v_t{static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                       static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                       static_cast<int>(a1.z), static_cast<int>(a1.w)};
      f.b[i] = int8v_t{static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                       static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                       static_cast<int>(b1.z), static_cast<int>(b1.w)};
    } else {
      f.a[i] = a0;
      f.b[i] = b0;
    }
  }
}

// Fragment n (A 0-3, then B 0-3) of sub-step kSubStep of stage st.
template <Fmt F, int kSubStep, int kN>
__device__ __forceinline__ void read_frag(Frags<F>& f, const uint8_t* __restrict__ lds, const FragOffsets& o,
                                          int st) {
  constexpr int kC = Traits<F>::kChunks, i = kN & 3;
  const int* off = kN < 4 ? o.a : o.b;
  const uint8_t* p = lds + st * kCodeBytes + i * 32 * kRowBytes;
  const uint4 v0 = *reinterpret_cast<const uint4*>(p + off[kSubStep * kC]);
  typename Frags<F>::Frag v;
  if constexpr (kC == 2) {
    const uint4 v1 = *reinterpret_cast<const uint4*>(p + off[kSubStep * kC + 1]);
    v = int8v_t{static_cast<int>(v0.x), static_cast<int>(v0.y), static_cast<int>(v0.z), static_cast<int>(v0.w),
                static_cast<int>(v1.x), static_cast<int>(v1.y), static_cast<int>(v1.z), static_cast<int>(v1.w)};
  } else {
    v = v0;
  }
  if constexpr (kN < 4) {
    f.a[i] = v;
  } else {
    f.b[i] = v;
  }
}

// The lane's scale words of step `step` (MXFP4): one 32-bit word per block
// of a full step, one 16-bit half of a half step.
template <bool kHalf>
__device__ __forceinline__ void read_scales(uint32_t (&sa)[4], uint32_t (&sb)[4], const uint8_t* __restrict__ lds,
                                            const FragOffsets& o, int step) {
  using T = Traits<Fmt::kMxFp4>;
  const int soff = ((step / T::kChunkSteps) & 1) * Lds<Fmt::kMxFp4>::kScaleBuf +
                   (((step % T::kChunkSteps) * T::kScaleRow) ^ o.sx);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kHalf) {
      sa[i] = *reinterpret_cast<const uint16_t*>(lds + o.sa + soff + i * 32 * T::kChunkRow);
      sb[i] = *reinterpret_cast<const uint16_t*>(lds + o.sb + soff + i * 32 * T::kChunkRow);
    } else {
      sa[i] = *reinterpret_cast<const uint32_t*>(lds + o.sa + soff + i * 32 * T::kChunkRow);
      sb[i] = *reinterpret_cast<const uint32_t*>(lds + o.sb + soff + i * 32 * T::kChunkRow);
    }
  }
}

// An FP4 operand: 16 bytes in the low half of the operand tuple (the
// instruction reads 4 registers for FP4).
// Scale word n (A blocks 0-3, then B) of step `step` (MXFP4, full step).
template <int kN>
__device__ __forceinline__ void read_scale_word(uint32_t (&sa)[4], uint32_t (&sb)[4], const uint8_t* __restrict__ lds,
                                                const FragOffsets& o, int step, IC<kN>) {
  using T = Traits<Fmt::kMxFp4>;
  const int soff = ((step / T::kChunkSteps) & 1) * Lds<Fmt::kMxFp4>::kScaleBuf +
                   (((step % T::kChunkSteps) * T::kScaleRow) ^ o.sx);
  constexpr int i = kN & 3;
  if constexpr (kN < 4) {
    sa[i] = *reinterpret_cast<const uint32_t*>(lds + o.sa + soff + i * 32 * T::kChunkRow);
  } else {
    sb[i] = *reinterpret_cast<const uint32_t*>(lds + o.sb + soff + i * 32 * T::kChunkRow);
  }
}

__device__ __forceinline__ int8v_t operand16(const uint4& v) {
  return int8v_t{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
                 static_cast<int>(v.w), 0, 0, 0, 0};
}

// Format codes of the f8f6f4 MFMA: 0 = FP8 E4M3, 4 = FP4 E2M1. E8M0 127 = 1.
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE2M1 = 4;
constexpr int kScaleOne = 127;

// The 16 MFMAs of a sub-step. B goes first, so each accumulator tile is C^T.
// MXFP4: op_sel kSel picks the scale byte of the lane's scale word.
template <Fmt F, int kSel>
__device__ __forceinline__ void mfma_substep(floatx16_t (&acc)[4][4], const Frags<F>& f,
                                             const uint32_t (&sa)[4], const uint32_t (&sb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (F == Fmt::kMxFp4) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            operand16(f.b[j]), operand16(f.a[i]), acc[i][j], kFmtE2M1, kFmtE2M1, kSel,
            static_cast<int>(sb[j]), kSel, static_cast<int>(sa[i]));
      } else {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.b[j], f.a[i], acc[i][j], kFmtE4M3,
            kFmtE4M3, 0, kScaleOne, 0, kScaleOne);
      }
    }
}

// MFMA n (= 4 i + j) of a sub-step.
template <Fmt F, int kSel, int kN>
__device__ __forceinline__ void mfma_one(floatx16_t (&acc)[4][4], const Frags<F>& f, const uint32_t (&sa)[4],
                                         const uint32_t (&sb)[4]) {
  constexpr int i = kN >> 2, j = kN & 3;
  if constexpr (F == Fmt::kMxFp4) {
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(operand16(f.b[j]), operand16(f.a[i]), acc[i][j],
                                                                kFmtE2M1, kFmtE2M1, kSel, static_cast<int>(sb[j]),
                                                                kSel, static_cast<int>(sa[i]));
  } else {
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], kFmtE4M3, kFmtE4M3, 0,
                                                                kScaleOne, 0, kScaleOne);
  }
}

// A sub-step's 16 MFMAs with kActions other instructions spread over them:
// action a (act(IC<a>)) follows MFMA (16 a) / kActions. Scheduling fences
// keep this order: loads issued in one burst stall the wave's instruction
// stream (the address unit's queue fills) while the matrix unit idles.
template <Fmt F, int kSel, int kActions, typename Act>
__device__ __forceinline__ void substep(floatx16_t (&acc)[4][4], const Frags<F>& f, const uint32_t (&sa)[4],
                                        const uint32_t (&sb)[4], Act&& act) {
  unroll<16>([&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    mfma_one<F, kSel, n>(acc, f, sa, sb);
    unroll<kActions>([&](auto a_c) {
      constexpr int a = decltype(a_c)::value;
      if constexpr ((16 * a) / kActions == n) act(a_c);
    });
    __builtin_amdgcn_sched_barrier(0);
  });
}

// s_waitcnt immediate: at most n vector memory loads outstanding (vmcnt is
// 6 bits, split over bits 3:0 and 15:14), expcnt and lgkmcnt not waited for.
constexpr int wait_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }


template <Fmt F, bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void block_gemm_kernel(BlockGemmParams p) {
  using T = Traits<F>;
  using L = Lds<F>;
  constexpr int kSub = T::kSub;
  // the stages, and after the K loop the epilogue's staging of C
  constexpr int kLdsBytes = L::kBytes > 4 * kEpilogueWaveBytes ? L::kBytes : 4 * kEpilogueWaveBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + kTile - 1) / kTile;
  const int64_t t = tile_of(blockIdx.x, (p.M + kTile - 1) / kTile, tiles_n);
  const int64_t m0 = (t / tiles_n) * kTile, n0 = (t - (t / tiles_n) * tiles_n) * kTile;
  const int64_t K = p.K;
  // K % (kBK / 2) == 0, K > 0: nfull whole steps and possibly a half step
  const int nfull = static_cast<int>(K / T::kBK);
  const bool tail = (K % T::kBK) != 0;
  const int nsteps = nfull + (tail ? 1 : 0);

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_address(lds);
  const Dma da = dma_setup<F>(p.qa, p.sa, m0, p.M, K, wave_u, lane);
  const Dma db = dma_setup<F>(p.qb, p.sb, n0, p.N, K, wave_u, lane);
  const FragOffsets o = frag_offsets<F>(wm, wn, lane, false);

  // prologue: steps 0 and 1 into stages 0 and 1 (step 0 again when it is
  // the only one), scale chunks 0 and 1 (0 again when it is the only one);
  // step 0 and chunk 0 must have landed
  const int nchunks = (nsteps + T::kChunkSteps - 1) / T::kChunkSteps;
  dma_both<F>(da, db, lds0, 0, nfull == 0, wave_u, lane);
  if constexpr (F == Fmt::kMxFp4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma_scales(da, db, lds0, 0, q, wave_u, lane);
  }
  {
    const int s1 = nsteps > 1 ? 1 : 0;
    dma_both<F>(da, db, lds0, s1, s1 == nfull, wave_u, lane);
  }
  if constexpr (F == Fmt::kMxFp4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma_scales(da, db, lds0, nchunks > 1 ? 1 : 0, q, wave_u, lane);
  }
  constexpr int kDmaStep = 2 * kDmaLoads + (F == Fmt::kMxFp4 ? 16 : 0);  // codes + a chunk per wave
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(kDmaStep));
  __syncthreads();

  Frags<F> f0, f1;
  uint32_t sa[4] = {0, 0, 0, 0}, sb[4] = {0, 0, 0, 0}, sa_n[4] = {0, 0, 0, 0}, sb_n[4] = {0, 0, 0, 0};
  if (nfull > 0) {
    read_frags<F, 0>(f0, lds, o, 0);
    if constexpr (F == Fmt::kMxFp4) read_scales<false>(sa, sb, lds, o, 0);
  }
  // The loads of step t (parts 0 and 1, see dma_code); a target past the
  // last step loads the last step again, into a stage that holds the same
  // bytes or is not read again (so the loop has no branch). Scale chunk c
  // loads quarter (t + 3) % 4 with step t, t = 4 c - 3 .. 4 c: after the
  // last reads of chunk c - 2 (the same buffer) and before step 4 c's
  // scales are read; chunks 0 and 1 are the prologue's.
  auto dma_part = [&](auto part_c, auto item_c, int t) {
    constexpr int part = decltype(part_c)::value, item = decltype(item_c)::value;
    const int tl = t < nsteps ? t : nsteps - 1;
    const bool half = tl == nfull;
    if constexpr (item < 8) {
      // codes: A (item < 4) or B loads 4 part + item % 4
      const Dma& d = item < 4 ? da : db;
      dma_code<F>(d, lds0 + (item < 4 ? L::kA : L::kB), tl, half, 4 * part + (item & 3), wave_u, lane);
    } else if constexpr (F == Fmt::kMxFp4) {
      const int c = (t + 3) >> 2;
      const int cl = c < 1 ? 1 : (c > nchunks - 1 ? nchunks - 1 : c);
      dma_scale(part == 0 ? da : db, lds0 + (part == 0 ? L::kSa : L::kSb), cl, (t + 3) & 3, item - 8, wave_u,
                lane);
    }
  };
  constexpr int kPart = F == Fmt::kMxFp4 ? 10 : 8;  // loads per part
  // A step in stage st (compile-time, so LDS addresses fold into the
  // instructions' offsets). Sub-step s computes from f[s % 2] while the
  // fragments of sub-step s + 1 load into the other buffer; after the
  // barrier that hands the stage back, the last sub-step issues part 0 of
  // step s + 2's loads (FP8: both parts), and FP4's part 1 follows with the
  // next step's sub-steps 0 and 1.
  auto do_step = [&](auto st_c, int step) {
    constexpr int st = decltype(st_c)::value;
    auto reads = [&](auto ss_c, Frags<F>& f) {
      return [&, ss_c](auto a_c) {
        constexpr int a = decltype(a_c)::value;
        read_frag<F, decltype(ss_c)::value, a>(f, lds, o, st);
      };
    };
    // Part 1 of step s + 1's loads: FP4 (16 MFMAs of 32 cycles per
    // sub-step) spreads it over sub-steps 0 and 1; FP8 (64-cycle MFMAs)
    // issued it with part 0 after the previous barrier (each measured faster
    // than the other placement).
    constexpr int kP0 = kSub == 4 ? kPart / 2 : 0;  // part 1 loads in sub-step 0
    constexpr int kP1 = kSub == 4 ? kPart - kP0 : 0;  // ... and in sub-step 1
    substep<F, 0, 8 + kP0>(acc, f0, sa, sb, [&](auto a_c) {
      constexpr int a = decltype(a_c)::value;
      if constexpr (a < 8) {
        read_frag<F, 1, a>(f1, lds, o, st);
      } else {
        dma_part(IC<1>{}, IC<a - 8>{}, step + 1);
      }
    });
    if constexpr (kSub == 4) {
      substep<F, 1, 8 + kP1>(acc, f1, sa, sb, [&](auto a_c) {
        constexpr int a = decltype(a_c)::value;
        if constexpr (a < 8) {
          read_frag<F, 2, a>(f0, lds, o, st);
        } else {
          dma_part(IC<1>{}, IC<a - 8 + kP0>{}, step + 1);
        }
      });
      substep<F, 2, 8>(acc, f0, sa, sb, reads(IC<3>{}, f1));
    }
    // every wave's reads of this stage are complete and its loads of step
    // + 1 have landed
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    constexpr int kScaleReads = F == Fmt::kMxFp4 ? 8 : 0;
    constexpr int kLast = kSub == 4 ? kPart : 2 * kPart;  // loads after the barrier
    substep<F, kSub - 1, 8 + kScaleReads + kLast>(acc, f1, sa, sb, [&](auto a_c) {
      constexpr int a = decltype(a_c)::value;
      if constexpr (a < 8) {
        read_frag<F, 0, a>(f0, lds, o, st ^ 1);
      } else if constexpr (a < 8 + kScaleReads) {
        read_scale_word(sa_n, sb_n, lds, o, step + 1, IC<a - 8>{});
      } else if constexpr (a < 8 + kScaleReads + kPart) {
        dma_part(IC<0>{}, IC<a - 8 - kScaleReads>{}, step + 2);
      } else {
        dma_part(IC<1>{}, IC<a - 8 - kScaleReads - kPart>{}, step + 2);
      }
    });
    if constexpr (F == Fmt::kMxFp4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[i] = sa_n[i];
        sb[i] = sb_n[i];
      }
    }
  };
  for (int step = 0; step + 1 < nfull; step += 2) {
    do_step(std::integral_constant<int, 0>{}, step);
    do_step(std::integral_constant<int, 1>{}, step + 1);
  }
  if (nfull & 1) do_step(std::integral_constant<int, 0>{}, nfull - 1);
  if (tail) {
    // the half step, in stage nfull & 1 (landed: the last full step's
    // barrier, or the prologue's)
    const int st = nfull & 1;
    const FragOffsets oh = frag_offsets<F>(wm, wn, lane, true);
    Frags<F> g0, g1;
    read_frags<F, 0>(g0, lds, oh, st);
    if constexpr (F == Fmt::kMxFp4) {
      read_scales<true>(sa, sb, lds, oh, nfull);
      read_frags<F, 1>(g1, lds, oh, st);
      mfma_substep<F, 0>(acc, g0, sa, sb);
      mfma_substep<F, 1>(acc, g1, sa, sb);
    } else {
      mfma_substep<F, 0>(acc, g0, sa, sb);
    }
  }
  float alpha = 1.0f;
  if constexpr (F == Fmt::kFp8) alpha = __fmul_rn(*p.ta, *p.tb);
  const int64_t r0 = m0 + wm * kWave, c0 = n0 + wn * kWave;
  constexpr int kElem = kBf16Out ? 2 : 4;
  const bool lines = r0 + kWave <= p.M && c0 + kWave <= p.N && ((p.ldc * kElem) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.c) & 15) == 0;
  // the loop's last (repeated) loads have landed and every wave is done
  // with the stages, which the epilogue reuses
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (lines) {
    store_tile_lds<kBf16Out>(acc, alpha, p.c, p.ldc, r0, c0, lane, lds + wave * kEpilogueWaveBytes);
  } else {
    store_tile<4, kBf16Out>(acc, alpha, p.c, p.ldc, p.M, p.N, r0, c0, lane);
  }
}

template <Fmt F>
int launch_block_gemm(const BlockGemmParams& p, bool c_bf16, hipStream_t stream) {
  if (p.K == 0) {
    int64_t blocks = (p.M * p.N + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    zero_output_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(p.c, p.M, p.N, p.ldc, c_bf16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int64_t tiles = ((p.M + kTile - 1) / kTile) * ((p.N + kTile - 1) / kTile);
  if (c_bf16) block_gemm_kernel<F, true><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
  else block_gemm_kernel<F, false><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                   int64_t M, int64_t N, int64_t K, void* c, bool c_bf16, int64_t ldc,
                   hipStream_t stream) {
  const BlockGemmParams p{qa, sa, qb, sb, nullptr, nullptr, c, M, N, K, ldc};
  return launch_block_gemm<Fmt::kMxFp4>(p, c_bf16, stream);
}

int launch_fp8_gemm(const uint8_t* qa, const float* ta, const uint8_t* qb, const float* tb,
                    int64_t M, int64_t N, int64_t K, void* c, bool c_bf16, int64_t ldc,
                    hipStream_t stream) {
  const BlockGemmParams p{qa, nullptr, qb, nullptr, ta, tb, c, M, N, K, ldc};
  return launch_block_gemm<Fmt::kFp8>(p, c_bf16, stream);
}

}  // namespace nvfp4
