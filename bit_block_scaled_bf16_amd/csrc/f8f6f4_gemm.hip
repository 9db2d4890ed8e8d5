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
  static constexpr int kScaleBytes = kTile * kScaleRow;
  static __device__ __forceinline__ int64_t row_bytes(int64_t K) { return K >> 1; }
};

template <>
struct Traits<Fmt::kFp8> {
  static constexpr int kBK = 128;
  static constexpr int kSub = 2;
  static constexpr int kChunks = 2;
  static constexpr int kScaleRow = 0;
  static constexpr int kScaleBytes = 0;
  static __device__ __forceinline__ int64_t row_bytes(int64_t K) { return K; }
};

// LDS: [A codes, stages 0 and 1][B codes][A scales][B scales].
template <Fmt F>
struct Lds {
  static constexpr int kA = 0;
  static constexpr int kB = 2 * kCodeBytes;
  static constexpr int kSa = 4 * kCodeBytes;
  static constexpr int kSb = kSa + 2 * Traits<F>::kScaleBytes;
  static constexpr int kBytes = kSb + 2 * Traits<F>::kScaleBytes;
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
// j % 8) and, for MXFP4, 2 scale loads of 32 rows (lane j: row
// 64 w + 32 k + j / 2, the 4 bytes (j % 2) of the row's 8 bytes of the step).
// (row >> 1) & 7 = (4 k + j / 16) & 7 for these rows, so the chunk depends
// on k only through k % 2, and load k is load k % 2 plus 8 k rows. Rows past
// the matrix read its last row instead (they only feed C outside M x N).
struct Dma {
  const uint8_t* rowp;   // this lane's row of load 0 (unclamped)
  const uint8_t* lastp;  // the matrix's last row (uniform)
  const uint8_t* srowp;  // this lane's scale row of scale load 0 (MXFP4; unclamped)
  const uint8_t* slastp; // the last scale row (uniform)
  int left, sleft;       // rows from load 0's (scale load 0's) row to the end of the matrix
  int64_t rb, srb;       // code and scale bytes per row (uniform)
};

__device__ __forceinline__ int dma_chunk(int k, int lane) { return (lane & 7) ^ ((4 * k + (lane >> 4)) & 7); }

template <Fmt F>
__device__ __forceinline__ Dma dma_setup(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                         int64_t row0, int64_t rows, int64_t K, int wave, int lane) {
  Dma d;
  d.rb = Traits<F>::row_bytes(K);
  d.srb = K / kMxBlock;
  const int64_t row = row0 + 64 * wave + (lane >> 3);
  const int64_t srow = row0 + 64 * wave + (lane >> 1);
  // rows - row, capped: only its comparison with the tile's row offsets matters
  d.left = static_cast<int>((rows - row) < kTile ? (rows - row) : kTile);
  d.sleft = static_cast<int>((rows - srow) < kTile ? (rows - srow) : kTile);
  d.rowp = q + row * d.rb;
  d.lastp = q + (rows - 1) * d.rb;
  d.srowp = nullptr;
  d.slastp = nullptr;
  if constexpr (F == Fmt::kMxFp4) {
    d.srowp = s + srow * d.srb + 4 * (lane & 1);
    d.slastp = s + (rows - 1) * d.srb + 4 * (lane & 1);
  }
  return d;
}

// Requests step `step` of one operand (this wave's 64 rows) into the LDS
// stage at byte addresses codes / scales. A half step (64 bytes per row, the
// last step of some K) reads chunk c & 3 for chunk c and the row's first 4
// scale bytes for both scale words: the slots of chunks 4-7 and the second
// scale word then hold copies that are never read.
template <Fmt F>
__device__ __forceinline__ void dma_step(const Dma& d, uint32_t codes, uint32_t scales, int step,
                                         bool half, int wave, int lane) {
  const int64_t off = static_cast<int64_t>(step) * kRowBytes;
  const uint32_t c0 = codes + 64 * wave * kRowBytes;
#pragma unroll
  for (int k = 0; k < kDmaLoads; ++k) {
    const int c = dma_chunk(k, lane) & (half ? 3 : 7);
    const uint8_t* g = (8 * k < d.left) ? d.rowp + (8 * k) * d.rb : d.lastp;
    lds_dma<16>(g + off + 16 * c, c0 + k * (8 * kRowBytes));
  }
  if constexpr (F == Fmt::kMxFp4) {
    const int64_t soff = static_cast<int64_t>(step) * Traits<F>::kScaleRow;
    const uint32_t s0 = scales + 64 * wave * Traits<F>::kScaleRow;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint8_t* g = (32 * k < d.sleft) ? d.srowp + (32 * k) * d.srb : d.slastp;
      const int back = (lane & 1) * (half ? 4 : 0);
      lds_dma<4>(g + soff - back, s0 + k * (32 * Traits<F>::kScaleRow));
    }
  }
}

// Step `step` of A and B into stage step % 2; a half step when step is the
// last and K leaves half a step (uniform choice).
template <Fmt F>
__device__ __forceinline__ void dma_both(const Dma& da, const Dma& db, uint32_t lds, int step, bool half,
                                         int wave, int lane) {
  using L = Lds<F>;
  const int st = step & 1;
  const uint32_t ca = lds + L::kA + st * kCodeBytes, sa = lds + L::kSa + st * Traits<F>::kScaleBytes;
  const uint32_t cb = lds + L::kB + st * kCodeBytes, sb = lds + L::kSb + st * Traits<F>::kScaleBytes;
  dma_step<F>(da, ca, sa, step, half, wave, lane);
  dma_step<F>(db, cb, sb, step, half, wave, lane);
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
  o.sa = L::kSa + ra * Traits<F>::kScaleRow + (half ? 2 * h : 4 * h);
  o.sb = L::kSb + rb * Traits<F>::kScaleRow + (half ? 2 * h : 4 * h);
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

// The lane's scale words of a step (MXFP4): one 32-bit word per block of a
// full step, one 16-bit half of a half step.
template <bool kHalf>
__device__ __forceinline__ void read_scales(uint32_t (&sa)[4], uint32_t (&sb)[4], const uint8_t* __restrict__ lds,
                                            const FragOffsets& o, int st) {
  constexpr int kRow = Traits<Fmt::kMxFp4>::kScaleRow, kBytes = Traits<Fmt::kMxFp4>::kScaleBytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kHalf) {
      sa[i] = *reinterpret_cast<const uint16_t*>(lds + o.sa + st * kBytes + i * 32 * kRow);
      sb[i] = *reinterpret_cast<const uint16_t*>(lds + o.sb + st * kBytes + i * 32 * kRow);
    } else {
      sa[i] = *reinterpret_cast<const uint32_t*>(lds + o.sa + st * kBytes + i * 32 * kRow);
      sb[i] = *reinterpret_cast<const uint32_t*>(lds + o.sb + st * kBytes + i * 32 * kRow);
    }
  }
}

// An FP4 operand: 16 bytes in the low half of the operand tuple (the
// instruction reads 4 registers for FP4).
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

// s_waitcnt immediate: at most n vector memory loads outstanding (vmcnt is
// 6 bits, split over bits 3:0 and 15:14), expcnt and lgkmcnt not waited for.
constexpr int wait_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

template <Fmt F, bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void block_gemm_kernel(BlockGemmParams p) {
  using T = Traits<F>;
  using L = Lds<F>;
  constexpr int kSub = T::kSub;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + kTile - 1) / kTile;
  const int64_t t = blockIdx.x;
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

  // prologue: steps 0 and 1 into stages 0 and 1; step 0 must have landed
  dma_both<F>(da, db, lds0, 0, nfull == 0, wave_u, lane);
  if (nsteps > 1) {
    dma_both<F>(da, db, lds0, 1, nfull == 1, wave_u, lane);
    constexpr int kDma = 2 * (kDmaLoads + (F == Fmt::kMxFp4 ? 2 : 0));
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kDma));
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  __syncthreads();

  Frags<F> f0, f1;
  uint32_t sa[4] = {0, 0, 0, 0}, sb[4] = {0, 0, 0, 0}, sa_n[4] = {0, 0, 0, 0}, sb_n[4] = {0, 0, 0, 0};
  if (nfull > 0) {
    read_frags<F, 0>(f0, lds, o, 0);
    if constexpr (F == Fmt::kMxFp4) read_scales<false>(sa, sb, lds, o, 0);
  }
  // a step in stage kSt (compile-time, so LDS addresses fold into the
  // instructions' offsets). Sub-step s computes from f[s % 2] while the
  // fragments of sub-step s + 1 load into the other buffer.
  auto hand_back = [&](auto st_c, int step) {
    // the last sub-step: the step's stage has been read (each wave's reads
    // complete before the barrier), every wave's loads of step + 1 have
    // landed after it, and the stage takes step + 2
    // (unconditional reads and barrier: after the last full step they read
    // a stage that is not used, which keeps the registers' flow the same on
    // every step)
    // The load is unconditional too: past the last step it loads the last
    // step again into the stage just read, which nothing reads afterwards
    // (a conditional load here let the compiler move the MFMAs out of
    // place).
    constexpr int st = decltype(st_c)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int ld = step + 2 < nsteps ? step + 2 : nsteps - 1;
    dma_both<F>(da, db, lds0, ld, ld == nfull, wave_u, lane);
    read_frags<F, 0>(f0, lds, o, st ^ 1);
    if constexpr (F == Fmt::kMxFp4) read_scales<false>(sa_n, sb_n, lds, o, st ^ 1);
  };
  auto do_step = [&](auto st_c, int step) {
    constexpr int st = decltype(st_c)::value;
    // scheduling fences between sub-steps keep each sub-step's fragment
    // reads from being hoisted further ahead (which would need more
    // registers than the two fragment buffers)
    if constexpr (kSub == 4) {
      read_frags<F, 1>(f1, lds, o, st);
      mfma_substep<F, 0>(acc, f0, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
      read_frags<F, 2>(f0, lds, o, st);
      mfma_substep<F, 1>(acc, f1, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
      read_frags<F, 3>(f1, lds, o, st);
      mfma_substep<F, 2>(acc, f0, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
      hand_back(st_c, step);
      mfma_substep<F, 3>(acc, f1, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      read_frags<F, 1>(f1, lds, o, st);
      mfma_substep<F, 0>(acc, f0, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
      hand_back(st_c, step);
      mfma_substep<F, 1>(acc, f1, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
    }
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
      read_scales<true>(sa, sb, lds, oh, st);
      read_frags<F, 1>(g1, lds, oh, st);
      mfma_substep<F, 0>(acc, g0, sa, sb);
      mfma_substep<F, 1>(acc, g1, sa, sb);
    } else {
      mfma_substep<F, 0>(acc, g0, sa, sb);
    }
  }
  float alpha = 1.0f;
  if constexpr (F == Fmt::kFp8) alpha = __fmul_rn(*p.ta, *p.tb);
  store_tile<4, kBf16Out>(acc, alpha, p.c, p.ldc, p.M, p.N, m0 + wm * kWave, n0 + wn * kWave, lane);
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
