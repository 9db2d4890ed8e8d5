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
// Staging (the NVFP4 GEMM's): a 256 x 256 tile per workgroup, 4 waves of
// 128 x 128, 64-byte code rows per step in an LDS ring filled by
// global_load_lds with XOR-swizzled 16-byte chunks. A step is K = 128 for
// FP4 (2 MFMA sub-steps of K = 64) and K = 64 for FP8 (one MFMA of K = 64 per
// 32 x 32 tile): either way 16 KiB of codes per operand and the same MFMA
// time. A step is short, so the ring has 4 stages and a step's loads are
// requested 4 steps ahead; the wait before a step's barrier leaves the 2
// newest steps' loads in flight.
//
// MXFP4 scale bytes: lane half h of sub-step s takes K [64h + 32s, +32), so
// its two scale bytes of the step are adjacent and one 16-bit LDS read
// serves both sub-steps (the MFMA's op_sel picks the byte).
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

using namespace gemm_common;

enum class Fmt { kMxFp4, kFp8 };

constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int kTile = 256;              // C rows and columns per workgroup
constexpr int kWave = 128;              // C rows and columns per wave
constexpr int kCodeStride = 64;         // bytes per LDS code row and step
constexpr int kCodeBytes = kTile * kCodeStride;
constexpr int kMxBlock = 32;

template <Fmt F>
struct Traits;

template <>
struct Traits<Fmt::kMxFp4> {
  static constexpr int kBK = 128;                  // K elements per step
  static constexpr int kScaleStride = 128 / 32;    // 4 scale bytes per LDS row
  static constexpr int kScaleBytes = kTile * kScaleStride;
  static constexpr int kDmaPerStep = 2 * (4 + 1);  // per wave: 4 code + 1 scale loads per operand
  static __device__ __forceinline__ int64_t row_bytes(int64_t K) { return K >> 1; }
};

template <>
struct Traits<Fmt::kFp8> {
  static constexpr int kBK = 64;
  static constexpr int kScaleStride = 0;
  static constexpr int kScaleBytes = 0;
  static constexpr int kDmaPerStep = 2 * 4;
  static __device__ __forceinline__ int64_t row_bytes(int64_t K) { return K; }
};

template <Fmt F>
constexpr int stage_bytes() {
  return 2 * kCodeBytes + 2 * Traits<F>::kScaleBytes;
}

typedef int int8v_t __attribute__((ext_vector_type(8)));

struct BlockGemmParams {
  const uint8_t *qa, *sa, *qb, *sb;  // scales: MXFP4 only
  const float *ta, *tb;              // per-tensor scales: FP8 only
  void* c;
  int64_t M, N, K, ldc;
};

// This lane's share of one operand's DMA per step: 4 code chunks (rows
// 64 w + 16 i + l / 4, LDS position l % 4) and, for MXFP4, the 4 scale bytes
// of row 64 w + l. Rows past the end are clamped (they only feed C outside
// M x N).
struct DmaSource {
  const uint8_t* q[4];
  const uint8_t* s;
};

template <Fmt F>
__device__ __forceinline__ DmaSource dma_source(const uint8_t* __restrict__ q,
                                                const uint8_t* __restrict__ s, int64_t row0,
                                                int64_t rows, int64_t K, int wave, int lane) {
  DmaSource d;
  const int64_t rb = Traits<F>::row_bytes(K);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * wave + 16 * i + (lane >> 2);
    const int64_t row = row0 + r;
    const int64_t rc = row < rows ? row : rows - 1;
    d.q[i] = q + rc * rb + 16 * chunk_pos(r, lane & 3);
  }
  d.s = nullptr;
  if constexpr (F == Fmt::kMxFp4) {
    const int64_t row = row0 + 64 * wave + lane;
    const int64_t rc = row < rows ? row : rows - 1;
    d.s = s + rc * (K / kMxBlock);
  }
  return d;
}

template <Fmt F>
__device__ __forceinline__ void dma_stage(const DmaSource& d, const uint8_t* codes,
                                          const uint8_t* scales, int step, int wave) {
  const int64_t off = static_cast<int64_t>(step) * kCodeStride;  // 64 bytes of a row per step
  const uint32_t c0 = lds_address(codes) + 64 * wave * kCodeStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) lds_dma<16>(d.q[i] + off, c0 + 16 * i * kCodeStride);
  if constexpr (F == Fmt::kMxFp4) {
    lds_dma<4>(d.s + static_cast<int64_t>(step) * (Traits<F>::kBK / kMxBlock),
               lds_address(scales) + 64 * wave * Traits<F>::kScaleStride);
  }
}

// The fragments of one step: 16-byte chunks [row or column block][half of
// the lane's 32 bytes] and, for MXFP4, the two scale bytes of each block.
struct Frags {
  uint4 a[4][2], b[4][2];
  uint32_t sa[4], sb[4];
};

struct Offsets {
  int a_code[2], b_code[2], a_scale, b_scale;
};

template <Fmt F>
__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* __restrict__ stage,
                                           const Offsets& o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f.a[i][s] = *reinterpret_cast<const uint4*>(stage + o.a_code[s] + i * 32 * kCodeStride);
      f.b[i][s] = *reinterpret_cast<const uint4*>(stage + kCodeBytes + o.b_code[s] + i * 32 * kCodeStride);
    }
    if constexpr (F == Fmt::kMxFp4) {
      constexpr int ss = Traits<F>::kScaleStride;
      f.sa[i] = *reinterpret_cast<const uint16_t*>(stage + 2 * kCodeBytes + o.a_scale + i * 32 * ss);
      f.sb[i] = *reinterpret_cast<const uint16_t*>(stage + 2 * kCodeBytes + Traits<F>::kScaleBytes +
                                                   o.b_scale + i * 32 * ss);
    }
  }
}

__device__ __forceinline__ int8v_t operand16(const uint4& v) {
  return int8v_t{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
                 static_cast<int>(v.w), 0, 0, 0, 0};
}

__device__ __forceinline__ int8v_t operand32(const uint4& lo, const uint4& hi) {
  return int8v_t{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                 static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                 static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// Format codes of the f8f6f4 MFMA: 0 = FP8 E4M3, 4 = FP4 E2M1. E8M0 127 = 1.
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE2M1 = 4;
constexpr int kScaleOne = 127;

// MXFP4 sub-step kS (K = 64): op_sel kS picks the scale byte of the
// sub-step. B goes first, so each accumulator tile is C^T.
template <int kS>
__device__ __forceinline__ void mx_substep(floatx16_t (&acc)[4][4], const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          operand16(f.b[j][kS]), operand16(f.a[i][kS]), acc[i][j], kFmtE2M1, kFmtE2M1, kS,
          static_cast<int>(f.sb[j]), kS, static_cast<int>(f.sa[i]));
}

// FP8 step (K = 64): the lane's 32 bytes are its two chunks.
__device__ __forceinline__ void fp8_step(floatx16_t (&acc)[4][4], const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          operand32(f.b[j][0], f.b[j][1]), operand32(f.a[i][0], f.a[i][1]), acc[i][j], kFmtE4M3,
          kFmtE4M3, 0, kScaleOne, 0, kScaleOne);
}

// s_waitcnt immediate: at most n vector memory loads outstanding (vmcnt is
// 6 bits, split over bits 3:0 and 15:14), expcnt and lgkmcnt not waited for.
constexpr int wait_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

template <Fmt F, bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void block_gemm_kernel(BlockGemmParams p) {
  using T = Traits<F>;
  constexpr int kStageBytes = stage_bytes<F>();
  constexpr int kDma = T::kDmaPerStep;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + kTile - 1) / kTile;
  const int64_t t = blockIdx.x;
  const int64_t m0 = (t / tiles_n) * kTile, n0 = (t - (t / tiles_n) * tiles_n) * kTile;
  const int64_t K = p.K;
  const int nsteps = static_cast<int>(K / T::kBK);  // >= 1 (K % kBK == 0, K > 0)
  const int last = nsteps - 1;

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const DmaSource da = dma_source<F>(p.qa, p.sa, m0, p.M, K, wave_u, lane);
  const DmaSource db = dma_source<F>(p.qb, p.sb, n0, p.N, K, wave_u, lane);
  // prologue: steps 0-3 into stages 0-3; steps 0 and 1 must have landed
#pragma unroll
  for (int q = 0; q < kStages; ++q) {
    uint8_t* st = lds + q * kStageBytes;
    const int ld = q < last ? q : last;
    dma_stage<F>(da, st, st + 2 * kCodeBytes, ld, wave_u);
    dma_stage<F>(db, st + kCodeBytes, st + 2 * kCodeBytes + T::kScaleBytes, ld, wave_u);
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kDma));
  __syncthreads();

  const int frag_row = lane & 31;
  const int half = lane >> 5;
  const int swz = ((frag_row >> 1) ^ (frag_row >> 2)) & 3;  // same for frag_row + 32 i
  Offsets o;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    o.a_code[s] = (wm * kWave + frag_row) * kCodeStride + 16 * ((2 * half + s) ^ swz);
    o.b_code[s] = (wn * kWave + frag_row) * kCodeStride + 16 * ((2 * half + s) ^ swz);
  }
  o.a_scale = (wm * kWave + frag_row) * T::kScaleStride + 2 * half;
  o.b_scale = (wn * kWave + frag_row) * T::kScaleStride + 2 * half;

  // Step s reads step s + 1's fragments from LDS (landed before the barrier
  // that ended step s - 1) while its own MFMAs run, and requests step s + 4
  // into stage s % 4: step s's own fragments were read during step s - 1,
  // before that barrier (for step 0: before the second prologue barrier).
  // Before a step's barrier, step s + 2 must have landed; the loads of steps
  // s + 3 and s + 4 stay in flight (loads complete in issue order).
  Frags cur, nxt;
  read_frags<F>(cur, lds, o);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int stage = step & (kStages - 1);
    const int sn = (step + 1) & (kStages - 1);
    // the LDS reads go first: the DMA's inline assembly is a compiler
    // memory barrier, and reads placed after it would sink below the MFMAs
    read_frags<F>(nxt, lds + sn * kStageBytes, o);
    {
      uint8_t* st = lds + stage * kStageBytes;
      const int ld = (step + kStages) < last ? (step + kStages) : last;
      dma_stage<F>(da, st, st + 2 * kCodeBytes, ld, wave_u);
      dma_stage<F>(db, st + kCodeBytes, st + 2 * kCodeBytes + T::kScaleBytes, ld, wave_u);
    }
    if constexpr (F == Fmt::kMxFp4) {
      mx_substep<0>(acc, cur);
      mx_substep<1>(acc, cur);
    } else {
      fp8_step(acc, cur);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kDma));
    __syncthreads();
    cur = nxt;
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
