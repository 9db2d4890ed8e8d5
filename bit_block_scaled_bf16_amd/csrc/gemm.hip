// GEMM on NVFP4 operands for gfx950: C[M][N] = (S_A S_B) * sum_k a_k b_k
// with a_k = e2m1(q) * s_f, float32 accumulation, bf16 or float32 output.
//
// Source: gist.science summary of "Pretraining Large Language Models with
// NVFP4", Resumen técnico §2 "Precisión Mixta Selectiva" (the linear-layer
// GEMMs run on NVFP4 operands) and "Formato NVFP4" (16-element blocks with an
// E4M3 scale each).
//
// Why fp16 MFMA. An element times its block scale, e2m1 * E4M3, has at most
// 2 + 4 = 6 significant bits and lies in [2^-10, 2688], so it is exact in
// fp16 (11 bits, normal down to 2^-14). The products of two such values are
// exact in float32, so the only rounding is the float32 accumulation. The
// gfx950 block-scaled FP4 MFMA cannot take these operands exactly: its scales
// are powers of two per 32 elements, while NVFP4 has an E4M3 scale (4
// significant bits) per 16. The dense fp16 MFMA has the same peak as bf16.
//
// Structure. A workgroup of 256 threads computes a 256 x 256 tile of C; its 4
// waves each own 128 x 128 (4 x 4 MFMA 32x32x16 tiles, float32 accumulators).
// The K loop runs in steps of 128. The packed FP4 codes (0.5 byte / element)
// and the scale bytes of a step go from global memory into a 3-stage LDS
// ring; each wave then reads the codes of its own rows and columns and
// expands them to fp16 in registers right before the MFMAs (the gfx950 FP4 ->
// fp16 converter, then one packed fp16 multiply by the block scale, both
// exact). Keeping the codes, not fp16 values, in LDS moves a quarter of the
// bytes through it.
//
// Tile order and epilogue. Tiles go to the XCDs in blocks of 32 that share
// operand panels (tile_of, gemm_common.h). A wave writes its 128 x 128
// results through LDS as whole 128-byte lines of C, with nontemporal stores
// (store_tile_lds); edge tiles store 8-byte pieces.
//
// Last round. 256 x 256 tiles keep one workgroup per CU busy; when the tile
// count leaves a last round that fills at most a quarter of the CUs, those
// tiles are computed as four 128 x 128 tiles each (the same kernel with
// 2 x 2 MFMA tiles per wave) by a second launch, so the round ends about four
// times sooner instead of leaving most of the chip idle.
//
// LDS layout of a stage (B = tile rows): codes [B][64 bytes] for A, then B,
// then the scale bytes [B][8] for A, then B. The four 16-byte chunks of code row r sit
// at positions chunk ^ swz(r), swz(r) = ((r >> 1) ^ (r >> 2)) & 3, so the
// fragment reads (one chunk of 16 or 8 consecutive rows per LDS cycle) hit
// distinct banks. When K % 128 == 0 the codes and scales travel from global
// memory straight into LDS (gfx950 global_load_lds, 16 and 4 bytes per lane);
// otherwise they go through registers, with blocks past K read as zero.
//
// K order inside a step. MFMA 32x32x16 takes k-slots 0-7 from lanes 0-31 and
// 8-15 from lanes 32-63. Any assignment of k to (sub-step, slot) works as
// long as A and B use the same one, so lane half h takes the 64 consecutive
// k of [64h, 64h + 64) and sub-step kk uses k = 64h + 8kk + [0, 8): each lane
// reads 32 contiguous code bytes of a row with two 16-byte LDS reads.
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

#include <atomic>

namespace nvfp4 {
namespace {

using namespace gemm_common;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;                 // K elements per step
constexpr int kThreads = 256;            // 4 waves, 2 x 2 over the tile
constexpr int kStages = 3;               // LDS ring depth
constexpr int kCodeStride = kBK / 2;     // bytes per LDS code row (swizzled)
constexpr int kScaleStride = kBK / 16;   // bytes per LDS scale row
constexpr int kBigTile = 256;            // tile edge of the main launch (kT = 4)

// Tile geometry for kT x kT MFMA 32x32 tiles per wave.
template <int kT>
struct Geo {
  static constexpr int kWave = 32 * kT;                  // C rows (and columns) per wave
  static constexpr int kTile = 2 * kWave;                // C rows (and columns) per workgroup
  static constexpr int kCodeBytes = kTile * kCodeStride;  // one operand's codes per stage
  static constexpr int kScaleBytes = kTile * kScaleStride;
  static constexpr int kStageBytes = 2 * kCodeBytes + 2 * kScaleBytes;
  static constexpr int kWaveRows = kTile / 4;            // operand rows each wave stages
};

struct GemmParams {
  const uint8_t* qa;
  const uint8_t* sa;
  const uint8_t* qb;
  const uint8_t* sb;
  const float* ta;
  const float* tb;
  void* c;
  int64_t M, N, K, ldc;
  int64_t tile0;  // tile_of argument of this launch's first tile (see the kernel)
};

// ---------------------------------------------------------------------------
// Register staging (K % 128 != 0).
// ---------------------------------------------------------------------------

// One thread's share of one operand for one K step: kT chunks of 16 code
// bytes (rows (tid >> 2) + 64 i, part tid & 3) and, for tid < tile rows, the
// 8 scale bytes of row tid.
template <int kT>
struct Stage {
  uint4 codes[kT];
  uint2 scales;
};

// Rows past the end are clamped to the last row, so every load stays in
// bounds; they only feed rows or columns of C that are never stored.
template <int kT>
struct OperandSource {
  const uint8_t* q[kT];  // code rows of the chunks (clamped)
  const uint8_t* s;      // scale row (clamped)
};

template <int kT, bool k2D>
__device__ __forceinline__ OperandSource<kT> operand_source(const uint8_t* __restrict__ q,
                                                            const uint8_t* __restrict__ s,
                                                            int64_t row0, int64_t rows, int64_t K,
                                                            int tid) {
  OperandSource<kT> src;
  const int part = tid & 3;
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int64_t row = row0 + (tid >> 2) + 64 * i;
    const int64_t r = row < rows ? row : rows - 1;
    src.q[i] = q + r * (K >> 1) + 16 * part;
  }
  const int64_t srow = row0 + (tid & (Geo<kT>::kTile - 1));
  const int64_t r = srow < rows ? srow : rows - 1;
  src.s = s + (k2D ? (r >> 4) : r) * (K >> 4);
  return src;
}

// Loads K step `step`; each 16-element block is loaded on its own and blocks
// past K read as zero.
template <int kT>
__device__ __forceinline__ Stage<kT> load_stage(const OperandSource<kT>& src, int step, int64_t K,
                                                int part) {
  Stage<kT> st;
  const int64_t k0 = static_cast<int64_t>(step) * kBK;
  const int64_t kb0 = k0 >> 4;  // first scale block of the step
  const int64_t nkb = K >> 4;   // scale blocks per row
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
    const int64_t b = kb0 + 2 * part;  // this chunk covers blocks b and b + 1
    if (b < nkb) lo = *reinterpret_cast<const uint2*>(src.q[i] + (k0 >> 1));
    if (b + 1 < nkb) hi = *reinterpret_cast<const uint2*>(src.q[i] + (k0 >> 1) + 8);
    st.codes[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t v = (kb0 + j < nkb) ? src.s[kb0 + j] : 0u;
    if (j < 4) w0 |= v << (8 * j);
    else w1 |= v << (8 * (j - 4));
  }
  st.scales = make_uint2(w0, w1);
  return st;
}

// Writes a register-staged step into LDS (swizzled code chunks).
template <int kT>
__device__ __forceinline__ void store_stage(uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                            const Stage<kT>& st, int tid) {
  const int part = tid & 3;
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int r = (tid >> 2) + 64 * i;
    *reinterpret_cast<uint4*>(codes + r * kCodeStride + 16 * chunk_pos(r, part)) = st.codes[i];
  }
  if (tid < Geo<kT>::kTile) *reinterpret_cast<uint2*>(scales + tid * kScaleStride) = st.scales;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS staging (K % 128 == 0). Wave w fills code rows
// [w R, w R + R), R = tile rows / 4, with R / 16 instructions of 16 rows x 64
// bytes (lane l: row 16 i + l / 4, LDS position l % 4, so it loads chunk
// (l % 4) ^ swz(row)) and the same scale rows with R / 32 instructions of
// 32 rows x 8 bytes.
// ---------------------------------------------------------------------------
template <int kT>
struct DmaSource {
  const uint8_t* q[kT];      // per instruction: this lane's code chunk at k = 0 (row clamped)
  const uint8_t* s[kT / 2];  // per instruction: this lane's 4 scale bytes at k = 0 (row clamped)
};

template <int kT, bool k2D>
__device__ __forceinline__ DmaSource<kT> dma_source(const uint8_t* __restrict__ q,
                                                    const uint8_t* __restrict__ s, int64_t row0,
                                                    int64_t rows, int64_t K, int wave, int lane) {
  constexpr int R = Geo<kT>::kWaveRows;
  DmaSource<kT> d;
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int r = R * wave + 16 * i + (lane >> 2);  // row within the tile
    const int64_t row = row0 + r;
    const int64_t rc = row < rows ? row : rows - 1;
    d.q[i] = q + rc * (K >> 1) + 16 * chunk_pos(r, lane & 3);
  }
#pragma unroll
  for (int i = 0; i < kT / 2; ++i) {
    const int64_t row = row0 + R * wave + 32 * i + (lane >> 1);
    const int64_t rc = row < rows ? row : rows - 1;
    d.s[i] = s + (k2D ? (rc >> 4) : rc) * (K >> 4) + 4 * (lane & 1);
  }
  return d;
}

template <int kT>
__device__ __forceinline__ void dma_stage(const DmaSource<kT>& d, const uint8_t* codes,
                                          const uint8_t* scales, int step, int wave) {
  constexpr int R = Geo<kT>::kWaveRows;
  const int64_t k0 = static_cast<int64_t>(step) * kBK;
  const uint32_t c0 = lds_address(codes) + R * wave * kCodeStride;
  const uint32_t s0 = lds_address(scales) + R * wave * kScaleStride;
#pragma unroll
  for (int i = 0; i < kT; ++i) lds_dma<16>(d.q[i] + (k0 >> 1), c0 + 16 * i * kCodeStride);
#pragma unroll
  for (int i = 0; i < kT / 2; ++i) lds_dma<4>(d.s[i] + (k0 >> 4), s0 + 32 * i * kScaleStride);
}

// ---------------------------------------------------------------------------
// Fragments.
// ---------------------------------------------------------------------------

// The block scale of sub-step kk as fp16: byte kk >> 1 of the lane's scale
// word. gfx950's FP8 (E4M3) -> fp16 converter decodes two bytes per
// instruction, exactly (every E4M3 value, subnormals included, is an fp16
// normal number; checked for all 256 bytes). With kk known at compile time
// the selects fold away and the two conversions of a word are shared by its
// eight sub-steps.
__device__ __forceinline__ _Float16 scale_f16(uint32_t w, int kk) {
  const half2_t p01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const half2_t p23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  const int q = kk >> 1;
  return q == 0 ? p01[0] : q == 1 ? p01[1] : q == 2 ? p23[0] : p23[1];
}

// Eight codes (one dword) times a block scale as one MFMA fragment: the
// FP4 converter gives the E2M1 values (scale 1), one packed multiply per
// pair applies s_f. Every factor and the product (at most 6 significant
// bits, in [2^-10, 2688]) are exact in fp16.
__device__ __forceinline__ half8_t expand8(uint32_t w, _Float16 sf) {
  const half2_t s2 = {sf, sf};
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// The codes of this wave's kT row blocks of A and kT column blocks of B for
// one step: two uint4 per block, [0] for sub-steps 0-3 and [1] for 4-7.
template <int kT>
struct Codes {
  uint4 a[kT][2];
  uint4 b[kT][2];
};

// Scale bytes (4 per block: sub-steps 2j and 2j + 1 use byte j).
template <int kT>
struct Scales {
  uint32_t a[kT];
  uint32_t b[kT];
};

// Where this lane's fragments sit inside a stage ([kHalf] for the code
// chunks of sub-steps 0-3 and 4-7).
struct FragOffsets {
  int a_code[2], b_code[2], a_scale, b_scale;
};

template <int kT, int kHalf>
__device__ __forceinline__ void read_codes(Codes<kT>& c, const uint8_t* __restrict__ stage,
                                           const FragOffsets& o) {
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    c.a[i][kHalf] = *reinterpret_cast<const uint4*>(stage + o.a_code[kHalf] + i * 32 * kCodeStride);
    c.b[i][kHalf] = *reinterpret_cast<const uint4*>(stage + Geo<kT>::kCodeBytes + o.b_code[kHalf] +
                                                    i * 32 * kCodeStride);
  }
}

template <int kT>
__device__ __forceinline__ void read_scales(Scales<kT>& sc, const uint8_t* __restrict__ stage,
                                            const FragOffsets& o) {
  constexpr int kScales = 2 * Geo<kT>::kCodeBytes;
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    sc.a[i] = *reinterpret_cast<const uint32_t*>(stage + kScales + o.a_scale + i * 32 * kScaleStride);
    sc.b[i] = *reinterpret_cast<const uint32_t*>(stage + kScales + Geo<kT>::kScaleBytes + o.b_scale +
                                                 i * 32 * kScaleStride);
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4 (&c)[2], int kk) {
  const uint4& v = c[kk >> 2];
  switch (kk & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}

// Expands the fragments of sub-step kk.
template <int kT>
__device__ __forceinline__ void expand_substep(half8_t (&af)[kT], half8_t (&bf)[kT],
                                               const Codes<kT>& c, const Scales<kT>& sc, int kk) {
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    af[i] = expand8(dword_of(c.a[i], kk), scale_f16(sc.a[i], kk));
    bf[i] = expand8(dword_of(c.b[i], kk), scale_f16(sc.b[i], kk));
  }
}

// ---------------------------------------------------------------------------
// The kernel. kT = 4: one 256 x 256 tile per workgroup, tile
// tile_of(tile0 + blockIdx). kT = 2: one 128 x 128 quarter of 256 x 256 tile
// tile_of(tile0 + blockIdx / 4) per workgroup. The two launches of a call
// take consecutive ranges of tile_of's argument, so they cover every tile
// once.
// ---------------------------------------------------------------------------
template <int kT, bool kA2D, bool kB2D, bool kAligned, bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
  using G = Geo<kT>;
  // the ring, and after the K loop (kT = 4) the epilogue's staging of C
  constexpr int kLdsBytes = (kT == 4 && 4 * kEpilogueWaveBytes > kStages * G::kStageBytes)
                                ? 4 * kEpilogueWaveBytes
                                : kStages * G::kStageBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + kBigTile - 1) / kBigTile;
  const int64_t tiles_m = (p.M + kBigTile - 1) / kBigTile;
  int64_t m0, n0;
  if constexpr (kT == 4) {
    const int64_t t = tile_of(p.tile0 + static_cast<int64_t>(blockIdx.x), tiles_m, tiles_n);
    m0 = (t / tiles_n) * kBigTile;
    n0 = (t - (t / tiles_n) * tiles_n) * kBigTile;
  } else {
    static_assert(kT == 2, "tile configurations: 4 x 4 and 2 x 2 MFMA tiles per wave");
    const int64_t t = tile_of(p.tile0 + static_cast<int64_t>(blockIdx.x >> 2), tiles_m, tiles_n);
    const int q = blockIdx.x & 3;
    m0 = (t / tiles_n) * kBigTile + G::kTile * (q >> 1);
    n0 = (t - (t / tiles_n) * tiles_n) * kBigTile + G::kTile * (q & 1);
    if (m0 >= p.M || n0 >= p.N) return;  // quarter past a ragged edge (whole workgroup)
  }
  const int64_t K = p.K;
  const int nsteps = static_cast<int>((K + kBK - 1) / kBK);  // >= 1
  const int last = nsteps - 1;
  const int part = tid & 3;

  floatx16_t acc[kT][kT];
#pragma unroll
  for (int i = 0; i < kT; ++i)
#pragma unroll
    for (int j = 0; j < kT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Staging state: DMA addressing (kAligned) or register staging.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  DmaSource<kT> dma_a, dma_b;
  OperandSource<kT> src_a, src_b;
  Stage<kT> a_fly, b_fly;
  if constexpr (kAligned) {
    // Prologue: steps 0 and 1 into stages 0 and 1.
    dma_a = dma_source<kT, kA2D>(p.qa, p.sa, m0, p.M, K, wave_u, lane);
    dma_b = dma_source<kT, kB2D>(p.qb, p.sb, n0, p.N, K, wave_u, lane);
    dma_stage<kT>(dma_a, lds, lds + 2 * G::kCodeBytes, 0, wave_u);
    dma_stage<kT>(dma_b, lds + G::kCodeBytes, lds + 2 * G::kCodeBytes + G::kScaleBytes, 0, wave_u);
    if (nsteps > 1) {
      uint8_t* st = lds + G::kStageBytes;
      dma_stage<kT>(dma_a, st, st + 2 * G::kCodeBytes, 1, wave_u);
      dma_stage<kT>(dma_b, st + G::kCodeBytes, st + 2 * G::kCodeBytes + G::kScaleBytes, 1, wave_u);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  } else {
    // Prologue: steps 0, 1 and 2 requested together; 0 and 1 go to stages 0
    // and 1, step 2 stays in flight.
    src_a = operand_source<kT, kA2D>(p.qa, p.sa, m0, p.M, K, tid);
    src_b = operand_source<kT, kB2D>(p.qb, p.sb, n0, p.N, K, tid);
    const int s1 = 1 < last ? 1 : last;
    const int s2 = 2 < last ? 2 : last;
    const Stage<kT> a0 = load_stage<kT>(src_a, 0, K, part);
    const Stage<kT> b0 = load_stage<kT>(src_b, 0, K, part);
    const Stage<kT> a1 = load_stage<kT>(src_a, s1, K, part);
    const Stage<kT> b1 = load_stage<kT>(src_b, s1, K, part);
    a_fly = load_stage<kT>(src_a, s2, K, part);
    b_fly = load_stage<kT>(src_b, s2, K, part);
    uint8_t* st = lds + G::kStageBytes;
    store_stage<kT>(lds, lds + 2 * G::kCodeBytes, a0, tid);
    store_stage<kT>(lds + G::kCodeBytes, lds + 2 * G::kCodeBytes + G::kScaleBytes, b0, tid);
    store_stage<kT>(st, st + 2 * G::kCodeBytes, a1, tid);
    store_stage<kT>(st + G::kCodeBytes, st + 2 * G::kCodeBytes + G::kScaleBytes, b1, tid);
  }
  __syncthreads();

  const int frag_row = lane & 31;
  const int half = lane >> 5;
  const int swz = ((frag_row >> 1) ^ (frag_row >> 2)) & 3;  // same for frag_row + 32 i
  FragOffsets o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    o.a_code[h] = (wm * G::kWave + frag_row) * kCodeStride + 16 * ((2 * half + h) ^ swz);
    o.b_code[h] = (wn * G::kWave + frag_row) * kCodeStride + 16 * ((2 * half + h) ^ swz);
  }
  o.a_scale = (wm * G::kWave + frag_row) * kScaleStride + 4 * half;
  o.b_scale = (wn * G::kWave + frag_row) * kScaleStride + 4 * half;

  // Software pipeline across steps. In sub-step kk of step s the MFMAs of kk
  // run while the fragments of kk + 1 are expanded (for kk = 7: sub-step 0
  // of step s + 1). The codes of step s + 1 are read from LDS as soon as the
  // ones they replace are dead: the sub-step 0-3 halves after sub-step 2,
  // the 4-7 halves in sub-step 7. Stage s + 1 was written in step s - 1,
  // before the barrier that ended it (DMA: requested at the start of step
  // s - 1 and waited for before that barrier).
  Codes<kT> c;
  Scales<kT> sc, sc_next;
  read_codes<kT, 0>(c, lds, o);
  read_codes<kT, 1>(c, lds, o);
  read_scales<kT>(sc, lds, o);
  half8_t af[2][kT], bf[2][kT];
  expand_substep<kT>(af[0], bf[0], c, sc, 0);

  int cur = 0;  // stage holding step s
  for (int step = 0; step < nsteps; ++step) {
    const int nxt = cur == 2 ? 0 : cur + 1;  // stage of step s + 1
    const int wr = cur == 0 ? 2 : cur - 1;   // stage for step s + 2
    const uint8_t* next_stage = lds + nxt * G::kStageBytes;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int b = kk & 1;
#pragma unroll
      for (int i = 0; i < kT; ++i)
#pragma unroll
        for (int j = 0; j < kT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[b][j], af[b][i], acc[i][j], 0, 0, 0);
      if (kk < 7) {
        expand_substep<kT>(af[b ^ 1], bf[b ^ 1], c, sc, kk + 1);
      } else {
        expand_substep<kT>(af[0], bf[0], c, sc_next, 0);  // step s + 1, sub-step 0
      }
      if constexpr (kAligned) {
        if (kk == 0) {
          // step s + 2 straight into the stage that held step s - 1 (past
          // the end: the last step again, into a stage nobody reads; no
          // branch, so the region stays one block for the scheduler)
          uint8_t* st = lds + wr * G::kStageBytes;
          const int ld = (step + 2) < last ? (step + 2) : last;
          dma_stage<kT>(dma_a, st, st + 2 * G::kCodeBytes, ld, wave_u);
          dma_stage<kT>(dma_b, st + G::kCodeBytes, st + 2 * G::kCodeBytes + G::kScaleBytes, ld, wave_u);
        }
      } else {
        if (kk == 1) {
          // step s + 2 (loaded during step s - 1) into the stage that held
          // step s - 1, then request step s + 3
          uint8_t* st = lds + wr * G::kStageBytes;
          store_stage<kT>(st, st + 2 * G::kCodeBytes, a_fly, tid);
          store_stage<kT>(st + G::kCodeBytes, st + 2 * G::kCodeBytes + G::kScaleBytes, b_fly, tid);
          const int ld = (step + 3) < last ? (step + 3) : last;
          a_fly = load_stage<kT>(src_a, ld, K, part);
          b_fly = load_stage<kT>(src_b, ld, K, part);
        }
      }
      if (kk == 3) {
        read_codes<kT, 0>(c, next_stage, o);
        read_scales<kT>(sc_next, next_stage, o);
      }
      if (kk == 6) read_codes<kT, 1>(c, next_stage, o);
      // MFMAs interleaved with the expansion: kT * kT MFMAs and 2 kT
      // fragments (about 9 VALU each) per sub-step
      constexpr int kValuPerMfma = kT == 4 ? 4 : 10;
#pragma unroll
      for (int g = 0; g < kT * kT; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kAligned) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    sc = sc_next;
    cur = nxt;
  }

  // Epilogue: C = acc * (S_A * S_B). Whole lines through LDS for a 128 x 128
  // wave tile inside C with aligned rows (the loop's last barrier follows
  // its last LDS read and load).
  const float alpha = __fmul_rn(*p.ta, *p.tb);
  const int64_t r0 = m0 + wm * G::kWave, c0 = n0 + wn * G::kWave;
  if constexpr (kT == 4) {
    constexpr int kElem = kBf16Out ? 2 : 4;
    const bool lines = r0 + G::kWave <= p.M && c0 + G::kWave <= p.N && ((p.ldc * kElem) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.c) & 15) == 0;
    if (lines) {
      store_tile_lds<kBf16Out>(acc, alpha, p.c, p.ldc, r0, c0, lane, lds + wave * kEpilogueWaveBytes);
      return;
    }
  }
  store_tile<kT, kBf16Out>(acc, alpha, p.c, p.ldc, p.M, p.N, r0, c0, lane);
}

}  // namespace

namespace gemm_common {
__global__ void zero_output_kernel(void* c, int64_t M, int64_t N, int64_t ldc, bool bf16) {
  const int64_t total = M * N;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / N, col = i - r * N;
    if (bf16) static_cast<uint16_t*>(c)[r * ldc + col] = 0;
    else static_cast<float*>(c)[r * ldc + col] = 0.0f;
  }
}
}  // namespace gemm_common

namespace {

template <int kT, bool kA2D, bool kB2D>
int launch_variant(const GemmParams& p, int64_t blocks, bool aligned, bool bf16, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(blocks));
  if (aligned) {
    if (bf16) gemm_kernel<kT, kA2D, kB2D, true, true><<<grid, kThreads, 0, stream>>>(p);
    else gemm_kernel<kT, kA2D, kB2D, true, false><<<grid, kThreads, 0, stream>>>(p);
  } else {
    if (bf16) gemm_kernel<kT, kA2D, kB2D, false, true><<<grid, kThreads, 0, stream>>>(p);
    else gemm_kernel<kT, kA2D, kB2D, false, false><<<grid, kThreads, 0, stream>>>(p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int kT>
int launch_tiles(const GemmParams& p, int64_t blocks, bool a_2d, bool b_2d, bool aligned, bool bf16,
                 hipStream_t stream) {
  if (a_2d) {
    return b_2d ? launch_variant<kT, true, true>(p, blocks, aligned, bf16, stream)
                : launch_variant<kT, true, false>(p, blocks, aligned, bf16, stream);
  }
  return b_2d ? launch_variant<kT, false, true>(p, blocks, aligned, bf16, stream)
              : launch_variant<kT, false, false>(p, blocks, aligned, bf16, stream);
}

}  // namespace

int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int launch_gemm(const GemmLaunch& g, hipStream_t stream) {
  if (g.K == 0) {
    int64_t blocks = (g.M * g.N + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    zero_output_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(g.c, g.M, g.N, g.ldc,
                                                                           g.c_bf16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  GemmParams p;
  p.qa = g.qa;
  p.sa = g.sa;
  p.qb = g.qb;
  p.sb = g.sb;
  p.ta = g.ta;
  p.tb = g.tb;
  p.c = g.c;
  p.M = g.M;
  p.N = g.N;
  p.K = g.K;
  p.ldc = g.ldc;
  const bool aligned = (g.K % kBK) == 0;
  // 256 x 256 tiles, one workgroup per CU; a last round that would fill at
  // most a quarter of the CUs runs as 128 x 128 quarters instead.
  const int64_t tiles = ((g.M + kBigTile - 1) / kBigTile) * ((g.N + kBigTile - 1) / kBigTile);
  const int64_t cus = device_compute_units();
  const int64_t rem = cus > 0 ? tiles % cus : 0;
  const int64_t tail = (rem > 0 && 4 * rem <= cus) ? rem : 0;
  const int64_t main_tiles = tiles - tail;
  if (main_tiles > 0) {
    p.tile0 = 0;
    if (launch_tiles<4>(p, main_tiles, g.a_2d, g.b_2d, aligned, g.c_bf16, stream) != 0) return -1;
  }
  if (tail > 0) {
    p.tile0 = main_tiles;
    if (launch_tiles<2>(p, 4 * tail, g.a_2d, g.b_2d, aligned, g.c_bf16, stream) != 0) return -1;
  }
  return 0;
}

}  // namespace nvfp4
