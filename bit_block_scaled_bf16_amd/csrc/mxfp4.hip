// MXFP4, the comparison format of the pages, for gfx950: a 1x32 quantizer,
// its dequantizer, and a GEMM on the chip's block-scaled FP4 MFMA.
//
// Source: gist.science summary of "Pretraining Large Language Models with
// NVFP4", Resumen técnico §2 "Formato NVFP4" (MXFP4 uses blocks of 32
// elements, NVFP4 blocks of 16) and §1 (MXFP4's coarser scales). The format:
// E2M1 codes, one E8M0 scale 2^(b - 127) per 32 elements along a row, b
// chosen so the block amax maps into [4, 8), round to nearest even, no
// tensor scale. Codes are packed as NVFP4's (even element in the low nibble).
//
// GEMM. v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands multiplies a
// 32 x 64 slice of A by a 32 x 64 slice of B with one E8M0 scale per row
// and 32 K: lane l supplies row l % 32 and the 32 K values of half l / 32
// (16 bytes) plus that block's scale byte. This is MXFP4's own definition,
// so the codes and scale bytes go to the MFMA as stored: no expansion, and
// the relevant peak is dense FP4 (10.1 PFLOP/s). The staging (256 x 256
// tile, 4 waves of 128 x 128, K steps of 128 into an LDS ring filled by
// global_load_lds, XOR-swizzled 64-byte code rows) is the NVFP4 GEMM's; a
// step is 2 MFMA sub-steps of K = 64 instead of 8 of K = 16, a quarter of
// the time, so the ring has 4 stages and a step's loads are requested 4
// steps ahead (the wait before a step's barrier leaves the 2 newest steps'
// loads in flight). Lane
// half h takes K [64h, 64h + 64) of a step, sub-step s its 32 values from
// 64h + 32s, so its two scale bytes of the step are adjacent and one 16-bit
// LDS read serves both sub-steps (the MFMA's op_sel picks the byte).
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

using namespace gemm_common;

constexpr int kMxBlock = 32;

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                                                __builtin_bit_cast(ushort2_t, b)));
}

// ---------------------------------------------------------------------------
// Quantize / dequantize: one thread per 32-element block; a workgroup of 256
// threads covers 8 rows x 32 consecutive blocks of a row (2 KiB of bf16 per
// row), and walks rows in steps of 8 * gridDim.y.
// ---------------------------------------------------------------------------
template <typename InT>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const InT* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ldx,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
  const int64_t nblk = cols / kMxBlock;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x & 31);
  if (blk >= nblk) return;  // no barrier in this kernel
  for (int64_t row = static_cast<int64_t>(blockIdx.y) * 8 + (threadIdx.x >> 5); row < rows;
       row += static_cast<int64_t>(gridDim.y) * 8) {
    const InT* src = x + row * ldx + blk * kMxBlock;
    float v[32];
    uint32_t amax_bits;
    if constexpr (sizeof(InT) == 2) {
      uint4 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = reinterpret_cast<const uint4*>(src)[i];
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          m = max_u16x2(m, w[k] & 0x7FFF7FFFu);
          v[8 * i + 2 * k] = bf16_lo(w[k]);
          v[8 * i + 2 * k + 1] = bf16_hi(w[k]);
        }
      }
      const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
      amax_bits = (lo > hi ? lo : hi) << 16;
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = reinterpret_cast<const float4*>(src)[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t a = abs_bits(v[i]);
        m = a > m ? a : m;
      }
      amax_bits = m;
    }
    // floor(log2 amax) is the float32 exponent field minus 127 (subnormal
    // and zero amax have field 0 and clamp to b = 0 like the definition)
    const uint32_t field = amax_bits >> 23;
    const uint32_t b = field > 2u ? field - 2u : 0u;
    const float mult = __uint_as_float((254u - b) << 23);  // 2^(127 - b), a normal float32
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = __fmul_rn(v[8 * i + j], mult);  // exact
      w[i] = pack8_rn(y);
    }
    *reinterpret_cast<uint4*>(q + row * (cols >> 1) + blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    s[row * nblk + blk] = static_cast<uint8_t>(b);
  }
}

typedef float float2_t __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void mx_dequantize_kernel(const uint8_t* __restrict__ q,
                                                            const uint8_t* __restrict__ s,
                                                            int64_t rows, int64_t cols,
                                                            bool out_bf16, void* __restrict__ y,
                                                            int64_t ldy) {
  const int64_t nblk = cols / kMxBlock;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x & 31);
  if (blk >= nblk) return;
  for (int64_t row = static_cast<int64_t>(blockIdx.y) * 8 + (threadIdx.x >> 5); row < rows;
       row += static_cast<int64_t>(gridDim.y) * 8) {
    const uint4 c = *reinterpret_cast<const uint4*>(q + row * (cols >> 1) + blk * 16);
    const uint32_t b = s[row * nblk + blk];
    // 2^(b - 127): the float32 with exponent field b; b = 0 is the subnormal 2^-127
    const float scale = __uint_as_float(b != 0u ? (b << 23) : 0x00400000u);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the converter with scale 1 gives the exact E2M1 values
      const float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
      const float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
      const float2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
      const float2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
      const float e[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * i + j] = __fmul_rn(e[j], scale);  // exact
    }
    if (out_bf16) {
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + row * ldy + blk * kMxBlock);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[i] = make_uint4(f32x2_to_bf16x2(v[8 * i], v[8 * i + 1]), f32x2_to_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                            f32x2_to_bf16x2(v[8 * i + 4], v[8 * i + 5]), f32x2_to_bf16x2(v[8 * i + 6], v[8 * i + 7]));
      }
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + row * ldy + blk * kMxBlock);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM.
// ---------------------------------------------------------------------------
constexpr int kBK = 128;                  // K elements per step
constexpr int kThreads = 256;
constexpr int kStages = 4;                // DMA runs 4 steps ahead (a step is short)
constexpr int kTile = 256;                // C rows and columns per workgroup
constexpr int kWave = 128;                // C rows and columns per wave
constexpr int kCodeStride = kBK / 2;      // 64 bytes per LDS code row
constexpr int kScaleStride = kBK / 32;    // 4 scale bytes per LDS row
constexpr int kCodeBytes = kTile * kCodeStride;
constexpr int kScaleBytes = kTile * kScaleStride;
constexpr int kStageBytes = 2 * kCodeBytes + 2 * kScaleBytes;

typedef int int8v_t __attribute__((ext_vector_type(8)));

struct MxGemmParams {
  const uint8_t *qa, *sa, *qb, *sb;
  void* c;
  int64_t M, N, K, ldc;
};

// This lane's share of one operand's DMA per step: 4 code chunks (rows
// 64 w + 16 i + l / 4, LDS position l % 4) and the 4 scale bytes of row
// 64 w + l. Rows past the end are clamped (they only feed C outside M x N).
struct MxDmaSource {
  const uint8_t* q[4];
  const uint8_t* s;
};

__device__ __forceinline__ MxDmaSource mx_dma_source(const uint8_t* __restrict__ q,
                                                     const uint8_t* __restrict__ s, int64_t row0,
                                                     int64_t rows, int64_t K, int wave, int lane) {
  MxDmaSource d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * wave + 16 * i + (lane >> 2);
    const int64_t row = row0 + r;
    const int64_t rc = row < rows ? row : rows - 1;
    d.q[i] = q + rc * (K >> 1) + 16 * chunk_pos(r, lane & 3);
  }
  const int64_t row = row0 + 64 * wave + lane;
  const int64_t rc = row < rows ? row : rows - 1;
  d.s = s + rc * (K / kMxBlock);
  return d;
}

__device__ __forceinline__ void mx_dma_stage(const MxDmaSource& d, const uint8_t* codes,
                                             const uint8_t* scales, int step, int wave) {
  const int64_t k0 = static_cast<int64_t>(step) * kBK;
  const uint32_t c0 = lds_address(codes) + 64 * wave * kCodeStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) lds_dma<16>(d.q[i] + (k0 >> 1), c0 + 16 * i * kCodeStride);
  lds_dma<4>(d.s + k0 / kMxBlock, lds_address(scales) + 64 * wave * kScaleStride);
}

// The fragments of one step: codes [row or column block][sub-step] and the
// two scale bytes of each block (byte s for sub-step s).
struct MxFrags {
  uint4 a[4][2], b[4][2];
  uint32_t sa[4], sb[4];
};

struct MxOffsets {
  int a_code[2], b_code[2], a_scale, b_scale;
};

__device__ __forceinline__ void mx_read_frags(MxFrags& f, const uint8_t* __restrict__ stage,
                                              const MxOffsets& o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f.a[i][s] = *reinterpret_cast<const uint4*>(stage + o.a_code[s] + i * 32 * kCodeStride);
      f.b[i][s] = *reinterpret_cast<const uint4*>(stage + kCodeBytes + o.b_code[s] + i * 32 * kCodeStride);
    }
    f.sa[i] = *reinterpret_cast<const uint16_t*>(stage + 2 * kCodeBytes + o.a_scale + i * 32 * kScaleStride);
    f.sb[i] = *reinterpret_cast<const uint16_t*>(stage + 2 * kCodeBytes + kScaleBytes + o.b_scale +
                                                 i * 32 * kScaleStride);
  }
}

__device__ __forceinline__ int8v_t as_operand(const uint4& v) {
  return int8v_t{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
                 static_cast<int>(v.w), 0, 0, 0, 0};
}

template <int kS>
__device__ __forceinline__ void mx_substep(floatx16_t (&acc)[4][4], const MxFrags& f) {
  // FP4 (E2M1) operands: format code 4 for both; op_sel kS picks the scale
  // byte of sub-step kS. B goes first, so each accumulator tile is C^T.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          as_operand(f.b[j][kS]), as_operand(f.a[i][kS]), acc[i][j], 4, 4, kS,
          static_cast<int>(f.sb[j]), kS, static_cast<int>(f.sa[i]));
}

// s_waitcnt immediate: at most n vector memory loads outstanding (vmcnt is
// 6 bits, split over bits 3:0 and 15:14), expcnt and lgkmcnt not waited for.
constexpr int wait_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
constexpr int kDmaPerStep = 2 * (4 + 1);  // per wave: 4 code and 1 scale loads per operand

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void mx_gemm_kernel(MxGemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + kTile - 1) / kTile;
  const int64_t t = blockIdx.x;
  const int64_t m0 = (t / tiles_n) * kTile, n0 = (t - (t / tiles_n) * tiles_n) * kTile;
  const int64_t K = p.K;
  const int nsteps = static_cast<int>(K / kBK);  // >= 1 (K % 128 == 0, K > 0)
  const int last = nsteps - 1;

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const MxDmaSource da = mx_dma_source(p.qa, p.sa, m0, p.M, K, wave_u, lane);
  const MxDmaSource db = mx_dma_source(p.qb, p.sb, n0, p.N, K, wave_u, lane);
  // prologue: steps 0-3 into stages 0-3; steps 0 and 1 must have landed
#pragma unroll
  for (int q = 0; q < kStages; ++q) {
    uint8_t* st = lds + q * kStageBytes;
    const int ld = q < last ? q : last;
    mx_dma_stage(da, st, st + 2 * kCodeBytes, ld, wave_u);
    mx_dma_stage(db, st + kCodeBytes, st + 2 * kCodeBytes + kScaleBytes, ld, wave_u);
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kDmaPerStep));
  __syncthreads();

  const int frag_row = lane & 31;
  const int half = lane >> 5;
  const int swz = ((frag_row >> 1) ^ (frag_row >> 2)) & 3;  // same for frag_row + 32 i
  MxOffsets o;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    o.a_code[s] = (wm * kWave + frag_row) * kCodeStride + 16 * ((2 * half + s) ^ swz);
    o.b_code[s] = (wn * kWave + frag_row) * kCodeStride + 16 * ((2 * half + s) ^ swz);
  }
  o.a_scale = (wm * kWave + frag_row) * kScaleStride + 2 * half;
  o.b_scale = (wn * kWave + frag_row) * kScaleStride + 2 * half;

  // Step s reads step s + 1's fragments from LDS (landed before the barrier
  // that ended step s - 1) while its own MFMAs run, and requests step s + 4
  // into stage s % 4: step s's own fragments were read during step s - 1,
  // before that barrier (for step 0: before the second prologue barrier).
  // Before a step's barrier, step s + 2 must have landed; the loads of steps
  // s + 3 and s + 4 stay in flight (loads complete in issue order).
  MxFrags cur, nxt;
  mx_read_frags(cur, lds, o);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int stage = step & (kStages - 1);
    const int sn = (step + 1) & (kStages - 1);
    // the LDS reads go first: the DMA's inline assembly is a compiler
    // memory barrier, and reads placed after it would sink below the MFMAs
    mx_read_frags(nxt, lds + sn * kStageBytes, o);
    {
      uint8_t* st = lds + stage * kStageBytes;
      const int ld = (step + kStages) < last ? (step + kStages) : last;
      mx_dma_stage(da, st, st + 2 * kCodeBytes, ld, wave_u);
      mx_dma_stage(db, st + kCodeBytes, st + 2 * kCodeBytes + kScaleBytes, ld, wave_u);
    }
    mx_substep<0>(acc, cur);
    mx_substep<1>(acc, cur);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kDmaPerStep));
    __syncthreads();
    cur = nxt;
  }
  store_tile<4, kBf16Out>(acc, 1.0f, p.c, p.ldc, p.M, p.N, m0 + wm * kWave, n0 + wn * kWave, lane);
}

}  // namespace

int launch_mx_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                       uint8_t* q, uint8_t* s, hipStream_t stream) {
  const int64_t nblk = cols / kMxBlock;
  const int64_t gy = (rows + 7) / 8;
  const dim3 grid(static_cast<unsigned>((nblk + 31) / 32), static_cast<unsigned>(gy < 65535 ? gy : 65535));
  if (x_bf16) {
    mx_quantize_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(x), rows, cols,
                                                          ldx, q, s);
  } else {
    mx_quantize_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), rows, cols, ldx,
                                                       q, s);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                         bool out_bf16, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t nblk = cols / kMxBlock;
  const int64_t gy = (rows + 7) / 8;
  const dim3 grid(static_cast<unsigned>((nblk + 31) / 32), static_cast<unsigned>(gy < 65535 ? gy : 65535));
  mx_dequantize_kernel<<<grid, 256, 0, stream>>>(q, s, rows, cols, out_bf16, y, ldy);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                   int64_t M, int64_t N, int64_t K, void* c, bool c_bf16, int64_t ldc,
                   hipStream_t stream) {
  if (K == 0) {
    int64_t blocks = (M * N + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    zero_output_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(c, M, N, ldc, c_bf16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  MxGemmParams p{qa, sa, qb, sb, c, M, N, K, ldc};
  const int64_t tiles = ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
  if (c_bf16) mx_gemm_kernel<true><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
  else mx_gemm_kernel<false><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
