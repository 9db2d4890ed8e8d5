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
// Per 64-wide K step, each thread loads one row's 32 code bytes of A and of
// B (plus their scale bytes) from global memory, expands them to fp16 with
// the gfx950 FP4 -> fp16 converter (exact) and one packed fp16 multiply by
// the block scale (exact), and writes them to one of two LDS buffers; the
// MFMAs of the current step read the other buffer. So every element is
// dequantized once per workgroup, and global loads of step k+1 overlap the
// MFMAs of step k.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;                 // K elements per step (4 scale blocks)
constexpr int kThreads = 256;
constexpr int kWaveM = 128;             // rows of C per wave
constexpr int kWaveN = 128;             // columns of C per wave
constexpr int kLdsStride = kBK + 8;     // fp16 elements per LDS row (+16 B pad)
constexpr int kTileHalves = kBM * kLdsStride;

struct GemmParams {
  const uint8_t* qa;
  const uint8_t* sa;
  const uint8_t* qb;
  const uint8_t* sb;
  const float* ta;
  const float* tb;
  void* c;
  int64_t M, N, K, ldc;
};

// Codes (32 bytes = 64 values) and the 4 scale bytes of one row of one K
// step, as loaded from global memory.
struct RowStage {
  uint4 codes[2];
  uint32_t scales;  // byte j: scale of values [16j, 16j + 16)
};

template <bool k2D, bool kAligned>
__device__ __forceinline__ RowStage load_row(const uint8_t* __restrict__ q,
                                             const uint8_t* __restrict__ s, int64_t row,
                                             int64_t rows, int64_t K, int64_t k0) {
  RowStage st;
  st.codes[0] = make_uint4(0, 0, 0, 0);
  st.codes[1] = make_uint4(0, 0, 0, 0);
  st.scales = 0;
  if (row >= rows) return st;
  const int64_t kb = K >> 4;                     // scale bytes per row
  const int64_t srow = k2D ? (row >> 4) : row;   // scale row
  const uint8_t* qp = q + row * (K >> 1) + (k0 >> 1);
  const uint8_t* sp = s + srow * kb + (k0 >> 4);
  if constexpr (kAligned) {
    // K % 64 == 0: code rows start on 32-byte and scale rows on 4-byte
    // boundaries, and there is no K tail
    st.codes[0] = *reinterpret_cast<const uint4*>(qp);
    st.codes[1] = *reinterpret_cast<const uint4*>(qp + 16);
    st.scales = *reinterpret_cast<const uint32_t*>(sp);
  } else {
    // rows are only 8-byte aligned; the last step may hold 16, 32 or 48 values
    const int64_t left = K - k0;
    const int nblk = left >= kBK ? 4 : static_cast<int>(left >> 4);
    const uint2* q8 = reinterpret_cast<const uint2*>(qp);
    uint2 part[4] = {make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0)};
    uint32_t sc = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nblk) {
        part[b] = q8[b];
        sc |= static_cast<uint32_t>(sp[b]) << (8 * b);
      }
    }
    st.codes[0] = make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
    st.codes[1] = make_uint4(part[2].x, part[2].y, part[3].x, part[3].y);
    st.scales = sc;
  }
  return st;
}

// fp16 value of an E4M3 scale byte (exact).
__device__ __forceinline__ _Float16 scale_f16(uint32_t byte) {
  return static_cast<_Float16>(e4m3_to_float(byte & 0xFFu));
}

// Expands 8 code bytes (16 values) times a block scale into two half8.
__device__ __forceinline__ void expand16(uint32_t w0, uint32_t w1, _Float16 sf, half8_t& lo,
                                         half8_t& hi) {
  const half2_t s2 = {sf, sf};
  half2_t h[8];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * s2;
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * s2;
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * s2;
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * s2;
  h[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0) * s2;
  h[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1) * s2;
  h[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) * s2;
  h[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) * s2;
  lo = half8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
  hi = half8_t{h[4][0], h[4][1], h[5][0], h[5][1], h[6][0], h[6][1], h[7][0], h[7][1]};
}

// Writes one row stage (64 values) into an LDS tile row.
__device__ __forceinline__ void store_row(_Float16* __restrict__ lds_row, const RowStage& st) {
  const uint32_t w[8] = {st.codes[0].x, st.codes[0].y, st.codes[0].z, st.codes[0].w,
                         st.codes[1].x, st.codes[1].y, st.codes[1].z, st.codes[1].w};
  half8_t* dst = reinterpret_cast<half8_t*>(lds_row);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    half8_t lo, hi;
    expand16(w[2 * b], w[2 * b + 1], scale_f16(st.scales >> (8 * b)), lo, hi);
    dst[2 * b] = lo;
    dst[2 * b + 1] = hi;
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return (b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <bool kA2D, bool kB2D, bool kAligned, bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[4 * kTileHalves];
  _Float16* lds_a = lds;                      // [2][kBM][kLdsStride]
  _Float16* lds_b = lds + 2 * kTileHalves;    // [2][kBN][kLdsStride]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + kBN - 1) / kBN;
  const int64_t bm = static_cast<int64_t>(blockIdx.x) / tiles_n;
  const int64_t bn = static_cast<int64_t>(blockIdx.x) - bm * tiles_n;
  const int64_t m0 = bm * kBM, n0 = bn * kBN;
  const int64_t K = p.K;
  const int nsteps = static_cast<int>((K + kBK - 1) / kBK);

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Thread tid stages row tid of the A tile and row tid of the B tile.
  RowStage sa_st = load_row<kA2D, kAligned>(p.qa, p.sa, m0 + tid, p.M, K, 0);
  RowStage sb_st = load_row<kB2D, kAligned>(p.qb, p.sb, n0 + tid, p.N, K, 0);
  if (nsteps > 0) {
    store_row(lds_a + tid * kLdsStride, sa_st);
    store_row(lds_b + tid * kLdsStride, sb_st);
  }
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      const int64_t k1 = static_cast<int64_t>(step + 1) * kBK;
      sa_st = load_row<kA2D, kAligned>(p.qa, p.sa, m0 + tid, p.M, K, k1);
      sb_st = load_row<kB2D, kAligned>(p.qb, p.sb, n0 + tid, p.N, K, k1);
    }
    const _Float16* a_tile = lds_a + cur * kTileHalves + (wm * kWaveM + frag_row) * kLdsStride + frag_k;
    const _Float16* b_tile = lds_b + cur * kTileHalves + (wn * kWaveN + frag_row) * kLdsStride + frag_k;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      half8_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const half8_t*>(a_tile + i * 32 * kLdsStride + kk);
        bf[i] = *reinterpret_cast<const half8_t*>(b_tile + i * 32 * kLdsStride + kk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      const int nxt = cur ^ 1;
      store_row(lds_a + nxt * kTileHalves + tid * kLdsStride, sa_st);
      store_row(lds_b + nxt * kTileHalves + tid * kLdsStride, sb_st);
    }
    __syncthreads();
  }

  // Epilogue: C = acc * (S_A * S_B); lane holds column lane % 32 and rows
  // 8 * (e / 4) + 4 * (lane / 32) + e % 4 of each 32 x 32 tile.
  const float scale = __fmul_rn(*p.ta, *p.tb);
  const int col_l = lane & 31;
  const int row_l = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * kWaveN + j * 32 + col_l;
      if (col >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * kWaveM + i * 32 + (e >> 2) * 8 + row_l + (e & 3);
        if (row < p.M) {
          const float v = __fmul_rn(acc[i][j][e], scale);
          if constexpr (kBf16Out) {
            static_cast<uint16_t*>(p.c)[row * p.ldc + col] = static_cast<uint16_t>(f32_to_bf16_bits(v));
          } else {
            static_cast<float*>(p.c)[row * p.ldc + col] = v;
          }
        }
      }
    }
  }
}

__global__ void zero_output_kernel(void* c, int64_t M, int64_t N, int64_t ldc, bool bf16) {
  const int64_t total = M * N;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / N, col = i - r * N;
    if (bf16) static_cast<uint16_t*>(c)[r * ldc + col] = 0;
    else static_cast<float*>(c)[r * ldc + col] = 0.0f;
  }
}

template <bool kA2D, bool kB2D, bool kAligned, bool kBf16>
int launch_variant(const GemmParams& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN);
  gemm_kernel<kA2D, kB2D, kAligned, kBf16><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool kA2D, bool kB2D>
int launch_blocks(const GemmParams& p, bool aligned, bool bf16, hipStream_t stream) {
  if (aligned) {
    return bf16 ? launch_variant<kA2D, kB2D, true, true>(p, stream)
                : launch_variant<kA2D, kB2D, true, false>(p, stream);
  }
  return bf16 ? launch_variant<kA2D, kB2D, false, true>(p, stream)
              : launch_variant<kA2D, kB2D, false, false>(p, stream);
}

}  // namespace

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
  const bool aligned = (g.K % 64) == 0;
  if (g.a_2d) {
    return g.b_2d ? launch_blocks<true, true>(p, aligned, g.c_bf16, stream)
                  : launch_blocks<true, false>(p, aligned, g.c_bf16, stream);
  }
  return g.b_2d ? launch_blocks<false, true>(p, aligned, g.c_bf16, stream)
                : launch_blocks<false, false>(p, aligned, g.c_bf16, stream);
}

}  // namespace nvfp4
