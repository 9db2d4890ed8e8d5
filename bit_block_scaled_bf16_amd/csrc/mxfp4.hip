// MXFP4, the comparison format of the pages, for gfx950: a 1x32 quantizer
// and its dequantizer (the GEMM on the block-scaled FP4 MFMA is in
// f8f6f4_gemm.hip).
//
// Source: gist.science summary of "Pretraining Large Language Models with
// NVFP4", Resumen técnico §2 "Formato NVFP4" (MXFP4 uses blocks of 32
// elements, NVFP4 blocks of 16) and §1 (MXFP4's coarser scales). The format:
// E2M1 codes, one E8M0 scale 2^(b - 127) per 32 elements along a row, b
// chosen so the block amax maps into [4, 8), round to nearest even, no
// tensor scale. Codes are packed as NVFP4's (even element in the low nibble).
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

using gemm_common::f32x2_to_bf16x2;

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

}  // namespace nvfp4
