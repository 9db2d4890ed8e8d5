// NVFP4 dequantization for gfx950: x_hat = (e2m1(q) * s_f) * S, float32 or
// bf16 (round to nearest even) output. The format is the one of the
// gist.science summary of "Pretraining Large Language Models with NVFP4",
// Resumen técnico §2 "Formato NVFP4".
//
// One thread expands one 16-element block: 8 code bytes and 1 scale byte in,
// 64 (float32) or 32 (bf16) bytes out.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

// Value of a 4-bit E2M1 code from its bit fields.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = (e == 0u) ? 0.5f * static_cast<float>(m)
                              : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return __uint_as_float(__float_as_uint(mag) | ((c & 8u) << 28));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <bool kBlock2D, bool kBf16>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ sc,
                                                         const float* __restrict__ tensor_scale,
                                                         int64_t rows, int64_t cols, void* y,
                                                         int64_t ldy) {
  const int64_t nbc = cols >> 4;
  const int64_t total = rows * nbc;
  const float s = *tensor_scale;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < total;
       b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = b / nbc, cb = b - r * nbc;
    const uint2 codes = *reinterpret_cast<const uint2*>(q + r * (cols >> 1) + cb * 8);
    const uint32_t sbyte = kBlock2D ? sc[(r >> 4) * nbc + cb] : sc[r * nbc + cb];
    const float sf = e4m3_to_float(sbyte);
    float out[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t word = (j < 8) ? codes.x : codes.y;
      const uint32_t c = (word >> (4 * (j & 7))) & 0xFu;
      out[j] = __fmul_rn(__fmul_rn(e2m1_value(c), sf), s);
    }
    if constexpr (kBf16) {
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + r * ldy + cb * 16);
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        w[k] = f32_to_bf16_rne(out[2 * k]) | (f32_to_bf16_rne(out[2 * k + 1]) << 16);
      }
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + r * ldy + cb * 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dst[k] = make_float4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
      }
    }
  }
}

}  // namespace

int launch_dequantize(const uint8_t* q, const uint8_t* s, const float* tensor_scale, int64_t rows,
                      int64_t cols, bool block_2d, bool out_bf16, void* y, int64_t ldy,
                      hipStream_t stream) {
  const int64_t total = rows * (cols >> 4);
  if (total == 0) return 0;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const unsigned g = static_cast<unsigned>(blocks);
  if (block_2d) {
    if (out_bf16) dequantize_kernel<true, true><<<g, 256, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy);
    else dequantize_kernel<true, false><<<g, 256, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy);
  } else {
    if (out_bf16) dequantize_kernel<false, true><<<g, 256, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy);
    else dequantize_kernel<false, false><<<g, 256, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
