// NVFP4 dequantization for gfx950: x_hat = (e2m1(q) * s_f) * S, float32 or
// bf16 (round to nearest even) output. The format is the one of the
// gist.science summary of "Pretraining Large Language Models with NVFP4",
// Resumen técnico §2 "Formato NVFP4".
//
// A wave expands 64 consecutive 16-byte pieces of one output row: 8 values
// per lane for bf16 output, 4 for float32, so each store instruction writes
// 1 KiB of contiguous output (whole 128-byte lines). A lane reads the 4 (or
// 2) code bytes of its values and its block's scale byte. The E2M1 values
// come from gfx950's FP4 -> float32 converter with scale 1.0 (exact), then
// two float32 multiplies in the order of the definition; bf16 output is the
// RNE of that float32, two values per conversion.
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

using gemm_common::f32x2_to_bf16x2;

typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;  // rows per workgroup (one per wave)

template <bool kBlock2D, bool kBf16>
__global__ __launch_bounds__(64 * kWaves) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                                 const uint8_t* __restrict__ sc,
                                                                 const float* __restrict__ tensor_scale,
                                                                 int64_t rows, int64_t cols, void* y,
                                                                 int64_t ldy, int64_t chunks, int64_t units) {
  constexpr int kPerLane = kBf16 ? 8 : 4;  // values per lane: 16 bytes of output
  constexpr int kChunk = 64 * kPerLane;    // values per wave
  const float s = *tensor_scale;
  const int64_t nbc = cols >> 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // unit u: rows 4 (u / chunks) .. + 3, columns kChunk (u % chunks) .. + kChunk - 1
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t rg = u / chunks;
    const int64_t row = rg * kWaves + wave;
    const int64_t col = (u - rg * chunks) * kChunk + lane * kPerLane;
    if (row >= rows || col >= cols) continue;
    const uint32_t sbyte = kBlock2D ? sc[(row >> 4) * nbc + (col >> 4)] : sc[row * nbc + (col >> 4)];
    const float sf = e4m3_to_float(sbyte);
    const uint8_t* qp = q + row * (cols >> 1) + (col >> 1);
    float v[kPerLane];
    if constexpr (kBf16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(qp);
      const float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      const float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      const float2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
      const float2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
      const float e[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __fmul_rn(__fmul_rn(e[j], sf), s);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + row * ldy + col) =
          make_uint4(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]), f32x2_to_bf16x2(v[4], v[5]),
                     f32x2_to_bf16x2(v[6], v[7]));
    } else {
      const uint32_t w = *reinterpret_cast<const uint16_t*>(qp);
      const float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      const float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      const float e[4] = {p0[0], p0[1], p1[0], p1[1]};
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(__fmul_rn(e[j], sf), s);
      *reinterpret_cast<float4*>(static_cast<float*>(y) + row * ldy + col) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

}  // namespace

int launch_dequantize(const uint8_t* q, const uint8_t* s, const float* tensor_scale, int64_t rows,
                      int64_t cols, bool block_2d, bool out_bf16, void* y, int64_t ldy,
                      hipStream_t stream) {
  if (rows == 0 || cols == 0) return 0;
  const int64_t chunk = out_bf16 ? 512 : 256;
  const int64_t chunks = (cols + chunk - 1) / chunk;
  const int64_t units = ((rows + kWaves - 1) / kWaves) * chunks;
  const unsigned g = static_cast<unsigned>(units < (int64_t(1) << 20) ? units : (int64_t(1) << 20));
  const unsigned t = 64 * kWaves;
  if (block_2d) {
    if (out_bf16) dequantize_kernel<true, true><<<g, t, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy, chunks, units);
    else dequantize_kernel<true, false><<<g, t, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy, chunks, units);
  } else {
    if (out_bf16) dequantize_kernel<false, true><<<g, t, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy, chunks, units);
    else dequantize_kernel<false, false><<<g, t, 0, stream>>>(q, s, tensor_scale, rows, cols, y, ldy, chunks, units);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
