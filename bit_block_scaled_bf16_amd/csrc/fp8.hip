// FP8 (E4M3FN, one float32 scale per tensor), the baseline format of the
// pages, for gfx950: a quantizer with a row copy and a transposed column
// copy, and its dequantizer (the GEMM is in f8f6f4_gemm.hip).
//
// Sources: gist.science summary of "Pretraining Large Language Models with
// NVFP4", Resumen técnico §1 and §4 (NVFP4 measured against FP8);
// deultimominuto.info, "Cómo funciona NVFP4" (E4M3: 4 exponent and 3
// mantissa bits). The scaling follows the library's definitions stated in
// include/nvfp4.h: S8 = fp32(amax / 448) (1 below 2^-100), r = fp32(1 / S8),
// y = fp32(x * r), byte = E4M3FN nearest to y, ties to even, saturating at
// +-448, sign of y kept.
//
// Quantizer. One workgroup per 64 x 256 tile. Thread (rg = tid / 16,
// cg = tid % 16) owns rows 4 rg .. 4 rg + 3 and columns 16 cg .. 16 cg + 15:
// per row one or two 16-byte loads (16 threads cover a row's 256 values
// contiguously) and one 16-byte store of the row copy. For the column copy
// the thread transposes its 4 x 16 bytes in registers (byte permutes) into
// 16 words, one per column holding its 4 rows, stages them in LDS as
// [column][64 rows], and then writes one column's 64 bytes. Tiles are
// numbered down the columns of tiles and handed to the XCDs in contiguous
// runs, so the two tiles that write the halves of a column-copy line are
// usually behind the same L2.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 64;
constexpr int kTileCols = 256;
constexpr float kE4M3Max = 448.0f;
constexpr int kXcds = 8;

__device__ __forceinline__ float fp8_scale_from_amax(float amax) {
  const float s = __fdiv_rn(amax, kE4M3Max);
  return (s < kTensorScaleFloor) ? 1.0f : s;  // also maps amax == 0 to 1
}

// Four E4M3FN bytes (a in byte 0) of values already multiplied by r.
// gfx950's converter rounds to nearest even into OCP E4M3FN and keeps the
// sign, but turns magnitudes above 464 into NaN; clamping to +-448 first
// gives the format's saturation.
__device__ __forceinline__ float clamp448(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max);
}

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return static_cast<uint32_t>(w);
}

// One thread's 4 rows x 16 values as loaded.
template <typename InT>
struct Rows4;

template <>
struct Rows4<uint16_t> {
  uint4 r[4][2];
  __device__ __forceinline__ float get(int i, int j) const {
    const uint4& v = r[i][j >> 3];
    const int k = (j >> 1) & 3;
    const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};

template <>
struct Rows4<float> {
  float4 r[4][4];
  __device__ __forceinline__ float get(int i, int j) const {
    const float4& v = r[i][j >> 2];
    return (j & 3) == 0 ? v.x : (j & 3) == 1 ? v.y : (j & 3) == 2 ? v.z : v.w;
  }
};

template <typename InT>
__device__ __forceinline__ void load_rows(const InT* __restrict__ x, int64_t ldx, int64_t r0,
                                          int64_t c0, int64_t rows, bool col_ok, Rows4<InT>& t) {
  constexpr int kLoads = sizeof(InT) == 2 ? 2 : 4;  // 16-byte loads per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = col_ok && (r0 + i) < rows;
    const uint4* src = reinterpret_cast<const uint4*>(x + (r0 + i) * ldx + c0);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const uint4 v = ok ? src[k] : make_uint4(0u, 0u, 0u, 0u);
      if constexpr (sizeof(InT) == 2) {
        t.r[i][k] = v;
      } else {
        t.r[i][k] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                __uint_as_float(v.w));
      }
    }
  }
}

// Word q (0..3) of a 16-byte vector.
__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

struct Fp8Params {
  const void* x;
  int64_t rows, cols, ldx;
  const float* amax_in;
  const uint32_t* partials;
  int n_partials;
  float* amax_out;
  float* tensor_scale;
  int32_t* dev_status;
  uint8_t *q_row, *q_col;
  int outputs;
};

template <typename InT>
__global__ __launch_bounds__(kThreads) void fp8_quantize_kernel(Fp8Params p) {
  // column copy staging: [column][16 words of 4 rows], columns of odd
  // 16-column groups swapped in pairs and word g of column c stored at
  // g ^ 2 ((c >> 5) & 7): the 16 word stores of a thread then hit 32
  // distinct banks per half wave
  __shared__ __attribute__((aligned(16))) uint32_t lds_t[kTileCols * 16];

  const int64_t rows = p.rows, cols = p.cols;
  const int64_t tiles_r = (rows + kTileRows - 1) / kTileRows;
  const int64_t tiles_c = (cols + kTileCols - 1) / kTileCols;
  const int64_t ntiles = tiles_r * tiles_c;
  // contiguous runs of tiles per XCD (workgroup b runs on XCD b % 8), tiles
  // numbered down each column of tiles
  const int64_t b = blockIdx.x;
  const int64_t q8 = ntiles / kXcds, rem = ntiles - q8 * kXcds;
  const int64_t xcd = b % kXcds, j8 = b / kXcds;
  const int64_t tile = xcd * q8 + (xcd < rem ? xcd : rem) + j8;
  const int64_t tc = tile / tiles_r, tr = tile - tc * tiles_r;

  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int64_t r0 = tr * kTileRows + 4 * rg;
  const int64_t c0 = tc * kTileCols + 16 * cg;
  const bool col_ok = c0 < cols;  // cols % 16 == 0: all 16 columns or none

  Rows4<InT> t;
  load_rows<InT>(static_cast<const InT*>(p.x), p.ldx, r0, c0, rows, col_ok, t);
  const float amax = p.amax_in != nullptr ? *p.amax_in : reduce_partials(p.partials, p.n_partials);
  const float s8 = fp8_scale_from_amax(amax);
  const float r = __fdiv_rn(1.0f, s8);
  if (blockIdx.x == 0 && tid == 0) {
    *p.tensor_scale = s8;
    if (p.amax_out != nullptr) *p.amax_out = amax;
    if (!(amax <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
  }

  uint4 code[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = fp8x4(__fmul_rn(t.get(i, 4 * q), r), __fmul_rn(t.get(i, 4 * q + 1), r),
                   __fmul_rn(t.get(i, 4 * q + 2), r), __fmul_rn(t.get(i, 4 * q + 3), r));
    }
    code[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }

  if (p.outputs & 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (col_ok && (r0 + i) < rows) {
        *reinterpret_cast<uint4*>(p.q_row + (r0 + i) * cols + c0) = code[i];
      }
    }
  }
  if ((p.outputs & 2) == 0) return;

  // 4 x 16 bytes -> 16 words (word j: column j's 4 rows, row 0 in byte 0)
  uint32_t col_w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t d0 = word_of(code[0], q), d1 = word_of(code[1], q);
    const uint32_t d2 = word_of(code[2], q), d3 = word_of(code[3], q);
    // v_perm_b32: selector byte values 0-3 pick bytes of the second
    // operand, 4-7 bytes of the first
    const uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);  // d0b0 d1b0 d0b1 d1b1
    const uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);  // d0b2 d1b2 d0b3 d1b3
    const uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
    col_w[4 * q + 0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    col_w[4 * q + 1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    col_w[4 * q + 2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    col_w[4 * q + 3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  }
  {
    const int swap = cg & 1, sw = 2 * (cg >> 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) lds_t[((16 * cg + j) ^ swap) * 16 + (rg ^ sw)] = col_w[j];
  }
  __syncthreads();

  // thread tid writes column tid of the tile: 16-row groups as 16-byte
  // stores (rows % 16 == 0 for the column copy)
  const int64_t col = tc * kTileCols + tid;
  if (col < cols) {
    const int cgx = tid >> 4;
    const int pcol = tid ^ (cgx & 1), sw = 2 * (cgx >> 1);
    const int64_t rows_here = (rows - tr * kTileRows) < kTileRows ? (rows - tr * kTileRows) : kTileRows;
    const int groups = static_cast<int>(rows_here >> 4);
    uint8_t* dst = p.q_col + col * rows + tr * kTileRows;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < groups) {
        uint4 v = *reinterpret_cast<const uint4*>(&lds_t[pcol * 16 + 4 * (k ^ (sw >> 2))]);
        if (sw & 2) v = make_uint4(v.z, v.w, v.x, v.y);
        *reinterpret_cast<uint4*>(dst + 16 * k) = v;
      }
    }
  }
}

// Signed E4M3FN byte value (NaN for 0x7F and 0xFF).
__device__ __forceinline__ float e4m3_signed(uint32_t b) {
  const float mag = ((b & 0x7Fu) == 0x7Fu) ? __builtin_nanf("") : e4m3_to_float(b & 0x7Fu);
  return __uint_as_float(__float_as_uint(mag) | ((b & 0x80u) << 24));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One thread expands 16 bytes of a row.
template <bool kBf16>
__global__ __launch_bounds__(256) void fp8_dequantize_kernel(const uint8_t* __restrict__ q,
                                                             const float* __restrict__ tensor_scale,
                                                             int64_t rows, int64_t cols, void* y,
                                                             int64_t ldy) {
  const int64_t nch = cols >> 4;
  const int64_t total = rows * nch;
  const float s = *tensor_scale;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / nch, ch = i - r * nch;
    const uint4 v = *reinterpret_cast<const uint4*>(q + r * cols + ch * 16);
    float out[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t b = (word_of(v, j >> 2) >> (8 * (j & 3))) & 0xFFu;
      out[j] = __fmul_rn(e4m3_signed(b), s);
    }
    if constexpr (kBf16) {
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + r * ldy + ch * 16);
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = f32_to_bf16_rne(out[2 * k]) | (f32_to_bf16_rne(out[2 * k + 1]) << 16);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + r * ldy + ch * 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = make_float4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
    }
  }
}

__global__ void fp8_empty_kernel(const float* amax_in, float* amax_ws, float* tensor_scale,
                                 int32_t* dev_status) {
  if (threadIdx.x != 0) return;
  float a = 0.0f;
  if (amax_in != nullptr) {
    a = *amax_in;
  } else {
    *amax_ws = 0.0f;
  }
  *tensor_scale = fp8_scale_from_amax(a);
  if (!(a <= 3.402823466e38f) && dev_status != nullptr) *dev_status = 1;
}

}  // namespace

int launch_fp8_quantize(const Fp8QuantizeLaunch& q, hipStream_t stream) {
  if (q.rows == 0 || q.cols == 0) {
    fp8_empty_kernel<<<1, 64, 0, stream>>>(q.amax_in, q.amax_ws, q.tensor_scale, q.dev_status);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  Fp8Params p;
  p.x = q.x;
  p.rows = q.rows;
  p.cols = q.cols;
  p.ldx = q.ldx;
  p.amax_in = q.amax_in;
  p.partials = nullptr;
  p.n_partials = 0;
  p.amax_out = nullptr;
  if (q.amax_in == nullptr) {
    const int n = launch_tensor_amax(q.x, q.x_bf16, q.rows, q.cols, q.ldx, q.amax_ws, stream);
    if (n < 0) return -1;
    p.partials = reinterpret_cast<const uint32_t*>(q.amax_ws) + kPartialsOffset;
    p.n_partials = n;
    p.amax_out = q.amax_ws;
  }
  p.tensor_scale = q.tensor_scale;
  p.dev_status = q.dev_status;
  p.q_row = q.q_row;
  p.q_col = q.q_col;
  p.outputs = q.outputs;
  const int64_t tiles = ((q.rows + kTileRows - 1) / kTileRows) * ((q.cols + kTileCols - 1) / kTileCols);
  const unsigned g = static_cast<unsigned>(tiles);
  if (q.x_bf16) fp8_quantize_kernel<uint16_t><<<g, kThreads, 0, stream>>>(p);
  else fp8_quantize_kernel<float><<<g, kThreads, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp8_dequantize(const uint8_t* q, const float* tensor_scale, int64_t rows, int64_t cols,
                          bool out_bf16, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t total = rows * (cols >> 4);
  if (total == 0) return 0;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const unsigned g = static_cast<unsigned>(blocks);
  if (out_bf16) fp8_dequantize_kernel<true><<<g, 256, 0, stream>>>(q, tensor_scale, rows, cols, y, ldy);
  else fp8_dequantize_kernel<false><<<g, 256, 0, stream>>>(q, tensor_scale, rows, cols, y, ldy);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
