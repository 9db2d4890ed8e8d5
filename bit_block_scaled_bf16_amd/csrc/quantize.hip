// NVFP4 quantization kernels for gfx950: tensor amax, 1x16 / 16x1 / 16x16
// block quantization with round-to-nearest or stochastic rounding, and the
// 16-point random Hadamard transform path of the weight-gradient operands.
//
// Sources (gist.science summary of "Pretraining Large Language Models with
// NVFP4", Resumen técnico §2): "Formato NVFP4" (16-element blocks, E4M3 block
// scale, FP32 tensor scale), "Transformadas de Hadamard Aleatorias (RHT)"
// (16x16 Hadamard, fixed random signs, weight-gradient inputs), "Escalado
// Bidimensional (2D) y Redondeo Estocástico" (16x16 weight tiles; stochastic
// rounding of gradients).
//
// Work decomposition. A workgroup of 256 threads (4 waves) owns a tile of
// 256 rows x 128 columns. Lane l of wave w owns the 16 rows starting at
// 64w + 16(l / 16) and the 8 columns starting at 8(l % 16): 16 loads of
// 16 bytes (bf16) whose 16-lane groups cover 256 contiguous bytes of a row.
// That one register tile serves every block shape:
//   * a 1x16 row block is the 8 values of this lane plus the 8 of lane ^ 1
//     (one DPP exchange for the block amax);
//   * a 16x1 column block (and a Hadamard block of 16 tokens) is one of the
//     8 columns, entirely in registers;
//   * a 16x16 tile is this lane's 16x8 half plus lane ^ 1's half.
// Column-blocked codes are stored transposed ([cols][rows/2]); they are
// staged in LDS so each column's 128 bytes leave as contiguous stores.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 256;
constexpr int kTileCols = 128;
constexpr int kLdsCodeStride = kTileRows / 2 + 8;  // bytes per staged column (+8 pad)
constexpr int kLdsScaleStride = kTileRows / 16 + 1;

enum Mode { kMode1D = 0, kMode2D = 1, kModeRHT = 2 };

struct Tile {
  int64_t tr, tc;  // tile coordinates
  int64_t r0, c0;  // first row / column of this lane's 16x8 sub-tile
  int lane, cg, rg, wave;
  int nrows;  // rows of the 16-row group that exist (16 unless at a ragged end)
  bool valid;
};

__device__ __forceinline__ Tile locate(int64_t rows, int64_t cols) {
  Tile t;
  const int tid = threadIdx.x;
  t.lane = tid & 63;
  t.wave = tid >> 6;
  t.cg = t.lane & 15;
  t.rg = t.lane >> 4;
  const int64_t tiles_c = (cols + kTileCols - 1) / kTileCols;
  t.tr = static_cast<int64_t>(blockIdx.x) / tiles_c;
  t.tc = static_cast<int64_t>(blockIdx.x) - t.tr * tiles_c;
  t.r0 = t.tr * kTileRows + t.wave * 64 + t.rg * 16;
  t.c0 = t.tc * kTileCols + t.cg * 8;
  t.valid = (t.r0 < rows) && (t.c0 < cols);
  t.nrows = (rows - t.r0) < 16 ? static_cast<int>(rows - t.r0) : 16;
  return t;
}

// Loads this lane's 16 x 8 values as float32 (bf16 widened exactly).
// Loads this lane's 16 x 8 values as float32 (bf16 widened exactly). With
// kRagged, rows at or beyond r0 + nrows (a row count that is not a multiple
// of 16, allowed only for the row-blocked copy) read as zero; otherwise all
// 16 rows exist and the loads are unconditional.
template <typename InT, bool kRagged>
__device__ __forceinline__ void load_sub_tile(const InT* __restrict__ x, int64_t ldx, int64_t r0,
                                              int64_t c0, int nrows, float (&v)[16][8]) {
  const InT* row = x + r0 * ldx + c0;
  if constexpr (sizeof(InT) == 2) {
    uint4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!kRagged || i < nrows) {
        raw[i] = *reinterpret_cast<const uint4*>(row);
      } else {
        raw[i] = make_uint4(0u, 0u, 0u, 0u);
      }
      row += ldx;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[i][2 * k] = bf16_lo(w[k]);
        v[i][2 * k + 1] = bf16_hi(w[k]);
      }
    }
  } else {
    float4 raw[16][2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!kRagged || i < nrows) {
        raw[i][0] = *reinterpret_cast<const float4*>(row);
        raw[i][1] = *reinterpret_cast<const float4*>(row + 4);
      } else {
        raw[i][0] = make_float4(0.f, 0.f, 0.f, 0.f);
        raw[i][1] = raw[i][0];
      }
      row += ldx;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i][0] = raw[i][0].x; v[i][1] = raw[i][0].y; v[i][2] = raw[i][0].z; v[i][3] = raw[i][0].w;
      v[i][4] = raw[i][1].x; v[i][5] = raw[i][1].y; v[i][6] = raw[i][1].z; v[i][7] = raw[i][1].w;
    }
  }
}

// Applies the Hadamard transform to each of the 8 columns (16 tokens each).
__device__ __forceinline__ void rht_columns(float (&v)[16][8], uint32_t sign_mask) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) col[i] = v[i][j];
    rht16(col, sign_mask);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i][j] = col[i];
  }
}

// Block-wide max of per-thread values, then one atomic max into *dst (the
// float bits of a non-negative amax order like unsigned integers).
__device__ __forceinline__ void block_max_to_global(uint32_t m, uint32_t* lds4, float* dst) {
  m = wave_max_u32(m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds4[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = lds4[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = (lds4[w] > r) ? lds4[w] : r;
    atomicMax(reinterpret_cast<unsigned int*>(dst), r);
  }
}

// ---------------------------------------------------------------------------
// Tensor amax (optionally of the Hadamard-transformed tensor).
// ---------------------------------------------------------------------------
template <typename InT, bool kRht, bool kRagged>
__global__ __launch_bounds__(kThreads) void amax_kernel(const InT* __restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t ldx,
                                                        uint32_t sign_mask, float* amax_out) {
  __shared__ uint32_t lds4[kThreads / 64];
  const Tile t = locate(rows, cols);
  uint32_t m = 0;
  if (t.valid) {
    float v[16][8];
    load_sub_tile<InT, kRagged>(x, ldx, t.r0, t.c0, t.nrows, v);
    if constexpr (kRht) rht_columns(v, sign_mask);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b = abs_bits(v[i][j]);
        m = (b > m) ? b : m;
      }
  }
  block_max_to_global(m, lds4, amax_out);
}

__global__ void fill_f32_kernel(float* p, float v) {
  if (threadIdx.x == 0) *p = v;
}

// Writes the tensor scale (and the status) for an empty tensor.
__global__ void empty_tensor_kernel(const float* amax_in, float* amax_ws, float* tensor_scale,
                                    int32_t* dev_status) {
  if (threadIdx.x != 0) return;
  float a = 0.0f;
  if (amax_in != nullptr) {
    a = *amax_in;
  } else {
    *amax_ws = 0.0f;
  }
  *tensor_scale = tensor_scale_from_amax(a);
  if (!(a <= 3.402823466e38f) && dev_status != nullptr) *dev_status = 1;
}

// ---------------------------------------------------------------------------
// Quantization.
// ---------------------------------------------------------------------------
struct QuantParams {
  const void* x;
  int64_t rows, cols, ldx;
  const float* amax;  // caller's amax or the workspace the amax kernel filled
  float* tensor_scale;
  int32_t* dev_status;
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
  uint32_t k0, k1, offset;
  uint32_t sign_mask;
  int outputs;
};

// Codes of one 16-value column block (or Hadamard block) as two words.
template <bool kSR>
__device__ __forceinline__ void column_block(const float (&col)[16], float six_s, float s,
                                             uint32_t k0, uint32_t k1, uint64_t e0,
                                             uint32_t offset, uint32_t& w0, uint32_t& w1,
                                             uint32_t& sbyte) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t b = abs_bits(col[i]);
    am = (b > am) ? b : am;
  }
  const BlockScale bs = block_scale(__uint_as_float(am), six_s, s);
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __fmul_rn(col[i], bs.mult);
  if constexpr (kSR) {
    const uint64_t g = e0 >> 3;
    w0 = pack8_sr(y, sr_words(k0, k1, g, offset, kStreamCol));
    w1 = pack8_sr(y + 8, sr_words(k0, k1, g + 1, offset, kStreamCol));
  } else {
    w0 = pack8_rn(y);
    w1 = pack8_rn(y + 8);
  }
  const uint32_t keep = (bs.byte == 0u) ? 0u : 0xFFFFFFFFu;
  w0 &= keep;
  w1 &= keep;
  sbyte = bs.byte;
}

template <typename InT, int kMode, bool kSR, bool kRagged>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[kTileCols * kLdsCodeStride];
  __shared__ uint8_t lds_scales[kTileCols * kLdsScaleStride];

  const int64_t rows = p.rows, cols = p.cols;
  const Tile t = locate(rows, cols);
  const float amax = *p.amax;
  const float s = tensor_scale_from_amax(amax);
  const float six_s = __fmul_rn(6.0f, s);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *p.tensor_scale = s;
    if (!(amax <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
  }
  const bool out_row = (p.outputs & 1) != 0 && kMode != kModeRHT;
  const bool out_col = (p.outputs & 2) != 0 || kMode == kModeRHT;
  const int c_local0 = t.cg * 8;
  const int r_local = t.wave * 64 + t.rg * 16;

  if (t.valid) {
    float v[16][8];
    load_sub_tile<InT, kRagged>(static_cast<const InT*>(p.x), p.ldx, t.r0, t.c0, t.nrows, v);
    if constexpr (kMode == kModeRHT) rht_columns(v, p.sign_mask);

    if constexpr (kMode == kMode2D) {
      // one scale per 16x16 tile: this lane's half and lane ^ 1's half
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b = abs_bits(v[i][j]);
          am = (b > am) ? b : am;
        }
      const uint32_t other = swap_adjacent_lanes(am);
      am = (other > am) ? other : am;
      const BlockScale bs = block_scale(__uint_as_float(am), six_s, s);
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = __fmul_rn(v[i][j], bs.mult);
      // codes of a zero-scale tile are 0 (a mask, not a branch)
      const uint32_t keep = (bs.byte == 0u) ? 0u : 0xFFFFFFFFu;
      if ((t.cg & 1) == 0) {
        if (out_row) p.s_row[(t.r0 >> 4) * (cols >> 4) + (t.c0 >> 4)] = static_cast<uint8_t>(bs.byte);
        if (out_col) p.s_col[(t.c0 >> 4) * (rows >> 4) + (t.r0 >> 4)] = static_cast<uint8_t>(bs.byte);
      }
      if (out_row) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t w = pack8_rn(v[i]) & keep;
          *reinterpret_cast<uint32_t*>(p.q_row + (t.r0 + i) * (cols >> 1) + (t.c0 >> 1)) = w;
        }
      }
      if (out_col) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float col[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) col[i] = v[i][j];
          const uint32_t w0 = pack8_rn(col) & keep;
          const uint32_t w1 = pack8_rn(col + 8) & keep;
          uint32_t* dst = reinterpret_cast<uint32_t*>(lds_codes + (c_local0 + j) * kLdsCodeStride +
                                                      (r_local >> 1));
          dst[0] = w0;
          dst[1] = w1;
        }
      }
    } else {
      if (out_row) {
        // 1x16 blocks along the row: this lane's 8 values + lane ^ 1's 8.
        // Rows past a ragged end are skipped by a predicate (the same for
        // both lanes of a pair), not a loop exit, so the register tile keeps
        // static indices.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (!kRagged || i < t.nrows) {
            uint32_t am = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t b = abs_bits(v[i][j]);
              am = (b > am) ? b : am;
            }
            const uint32_t other = swap_adjacent_lanes(am);
            am = (other > am) ? other : am;
            const BlockScale bs = block_scale(__uint_as_float(am), six_s, s);
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = __fmul_rn(v[i][j], bs.mult);
            uint32_t w;
            if constexpr (kSR) {
              const uint64_t e = static_cast<uint64_t>(t.r0 + i) * static_cast<uint64_t>(cols) +
                                 static_cast<uint64_t>(t.c0);
              w = pack8_sr(y, sr_words(p.k0, p.k1, e >> 3, p.offset, kStreamRow));
            } else {
              w = pack8_rn(y);
            }
            w &= (bs.byte == 0u) ? 0u : 0xFFFFFFFFu;
            *reinterpret_cast<uint32_t*>(p.q_row + (t.r0 + i) * (cols >> 1) + (t.c0 >> 1)) = w;
            if ((t.cg & 1) == 0) {
              p.s_row[(t.r0 + i) * (cols >> 4) + (t.c0 >> 4)] = static_cast<uint8_t>(bs.byte);
            }
          }
        }
      }
      if (out_col) {
        // 16x1 blocks along the rows (tokens), one per column
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float col[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) col[i] = v[i][j];
          const uint64_t e0 = static_cast<uint64_t>(t.c0 + j) * static_cast<uint64_t>(rows) +
                              static_cast<uint64_t>(t.r0);
          uint32_t w0, w1, sb;
          column_block<kSR>(col, six_s, s, p.k0, p.k1, e0, p.offset, w0, w1, sb);
          uint32_t* dst = reinterpret_cast<uint32_t*>(lds_codes + (c_local0 + j) * kLdsCodeStride +
                                                      (r_local >> 1));
          dst[0] = w0;
          dst[1] = w1;
          lds_scales[(c_local0 + j) * kLdsScaleStride + (r_local >> 4)] = static_cast<uint8_t>(sb);
        }
      }
    }
  }

  if (!out_col) return;
  __syncthreads();
  // Column-blocked copy: each column's codes for this tile's rows are
  // contiguous in q_col; 16 lanes write one column's 128 bytes.
  const int64_t rows_here = (rows - t.tr * kTileRows) < kTileRows ? (rows - t.tr * kTileRows)
                                                                   : kTileRows;
  const int code_chunks = static_cast<int>(rows_here >> 4);  // 8-byte chunks per column
  for (int k = threadIdx.x; k < kTileCols * (kTileRows / 16); k += kThreads) {
    const int c_local = k >> 4, ch = k & 15;
    const int64_t col = t.tc * kTileCols + c_local;
    if (col < cols && ch < code_chunks) {
      const uint2 val = *reinterpret_cast<const uint2*>(lds_codes + c_local * kLdsCodeStride + ch * 8);
      *reinterpret_cast<uint2*>(p.q_col + col * (rows >> 1) + t.tr * (kTileRows / 2) + ch * 8) = val;
      if constexpr (kMode != kMode2D) {
        p.s_col[col * (rows >> 4) + t.tr * (kTileRows / 16) + ch] =
            lds_scales[c_local * kLdsScaleStride + ch];
      }
    }
  }
}

template <typename InT>
int launch_amax(const InT* x, int64_t rows, int64_t cols, int64_t ldx, bool rht,
                uint32_t sign_mask, float* amax_ws, hipStream_t stream) {
  fill_f32_kernel<<<1, 64, 0, stream>>>(amax_ws, 0.0f);
  const int64_t tiles = ((rows + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
  const unsigned g = static_cast<unsigned>(tiles);
  const bool ragged = (rows % 16) != 0;
  if (rht) {
    amax_kernel<InT, true, false><<<g, kThreads, 0, stream>>>(x, rows, cols, ldx, sign_mask, amax_ws);
  } else if (ragged) {
    amax_kernel<InT, false, true><<<g, kThreads, 0, stream>>>(x, rows, cols, ldx, sign_mask, amax_ws);
  } else {
    amax_kernel<InT, false, false><<<g, kThreads, 0, stream>>>(x, rows, cols, ldx, sign_mask, amax_ws);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename InT, int kMode, bool kSR, bool kRagged>
void launch_quant(const QuantParams& p, hipStream_t stream) {
  const int64_t tiles =
      ((p.rows + kTileRows - 1) / kTileRows) * ((p.cols + kTileCols - 1) / kTileCols);
  quantize_kernel<InT, kMode, kSR, kRagged><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
}

// Ragged row counts (rows % 16 != 0) only reach the 1x16 row-only path: the
// column copy, 16x16 blocks and the RHT path require rows % 16 == 0.
template <typename InT>
void dispatch_quant(const QuantParams& p, int mode, bool sr, hipStream_t stream) {
  const bool ragged = (p.rows % 16) != 0;
  if (mode == kMode2D) {
    launch_quant<InT, kMode2D, false, false>(p, stream);
  } else if (mode == kModeRHT) {
    if (sr) launch_quant<InT, kModeRHT, true, false>(p, stream);
    else launch_quant<InT, kModeRHT, false, false>(p, stream);
  } else if (ragged) {
    if (sr) launch_quant<InT, kMode1D, true, true>(p, stream);
    else launch_quant<InT, kMode1D, false, true>(p, stream);
  } else {
    if (sr) launch_quant<InT, kMode1D, true, false>(p, stream);
    else launch_quant<InT, kMode1D, false, false>(p, stream);
  }
}

// ---------------------------------------------------------------------------
// Inspection hooks: the same loads, transform and random words as above.
// ---------------------------------------------------------------------------
template <typename InT>
__global__ __launch_bounds__(kThreads) void rht_transform_kernel(const InT* __restrict__ x,
                                                                 int64_t rows, int64_t cols,
                                                                 int64_t ldx, uint32_t sign_mask,
                                                                 float* __restrict__ out) {
  const Tile t = locate(rows, cols);
  if (!t.valid) return;
  float v[16][8];
  load_sub_tile<InT, false>(x, ldx, t.r0, t.c0, 16, v);
  rht_columns(v, sign_mask);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float4* dst = reinterpret_cast<float4*>(out + (t.r0 + i) * cols + t.c0);
    dst[0] = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
    dst[1] = make_float4(v[i][4], v[i][5], v[i][6], v[i][7]);
  }
}

__global__ void philox_fill_kernel(uint32_t k0, uint32_t k1, uint32_t c2, uint32_t c3,
                                   int64_t n_groups, uint32_t* __restrict__ out) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const U4 w = sr_words(k0, k1, static_cast<uint64_t>(g), c2, c3);
  reinterpret_cast<uint4*>(out)[g] = make_uint4(w.x, w.y, w.z, w.w);
}

}  // namespace

int launch_quantize(const QuantizeLaunch& q, hipStream_t stream) {
  const bool bf16 = q.x_bf16;
  if (q.rows == 0 || q.cols == 0) {
    empty_tensor_kernel<<<1, 64, 0, stream>>>(q.amax_in, q.amax_ws, q.tensor_scale, q.dev_status);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const float* amax = q.amax_in;
  if (amax == nullptr) {
    const int rc = bf16 ? launch_amax(static_cast<const uint16_t*>(q.x), q.rows, q.cols, q.ldx,
                                      q.rht, q.sign_mask, q.amax_ws, stream)
                        : launch_amax(static_cast<const float*>(q.x), q.rows, q.cols, q.ldx,
                                      q.rht, q.sign_mask, q.amax_ws, stream);
    if (rc != 0) return rc;
    amax = q.amax_ws;
  }
  QuantParams p;
  p.x = q.x;
  p.rows = q.rows;
  p.cols = q.cols;
  p.ldx = q.ldx;
  p.amax = amax;
  p.tensor_scale = q.tensor_scale;
  p.dev_status = q.dev_status;
  p.q_row = q.q_row;
  p.s_row = q.s_row;
  p.q_col = q.q_col;
  p.s_col = q.s_col;
  p.k0 = static_cast<uint32_t>(q.seed);
  p.k1 = static_cast<uint32_t>(q.seed >> 32);
  p.offset = q.offset;
  p.sign_mask = q.sign_mask;
  p.outputs = q.outputs;
  const int mode = q.rht ? kModeRHT : (q.block_2d ? kMode2D : kMode1D);
  if (bf16) dispatch_quant<uint16_t>(p, mode, q.sr, stream);
  else dispatch_quant<float>(p, mode, q.sr, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4

namespace nvfp4 {

int launch_rht_transform(const void* x, bool x_bf16, int64_t tokens, int64_t cols, int64_t ldx,
                         uint32_t sign_mask, float* out, hipStream_t stream) {
  if (tokens == 0 || cols == 0) return 0;
  const int64_t tiles = ((tokens + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
  if (x_bf16) {
    rht_transform_kernel<uint16_t><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(x), tokens, cols, ldx, sign_mask, out);
  } else {
    rht_transform_kernel<float><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(
        static_cast<const float*>(x), tokens, cols, ldx, sign_mask, out);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_philox_fill(uint64_t seed, uint32_t c2, uint32_t c3, int64_t n_groups, uint32_t* out,
                       hipStream_t stream) {
  if (n_groups == 0) return 0;
  const int64_t blocks = (n_groups + 255) / 256;
  philox_fill_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), c2, c3, n_groups, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
