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
// Three quantize kernels. A call that asks for the 1x16 row copy alone goes
// through quantize_rows_kernel (see its comment), which streams rows. The
// Hadamard path of bf16 input (alone, or with the 1x16 row copy from the
// same read) goes through rht_quantize_mfma_kernel, which transforms on the
// matrix cores (see "The Hadamard path of bf16 inputs on the matrix cores").
// Every other call (a column copy, both copies, 16x16 blocks, the Hadamard
// path of float32 input) goes through quantize_kernel, whose decomposition
// follows; the MFMA kernel keeps its 256 x 128 tile and its LDS staging.
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
#include "nvfp4.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 256;
constexpr int kTileCols = 128;
constexpr int kLdsCodeStride = kTileRows / 2;  // bytes per staged column

// LDS byte offset of byte `byte` of staged column `col` (tile-local). The
// 16-byte granules of a column are XOR-swizzled by (col >> 3) & 7: the
// lanes that stage the same rows of 16 different columns then spread over
// 8 granules (2-way bank conflicts instead of 8-way with a padded row), and a
// granule stays 16-byte aligned for the write-out.
__device__ __forceinline__ int staged_code_offset(int col, int byte) {
  return col * kLdsCodeStride + ((((byte >> 4) ^ ((col >> 3) & 7)) << 4) | (byte & 15));
}
constexpr int64_t kMaxTileBlocks = 1024;  // workgroups of the tile-shaped amax kernels

// kModeRowRHT: the 1x16 row copy (round to nearest) and the Hadamard column
// copy of the same tensor, each with its own tensor scale, from one read.
enum Mode { kMode1D = 0, kMode2D = 1, kModeRHT = 2, kModeRowRHT = 3 };

struct Tile {
  int64_t tr, tc;  // tile coordinates
  int64_t r0, c0;  // first row / column of this lane's 16x8 sub-tile
  int lane, cg, rg, wave;
  int nrows;  // rows of the 16-row group that exist (16 unless at a ragged end)
  bool valid;
};

__device__ __forceinline__ Tile locate_rc(int64_t tr, int64_t tc, int64_t rows, int64_t cols) {
  Tile t;
  const int tid = threadIdx.x;
  t.lane = tid & 63;
  t.wave = tid >> 6;
  t.cg = t.lane & 15;
  t.rg = t.lane >> 4;
  t.tr = tr;
  t.tc = tc;
  t.r0 = t.tr * kTileRows + t.wave * 64 + t.rg * 16;
  t.c0 = t.tc * kTileCols + t.cg * 8;
  t.valid = (t.r0 < rows) && (t.c0 < cols);
  t.nrows = (rows - t.r0) < 16 ? static_cast<int>(rows - t.r0) : 16;
  return t;
}

// Tile `tile` in row-major order.
__device__ __forceinline__ Tile locate_tile(int64_t tile, int64_t rows, int64_t cols) {
  const int64_t tiles_c = (cols + kTileCols - 1) / kTileCols;
  const int64_t tr = tile / tiles_c;
  return locate_rc(tr, tile - tr * tiles_c, rows, cols);
}

// Workgroups are handed to the 8 XCDs of the chip round-robin (workgroup b
// to XCD b % 8), and each XCD has its own L2. Numbering the tiles so that XCD
// x gets a contiguous run of them puts horizontally adjacent tiles, which
// write the two halves of the same 128-byte lines of the row copy, behind
// the same L2, where the halves merge before they reach memory. The mapping
// is a permutation of [0, ntiles) for any tile count.
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t ntiles) {
  const int64_t q = ntiles / kXcds, r = ntiles - q * kXcds;
  const int64_t x = b % kXcds, j = b / kXcds;
  return x * q + (x < r ? x : r) + j;
}

// Tile k of the band order: bands of 8 tile rows, each walked column by
// column (its 8 tiles down, then the next column). With xcd_tile handing
// each XCD a contiguous run of this order, the 128-160 workgroups an XCD
// runs at once cover about 16-20 columns x 8 rows of tiles. Every 128-byte
// line of the row scales (8 bytes from each of 16 horizontally adjacent
// tiles), of the column scales (16 bytes from each of 8 vertically adjacent
// tiles) and of the row codes (two horizontal halves) is then written by
// workgroups that run together behind one L2, which merges the pieces. A
// permutation of [0, tiles_r * tiles_c).
constexpr int64_t kBandRows = 8;

__device__ __forceinline__ void band_tile(int64_t k, int64_t tiles_r, int64_t tiles_c, int64_t& tr,
                                          int64_t& tc) {
  const int64_t band = k / (kBandRows * tiles_c);
  const int64_t tr0 = band * kBandRows;
  const int64_t h = tiles_r - tr0 < kBandRows ? tiles_r - tr0 : kBandRows;
  const int64_t kin = k - band * kBandRows * tiles_c;
  tc = kin / h;
  tr = tr0 + (kin - tc * h);
}

__device__ __forceinline__ Tile locate(int64_t rows, int64_t cols) {
  const int64_t tiles_r = (rows + kTileRows - 1) / kTileRows, tiles_c = (cols + kTileCols - 1) / kTileCols;
  int64_t tr, tc;
  band_tile(xcd_tile(static_cast<int64_t>(blockIdx.x), tiles_r * tiles_c), tiles_r, tiles_c, tr, tc);
  return locate_rc(tr, tc, rows, cols);
}

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
  const RhtSigns g = rht_signs(sign_mask);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) col[i] = v[i][j];
    rht16(col, g);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i][j] = col[i];
  }
}

// Partials instead of one atomic maximum need no zeroed word before the
// reduction, so a call is two kernels, not three.
static_assert(kPartialsOffset + 2 * kMaxPartials <= NVFP4_AMAX_WS_BYTES / 4, "workspace size");
static_assert(kMaxTileBlocks <= kMaxPartials, "one partial per workgroup");

// Block-wide max of per-thread values, written by thread 0 to *dst.
__device__ __forceinline__ void block_max_store(uint32_t m, uint32_t* lds4, uint32_t* dst) {
  m = wave_max_u32(m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds4[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = lds4[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = (lds4[w] > r) ? lds4[w] : r;
    *dst = r;
  }
}

// ---------------------------------------------------------------------------
// Tensor amax.
// ---------------------------------------------------------------------------

// Contiguous input (ldx == cols), no transform: a flat stream of 16-byte
// nontemporal loads (the data is not reused from the cache), 8 per thread in
// flight per iteration. bf16 magnitudes are compared
// two at a time as packed 16-bit integers (the bf16 bits of |x| order like
// its value, NaN above infinity).
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
constexpr int kFlatUnroll = 8;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                                                __builtin_bit_cast(ushort2_t, b)));
}

template <typename InT>
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const InT* __restrict__ x, int64_t n,
                                                             uint32_t* __restrict__ partials) {
  __shared__ uint32_t lds4[kThreads / 64];
  constexpr int kVec = 16 / sizeof(InT);  // elements per 16-byte load
  const int64_t nvec = n / kVec;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kFlatUnroll;
  uint32_t m = 0;  // bf16: two packed 16-bit maxima; float32: one
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kFlatUnroll + threadIdx.x;
       base < nvec; base += stride) {
    uint4 r[kFlatUnroll];
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      r[u] = i < nvec ? load_stream(xv + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
      const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (sizeof(InT) == 2) {
          m = max_u16x2(m, w[k] & 0x7FFF7FFFu);
        } else {
          const uint32_t a = w[k] & 0x7FFFFFFFu;
          m = a > m ? a : m;
        }
      }
    }
  }
  // the last n % kVec elements
  if (blockIdx.x == 0 && threadIdx.x < n - nvec * kVec) {
    if constexpr (sizeof(InT) == 2) {
      m = max_u16x2(m, static_cast<uint32_t>(x[nvec * kVec + threadIdx.x]) & 0x7FFFu);
    } else {
      const uint32_t a = __float_as_uint(x[nvec * kVec + threadIdx.x]) & 0x7FFFFFFFu;
      m = a > m ? a : m;
    }
  }
  if constexpr (sizeof(InT) == 2) {
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    m = (lo > hi ? lo : hi) << 16;  // float bits of the larger bf16 magnitude
  }
  block_max_store(m, lds4, partials + blockIdx.x);
}

// Tile-shaped amax (the Hadamard transform needs whole 16-token columns; a
// padded input needs its row stride): each workgroup walks tiles
// blockIdx.x, blockIdx.x + gridDim.x, ... For bf16 the next tile's 16 x 16
// bytes are requested before the current one is transformed, and the
// transform goes one pair of columns at a time (32 floats live).
template <bool kRht>
__device__ __forceinline__ uint32_t absmax_bf16_tile(const uint4 (&raw)[16], const RhtSigns& g,
                                                     uint32_t m) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float c0[16], c1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w = k == 0 ? raw[i].x : k == 1 ? raw[i].y : k == 2 ? raw[i].z : raw[i].w;
      c0[i] = bf16_lo(w);
      c1[i] = bf16_hi(w);
    }
    if constexpr (kRht) {
      rht16_unscaled(c0, g);
      rht16_unscaled(c1, g);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b0 = abs_bits(c0[i]), b1 = abs_bits(c1[i]);
      m = (b0 > m) ? b0 : m;
      m = (b1 > m) ? b1 : m;
    }
  }
  return m;
}

template <bool kRagged>
__device__ __forceinline__ void load_raw_bf16(const uint16_t* __restrict__ x, int64_t ldx,
                                              const Tile& t, uint4 (&raw)[16]) {
  const uint16_t* row = x + t.r0 * ldx + t.c0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    raw[i] = (t.valid && (!kRagged || i < t.nrows)) ? load_stream(row) : make_uint4(0u, 0u, 0u, 0u);
    row += ldx;
  }
}

// With kDual (and kRht) the workgroup also writes the largest magnitude of
// the untransformed values to partials_plain (the row copy's amax of a
// tensor quantized both ways in one call).
template <typename InT, bool kRht, bool kRagged, bool kDual = false>
__global__ __launch_bounds__(kThreads) void amax_tile_kernel(const InT* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ldx,
                                                             uint32_t sign_mask, int64_t tiles,
                                                             uint32_t* __restrict__ partials,
                                                             uint32_t* __restrict__ partials_plain) {
  static_assert(!kDual || kRht, "the dual maximum comes with the transform");
  __shared__ uint32_t lds4[kThreads / 64];
  __shared__ uint32_t lds4_plain[kThreads / 64];
  uint32_t m = 0;
  uint32_t m_plain = 0;  // bf16: two packed 16-bit maxima; float32: one
  const RhtSigns g = rht_signs(sign_mask);
  if constexpr (sizeof(InT) == 2) {
    // invalid lanes (past the columns) load zeros, which leave the max alone
    int64_t tile = blockIdx.x;
    uint4 raw[16];
    load_raw_bf16<kRagged>(x, ldx, locate_tile(tile, rows, cols), raw);
    for (; tile < tiles; tile += gridDim.x) {
      uint4 cur[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) cur[i] = raw[i];
      const int64_t next = tile + gridDim.x;
      if (next < tiles) load_raw_bf16<kRagged>(x, ldx, locate_tile(next, rows, cols), raw);
      if constexpr (kDual) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          m_plain = max_u16x2(m_plain, cur[i].x & 0x7FFF7FFFu);
          m_plain = max_u16x2(m_plain, cur[i].y & 0x7FFF7FFFu);
          m_plain = max_u16x2(m_plain, cur[i].z & 0x7FFF7FFFu);
          m_plain = max_u16x2(m_plain, cur[i].w & 0x7FFF7FFFu);
        }
      }
      m = absmax_bf16_tile<kRht>(cur, g, m);
    }
    if constexpr (kDual) {
      const uint32_t lo = m_plain & 0xFFFFu, hi = m_plain >> 16;
      m_plain = (lo > hi ? lo : hi) << 16;  // float bits of the larger bf16 magnitude
    }
    // the 1/4 of the transform, applied to the maximum: rounding is
    // monotonic and symmetric, so max |RN(h / 4)| = RN(max |h| / 4)
    if constexpr (kRht) m = __float_as_uint(__fmul_rn(__uint_as_float(m), 0.25f));
  } else {
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
      const Tile t = locate_tile(tile, rows, cols);
      if (!t.valid) continue;
      float v[16][8];
      load_sub_tile<InT, kRagged>(x, ldx, t.r0, t.c0, t.nrows, v);
      if constexpr (kDual) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t b = abs_bits(v[i][j]);
            m_plain = (b > m_plain) ? b : m_plain;
          }
      }
      if constexpr (kRht) rht_columns(v, sign_mask);
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b = abs_bits(v[i][j]);
          m = (b > m) ? b : m;
        }
    }
  }
  block_max_store(m, lds4, partials + blockIdx.x);
  if constexpr (kDual) block_max_store(m_plain, lds4_plain, partials_plain + blockIdx.x);
}

// Writes the tensor scale (and the status) for an empty tensor.
__global__ void empty_tensor_kernel(const float* amax_in, float* amax_ws, float* tensor_scale,
                                    int32_t* dev_status) {
  if (threadIdx.x != 0) return;
  float a = 0.0f;
  if (amax_in != nullptr) {
    a = *amax_in;
  } else {
    *amax_ws = 0.0f;  // [0] of the workspace: the tensor amax
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
  const float* amax_in;       // caller's amax, or NULL: reduce the partials
  const uint32_t* partials;   // per-workgroup maxima of the amax kernel
  int n_partials;
  float* amax_out;            // receives the reduced amax (workspace [0]), or NULL
  float* tensor_scale;
  int32_t* dev_status;
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
  uint32_t k0, k1, offset;
  uint32_t sign_mask;
  int outputs;
  // kModeRowRHT: the Hadamard column copy's own amax and tensor scale (the
  // fields above serve the row copy)
  const float* amax_in_t;
  const uint32_t* partials_t;
  float* amax_out_t;
  float* tensor_scale_t;
};

// Random words of stochastic rounding for one launch and one copy (stream):
// the launch-constant form of Philox when every counter's g fits 32 bits
// (fewer than 2^35 elements; a uniform branch), the plain one otherwise.
struct SrKey {
  PhiloxSr ps;
  uint32_t k0, k1, offset, stream;
  bool small;
};

__device__ __forceinline__ SrKey sr_key(const QuantParams& p, uint32_t stream) {
  SrKey k;
  k.ps = philox_sr_setup(p.k0, p.k1, p.offset, stream);
  k.k0 = p.k0;
  k.k1 = p.k1;
  k.offset = p.offset;
  k.stream = stream;
  k.small = static_cast<uint64_t>(p.rows) * static_cast<uint64_t>(p.cols) < (uint64_t(1) << 35);
  return k;
}

__device__ __forceinline__ U4 words_for(const SrKey& k, uint64_t g) {
  if (k.small) return sr_words_fast(k.ps, static_cast<uint32_t>(g));
  return sr_words(k.k0, k.k1, g, k.offset, k.stream);
}

// Scale byte and element multiplier of a block with amax a_b: the byte is
// E4M3(fp32(a_b / 6S)); the multiplier r = fp32(1 / fp32(s_f S)) comes from
// the workgroup's table of the 127 byte values (0 for the zero byte).
struct BlockMult {
  uint32_t byte;
  float mult;
};

// Division by the tensor's 6 S, which every block of a launch shares. With
// y = fp32(1 / d) taken once, q0 = fp32(a y), the remainder r = a - q0 d
// (exact in one fused multiply-add) and fp32(q0 + r y) (one more) give the
// correctly rounded quotient fp32(a / d) (Markstein's correction step; a
// CPU check found no exception in 3e10 cases with d in [2^-60, 2^120] and
// quotients in [2^-12, 2^13], and quotients outside that range are either
// far below E4M3's smallest step or saturate). The remainder must not be a
// float32 subnormal, so for d < 2^-60 (a tensor amax below about 2^-52) the
// division is a plain IEEE division instead: the branch is uniform.
struct ScaleDiv {
  float d, y;
  bool fast;
};

__device__ __forceinline__ ScaleDiv scale_div(float six_s) {
  ScaleDiv sd;
  // the same value in every lane; made explicit so that the branch in div_by
  // is a scalar one
  sd.d = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(six_s)));
  sd.y = __fdiv_rn(1.0f, sd.d);
  sd.fast = sd.d >= 0x1p-60f;
  return sd;
}

__device__ __forceinline__ float div_by(float a, const ScaleDiv& sd) {
  if (sd.fast) {
    const float q0 = __fmul_rn(a, sd.y);
    const float r = __builtin_fmaf(-q0, sd.d, a);
    return __builtin_fmaf(r, sd.y, q0);
  }
  return __fdiv_rn(a, sd.d);
}

__device__ __forceinline__ BlockMult block_mult(float amax_b, const ScaleDiv& six_s, const float* rtab) {
  BlockMult b;
  b.byte = e4m3_from_float(div_by(amax_b, six_s));
  b.mult = rtab[b.byte];
  return b;
}

// Fills rtab[0..127] (LDS) for tensor scale s; the caller synchronizes.
__device__ __forceinline__ void fill_recip_table(float* rtab, float s) {
  const int b = threadIdx.x;
  if (b < 128) rtab[b] = (b == 0 || b == 127) ? 0.0f : __fdiv_rn(1.0f, __fmul_rn(e4m3_to_float(b), s));
}

// Largest magnitude of n floats (finite inputs; a NaN is skipped, which only
// matters where the outputs are unspecified anyway).
template <int n>
__device__ __forceinline__ float abs_max(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < n; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// Codes of one 16-value column block as two words. With kQuarter the values
// are the Hadamard butterfly's, which leaves out the final 1/4: the block
// maximum and the multiplier take the 1/4 instead. Scaling by a power of two
// commutes with the maximum and with the rounding of y = x * r, so the bits
// are those of quantizing the scaled values, unless a scaled value or r / 4
// would be a float32 subnormal.
template <bool kSR, bool kQuarter>
__device__ __forceinline__ void column_block(const float (&col)[16], const ScaleDiv& six_s, const float* rtab,
                                             const SrKey& key, uint64_t e0, uint32_t& w0,
                                             uint32_t& w1, uint32_t& sbyte) {
  float am = abs_max<16>(col);
  if constexpr (kQuarter) am = __fmul_rn(am, 0.25f);
  BlockMult bm = block_mult(am, six_s, rtab);
  if constexpr (kQuarter) bm.mult = __fmul_rn(bm.mult, 0.25f);
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __fmul_rn(col[i], bm.mult);
  if constexpr (kSR) {
    const uint64_t g = e0 >> 3;
    w0 = pack8_sr(y, words_for(key, g));
    w1 = pack8_sr(y + 8, words_for(key, g + 1));
  } else {
    w0 = pack8_rn(y);
    w1 = pack8_rn(y + 8);
  }
  const uint32_t keep = (bm.byte == 0u) ? 0u : 0xFFFFFFFFu;
  w0 &= keep;
  w1 &= keep;
  sbyte = bm.byte;
}

// One lane's 16 x 8 register tile as loaded (bf16 words or float32 values),
// read back as float32 value by value: only the values a step needs are
// widened, which keeps the register count (and so the waves per SIMD that
// hide the load latency) where it is with the raw words alone.
template <typename InT>
struct RawTile;

template <>
struct RawTile<uint16_t> {
  uint4 r[16];
  __device__ __forceinline__ float get(int i, int j) const {
    const uint32_t w = (j >> 1) == 0 ? r[i].x : (j >> 1) == 1 ? r[i].y : (j >> 1) == 2 ? r[i].z : r[i].w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  // float32 bits of the largest magnitude (packed 16-bit maxima of the bf16
  // magnitudes, then the larger half)
  __device__ __forceinline__ uint32_t absmax_bits() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      m = max_u16x2(m, r[i].x & 0x7FFF7FFFu);
      m = max_u16x2(m, r[i].y & 0x7FFF7FFFu);
      m = max_u16x2(m, r[i].z & 0x7FFF7FFFu);
      m = max_u16x2(m, r[i].w & 0x7FFF7FFFu);
    }
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    return (lo > hi ? lo : hi) << 16;
  }
  // Hides the words from value numbering: a second pass over the tile then
  // widens them again (one shift or mask per value) instead of keeping the
  // first pass's 128 widened floats alive, which would halve the occupancy.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(r[i].x), "+v"(r[i].y), "+v"(r[i].z), "+v"(r[i].w));
  }
};

template <>
struct RawTile<float> {
  float4 r[16][2];
  __device__ __forceinline__ float get(int i, int j) const {
    const float4& v = r[i][j >> 2];
    return (j & 3) == 0 ? v.x : (j & 3) == 1 ? v.y : (j & 3) == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ uint32_t absmax_bits() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b = abs_bits(get(i, j));
        m = b > m ? b : m;
      }
    return m;
  }
  __device__ __forceinline__ void opaque() {}
};

// Loads this lane's 16 x 8 values (nontemporal: the tile is read once). Every
// call reaching the tile kernel has
// rows % 16 == 0, so a lane's 16 rows all exist or none does. A lane past the
// matrix reads the matrix's first 16 x 8 values instead (such calls have at
// least 16 rows and 16 columns) and never uses them: loads without a
// condition go out back to back, where a select per load became a branch and
// a wait per load.
template <typename InT>
__device__ __forceinline__ void load_raw(const InT* __restrict__ x, int64_t ldx, const Tile& t,
                                         RawTile<InT>& raw) {
  const InT* row = x + (t.valid ? t.r0 * ldx + t.c0 : 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (sizeof(InT) == 2) {
      raw.r[i] = load_stream(row);
    } else {
      const uint4 a = load_stream(row), b = load_stream(row + 4);
      raw.r[i][0] = make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                                __uint_as_float(a.w));
      raw.r[i][1] = make_float4(__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z),
                                __uint_as_float(b.w));
    }
    row += ldx;
  }
}

// LDS staging of the tile's outputs that leave in another shape than they
// are computed: the column copy (codes and scales of each column) and the
// row-block scales of the 1x16 row copy (8 bytes per row, one 8-byte store
// instead of eight byte stores).
struct Staging {
  uint8_t codes[kTileCols * kLdsCodeStride];
  uint8_t col_scales[kTileCols * 16];
  uint8_t row_scales[kTileRows * 8];
};

// Writes a tile's staged outputs after the barrier that ends its staging:
// the row-block scales (8 bytes per row of the tile) and the column copy
// (128 code bytes and, with col_scales, 16 scale bytes per column).
__device__ __forceinline__ void store_staged(const Staging& st, const QuantParams& p, int64_t tr,
                                             int64_t tc, bool stage_row_scales, bool out_col,
                                             bool col_scales) {
  const int64_t rows = p.rows, cols = p.cols;
  const int tid = threadIdx.x;
  if (stage_row_scales) {
    // one row's 8 scale bytes of this tile per thread
    const int64_t row = tr * kTileRows + tid;
    const int64_t nblk = (cols - tc * kTileCols) < kTileCols ? (cols - tc * kTileCols) >> 4 : 8;
    if (row < rows) {
      uint8_t* dst = p.s_row + row * (cols >> 4) + tc * 8;
      if (nblk == 8 && ((cols >> 4) & 7) == 0) {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(st.row_scales + tid * 8);
      } else {
        for (int b = 0; b < nblk; ++b) dst[b] = st.row_scales[tid * 8 + b];
      }
    }
  }
  if (out_col) {
    // each column's codes for this tile's rows are contiguous in q_col: 8
    // lanes write one column's 128 bytes as 16-byte granules (8-byte chunks
    // when rows % 32 != 0 leaves column starts only 8-byte aligned), and its
    // 16 scale bytes (1D) leave as one store where alignment allows
    const int64_t rows_here = (rows - tr * kTileRows) < kTileRows ? (rows - tr * kTileRows) : kTileRows;
    const int code_chunks = static_cast<int>(rows_here >> 4);  // 8-byte chunks per column
    if ((rows & 31) == 0) {
      const int granules = code_chunks >> 1;
#pragma unroll
      for (int k = tid; k < kTileCols * (kTileRows / 32); k += kThreads) {
        const int c_local = k >> 3, g = k & 7;
        const int64_t col = tc * kTileCols + c_local;
        if (col < cols && g < granules) {
          const uint4 val = *reinterpret_cast<const uint4*>(st.codes + staged_code_offset(c_local, 16 * g));
          *reinterpret_cast<uint4*>(p.q_col + col * (rows >> 1) + tr * (kTileRows / 2) + 16 * g) = val;
        }
      }
    } else {
#pragma unroll
      for (int k = tid; k < kTileCols * (kTileRows / 16); k += kThreads) {
        const int c_local = k >> 4, ch = k & 15;
        const int64_t col = tc * kTileCols + c_local;
        if (col < cols && ch < code_chunks) {
          const uint2 val = *reinterpret_cast<const uint2*>(st.codes + staged_code_offset(c_local, 8 * ch));
          *reinterpret_cast<uint2*>(p.q_col + col * (rows >> 1) + tr * (kTileRows / 2) + ch * 8) = val;
        }
      }
    }
    if (col_scales) {
      if (tid < kTileCols) {
        const int64_t col = tc * kTileCols + tid;
        if (col < cols) {
          uint8_t* dst = p.s_col + col * (rows >> 4) + tr * (kTileRows / 16);
          if (code_chunks == 16 && ((rows >> 4) & 15) == 0) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(st.col_scales + tid * 16);
          } else {
            for (int b = 0; b < code_chunks; ++b) dst[b] = st.col_scales[tid * 16 + b];
          }
        }
      }
    }
  }
}

// One workgroup per 256 x 128 tile.
template <typename InT, int kMode, bool kSR>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  constexpr bool kRhtCol = kMode == kModeRHT || kMode == kModeRowRHT;
  constexpr bool kDualScale = kMode == kModeRowRHT;
  __shared__ __attribute__((aligned(16))) Staging st;
  __shared__ float rtab[128];
  __shared__ float rtab_t[kDualScale ? 128 : 1];

  const int64_t rows = p.rows, cols = p.cols;
  const Tile t = locate(rows, cols);
  // The partial maxima are requested first and the tile right after: the
  // amax reduction, the reciprocal tables and the barrier then wait only for
  // the partials, while the tile is still in flight.
  const bool reduce = p.amax_in == nullptr;
  const bool reduce_t = kDualScale && p.amax_in_t == nullptr;
  PartialWords pw{}, pw_t{};
  if (reduce) load_partials(p.partials, pw);
  if (reduce_t) load_partials(p.partials_t, pw_t);
  RawTile<InT> cur;
  load_raw<InT>(static_cast<const InT*>(p.x), p.ldx, t, cur);
  const float amax = reduce ? reduce_loaded_partials(pw, p.n_partials) : *p.amax_in;
  const float s = tensor_scale_from_amax(amax);
  const ScaleDiv six_s = scale_div(__fmul_rn(6.0f, s));
  float s_t = s;
  ScaleDiv six_s_t = six_s;
  if constexpr (kDualScale) {
    const float amax_t = reduce_t ? reduce_loaded_partials(pw_t, p.n_partials) : *p.amax_in_t;
    s_t = tensor_scale_from_amax(amax_t);
    six_s_t = scale_div(__fmul_rn(6.0f, s_t));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *p.tensor_scale_t = s_t;
      if (p.amax_out_t != nullptr) *p.amax_out_t = amax_t;
      if (!(amax_t <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *p.tensor_scale = s;
    if (p.amax_out != nullptr) *p.amax_out = amax;
    if (!(amax <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
  }
  fill_recip_table(rtab, s);
  if constexpr (kDualScale) fill_recip_table(rtab_t, s_t);
  __syncthreads();
  // the column copy's scale: in kModeRowRHT the Hadamard copy's own
  const ScaleDiv six_s_col = kDualScale ? six_s_t : six_s;
  const float* rtab_col = kDualScale ? rtab_t : rtab;
  const RhtSigns g = rht_signs(p.sign_mask);
  const SrKey key_row = sr_key(p, kStreamRow), key_col = sr_key(p, kStreamCol);
  const bool out_row = (p.outputs & 1) != 0 && kMode != kModeRHT;
  const bool out_col = (p.outputs & 2) != 0 || kRhtCol;
  const bool stage_row_scales = out_row && kMode != kMode2D;
  {
    const int c_local0 = t.cg * 8;
    const int r_local = t.wave * 64 + t.rg * 16;

    if (t.valid) {
      if constexpr (kMode == kMode2D) {
        // one scale per 16x16 tile: this lane's half and lane ^ 1's half
        uint32_t am = cur.absmax_bits();
        const uint32_t other = swap_adjacent_lanes(am);
        am = (other > am) ? other : am;
        const BlockMult bs = block_mult(__uint_as_float(am), six_s, rtab);
        // codes of a zero-scale tile are 0 (a mask, not a branch)
        const uint32_t keep = (bs.byte == 0u) ? 0u : 0xFFFFFFFFu;
        if ((t.cg & 1) == 0) {
          if (out_row) p.s_row[(t.r0 >> 4) * (cols >> 4) + (t.c0 >> 4)] = static_cast<uint8_t>(bs.byte);
          if (out_col) p.s_col[(t.c0 >> 4) * (rows >> 4) + (t.r0 >> 4)] = static_cast<uint8_t>(bs.byte);
        }
        if (out_row) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = __fmul_rn(cur.get(i, j), bs.mult);
            const uint32_t w = pack8_rn(y) & keep;
            *reinterpret_cast<uint32_t*>(p.q_row + (t.r0 + i) * (cols >> 1) + (t.c0 >> 1)) = w;
          }
        }
        if (out_col) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float col[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) col[i] = __fmul_rn(cur.get(i, j), bs.mult);
            uint32_t* dst = reinterpret_cast<uint32_t*>(st.codes +
                                                        staged_code_offset(c_local0 + j, r_local >> 1));
            dst[0] = pack8_rn(col) & keep;
            dst[1] = pack8_rn(col + 8) & keep;
          }
        }
      } else {
        if (out_row) {
          // 1x16 blocks along the row: this lane's 8 values + lane ^ 1's 8
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x8[j] = cur.get(i, j);
            const float mine = abs_max<8>(x8);
            const float am = fmaxf(mine, __uint_as_float(swap_adjacent_lanes(__float_as_uint(mine))));
            const BlockMult bs = block_mult(am, six_s, rtab);
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = __fmul_rn(x8[j], bs.mult);
            uint32_t w;
            if constexpr (kSR && !kDualScale) {
              const uint64_t e = static_cast<uint64_t>(t.r0 + i) * static_cast<uint64_t>(cols) +
                                 static_cast<uint64_t>(t.c0);
              w = pack8_sr(y, words_for(key_row, e >> 3));
            } else {
              w = pack8_rn(y);
            }
            w &= (bs.byte == 0u) ? 0u : 0xFFFFFFFFu;
            *reinterpret_cast<uint32_t*>(p.q_row + (t.r0 + i) * (cols >> 1) + (t.c0 >> 1)) = w;
            if ((t.cg & 1) == 0) st.row_scales[(r_local + i) * 8 + (t.cg >> 1)] = static_cast<uint8_t>(bs.byte);
          }
        }
        if (out_col) {
          if constexpr (kDualScale) cur.opaque();
          // 16x1 blocks along the rows (tokens), one per column, after the
          // Hadamard transform on the RHT path; two columns at a time
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float c0[16], c1[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              c0[i] = cur.get(i, 2 * k);
              c1[i] = cur.get(i, 2 * k + 1);
            }
            if constexpr (kRhtCol) {
              rht16_unscaled(c0, g);
              rht16_unscaled(c1, g);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int j = 2 * k + h;
              const uint64_t e0 = static_cast<uint64_t>(t.c0 + j) * static_cast<uint64_t>(rows) +
                                  static_cast<uint64_t>(t.r0);
              uint32_t w0, w1, sb;
              column_block<kSR, kRhtCol>(h == 0 ? c0 : c1, six_s_col, rtab_col, key_col, e0, w0, w1,
                                         sb);
              uint32_t* dst = reinterpret_cast<uint32_t*>(
                  st.codes + staged_code_offset(c_local0 + j, r_local >> 1));
              dst[0] = w0;
              dst[1] = w1;
              st.col_scales[(c_local0 + j) * 16 + (r_local >> 4)] = static_cast<uint8_t>(sb);
            }
          }
        }
      }
    }

    if (!out_col && !stage_row_scales) return;
    __syncthreads();
    store_staged(st, p, t.tr, t.tc, stage_row_scales, out_col, kMode != kMode2D);
  }
}

// ---------------------------------------------------------------------------
// The Hadamard path of bf16 inputs on the matrix cores.
//
// A 16-token block of one column transforms as x' = A x with
// A = H diag(d) / 4, whose entries are +-1/4 and exact in bf16. So
// v_mfma_f32_16x16x16_bf16 forms every product exactly and sums them in
// float32. Its results are within one float32 unit of the block's largest
// magnitude of the exact transform (measured on MI355X), and the same inputs
// always give the same bits, so the amax pass, the quantize pass and the
// inspection hook agree exactly. (float32 inputs keep the butterfly.)
//
// Lane layout of the MFMA operands: lane l owns the 4 consecutive tokens
// 4 (l / 16) + i (i = 0..3) of a 16-token step and the 8 consecutive columns
// 8 (l % 16) + j (j = 0..7), i.e. four 16-byte loads. MFMA j takes the lane's
// column j (4 tokens) as its B operand and the lane's slice of A, and
// returns the transformed values of the same 4 tokens of column j: each lane
// ends up holding its own 4 x 8 block, transformed. A 16x1 column block then
// lies in the 4 lanes with the same l % 16; a 1x16 row block (the row copy)
// in lanes 2m and 2m + 1. The workgroup keeps the 256 x 128 tile of the
// other modes; wave w owns its tokens 64 w .. 64 w + 63 as 4 steps of 16.
// ---------------------------------------------------------------------------
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kSteps = 4;  // 16-token steps per wave and tile
static_assert(kTileRows == (kThreads / 64) * 16 * kSteps, "each wave owns 4 steps of the tile");

// Lane l's A operand: A[m][k] for m = l % 16, k = 4 (l / 16) + v, i.e.
// (-1)^popcount(m & k) * d_k / 4 as bf16 (+-0.25 = 0x3E80 / 0xBE80).
__device__ __forceinline__ bf16x4_t rht_a_operand(uint32_t sign_mask) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, k0 = 4 * (lane >> 4);
  bf16x4_t a;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int k = k0 + v;
    const uint32_t neg = (static_cast<uint32_t>(__popc(m & k)) ^ (sign_mask >> k)) & 1u;
    a[v] = static_cast<short>(neg ? 0xBE80 : 0x3E80);
  }
  return a;
}

template <int q>
__device__ __forceinline__ uint32_t word_of(const uint4& r) {
  return q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
}

// Transformed values of the lane's column j from its 4 token rows (8 bf16
// each): the j-th bf16 of every row, paired into the B operand by two byte
// permutes, then one MFMA. Result v = token 4 (l / 16) + v of column j.
template <int j>
__device__ __forceinline__ u32x2_t rht_b_operand(const uint4* rows4) {
  constexpr uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t lo = __builtin_amdgcn_perm(word_of<j / 2>(rows4[1]), word_of<j / 2>(rows4[0]), sel);
  const uint32_t hi = __builtin_amdgcn_perm(word_of<j / 2>(rows4[3]), word_of<j / 2>(rows4[2]), sel);
  return u32x2_t{lo, hi};
}

// Columns j0 .. j0 + 3 in one block: the results land in VGPRs that do not
// overlap the sources (early-clobber), with the wait states around the four
// MFMAs written out (2 before for the B operands' producers, 16 after for the
// readers of the results).
template <int j0>
__device__ __forceinline__ void rht_mfma4(bf16x4_t a, const uint4* rows4, f32x4_t (&o)[4]) {
  const u32x2_t b0 = rht_b_operand<j0>(rows4), b1 = rht_b_operand<j0 + 1>(rows4);
  const u32x2_t b2 = rht_b_operand<j0 + 2>(rows4), b3 = rht_b_operand<j0 + 3>(rows4);
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x16_bf16 %0, %4, %5, 0\n\t"
      "v_mfma_f32_16x16x16_bf16 %1, %4, %6, 0\n\t"
      "v_mfma_f32_16x16x16_bf16 %2, %4, %7, 0\n\t"
      "v_mfma_f32_16x16x16_bf16 %3, %4, %8, 0\n\t"
      "s_nop 7\n\ts_nop 7"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a), "v"(b0), "v"(b1), "v"(b2), "v"(b3));
}

template <int j>
__device__ __forceinline__ f32x4_t rht_mfma(bf16x4_t a, const uint4* rows4) {
  constexpr uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t lo = __builtin_amdgcn_perm(word_of<j / 2>(rows4[1]), word_of<j / 2>(rows4[0]), sel);
  const uint32_t hi = __builtin_amdgcn_perm(word_of<j / 2>(rows4[3]), word_of<j / 2>(rows4[2]), sel);
  const u32x2_t b = {lo, hi};
  const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(bf16x4_t, b), zero, 0, 0, 0);
}

// maximum(m, |a|, |b|), propagating NaN (a NaN or an infinity in the data
// must reach the tensor amax and the status flag).
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
  float r;
  asm("v_maximum3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float max_of(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Largest magnitude of one column's 4 transformed values of this lane.
__device__ __forceinline__ float col_absmax(const f32x4_t& o) {
  return max3_abs(max3_abs(0.0f, o[0], o[1]), o[2], o[3]);
}

struct MfmaTile {
  int64_t tr, tc;
  int64_t r0;      // token of this lane's first row in step 0
  int64_t c0;      // first of this lane's 8 columns
  int steps;       // this wave's steps inside the matrix (0..4), wave-uniform
  bool col_valid;  // the lane's columns exist
};

// kColMajor numbers the tiles down the token dimension first. A column copy
// alone then has the workgroups that run together on an XCD (see xcd_tile)
// write consecutive pieces of the same output rows (columns of x): its code
// and scale bytes leave as longer runs, and the 16-byte scale pieces of one
// 128-byte line meet in the L2. With a row copy too, the band order (see
// band_tile) does it for both copies' scale lines and the row copy's half
// lines.
enum class TileOrder { kRowMajor, kColMajor, kBand };

template <TileOrder kOrder = TileOrder::kRowMajor>
__device__ __forceinline__ MfmaTile locate_mfma(int64_t tile, int64_t rows, int64_t cols) {
  MfmaTile t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tiles_r = (rows + kTileRows - 1) / kTileRows, tiles_c = (cols + kTileCols - 1) / kTileCols;
  if constexpr (kOrder == TileOrder::kColMajor) {
    t.tc = tile / tiles_r;
    t.tr = tile - t.tc * tiles_r;
  } else if constexpr (kOrder == TileOrder::kBand) {
    band_tile(tile, tiles_r, tiles_c, t.tr, t.tc);
  } else {
    t.tr = tile / tiles_c;
    t.tc = tile - t.tr * tiles_c;
  }
  const int64_t wave_r0 = t.tr * kTileRows + 64 * wave;
  const int64_t left = (rows - wave_r0) >> 4;  // whole steps left (rows % 16 == 0)
  t.steps = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left >= kSteps ? kSteps : static_cast<int>(left)));
  t.r0 = wave_r0 + 4 * (lane >> 4);
  t.c0 = t.tc * kTileCols + 8 * (lane & 15);
  t.col_valid = t.c0 < cols;
  return t;
}

// raw[4 s + i] = the 8 bf16 of token r0 + 16 s + i, columns c0 .. c0 + 7,
// for one step s (nontemporal). A step or columns past the matrix read the
// matrix's first 8 values instead (every call has them), which are never
// used, so every load goes out unconditionally.
__device__ __forceinline__ void load_mfma_step(const uint16_t* __restrict__ x, int64_t ldx,
                                               const MfmaTile& t, int s, uint4 (&raw)[16]) {
  const bool ok = t.col_valid && s < t.steps;
  const uint16_t* base = x + (ok ? (t.r0 + 16 * s) * ldx + t.c0 : 0);
  const int64_t stride = ok ? ldx : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[4 * s + i] = load_stream(base + i * stride);
}

__device__ __forceinline__ void load_mfma_raw(const uint16_t* __restrict__ x, int64_t ldx,
                                              const MfmaTile& t, uint4 (&raw)[16]) {
#pragma unroll
  for (int s = 0; s < kSteps; ++s) load_mfma_step(x, ldx, t, s, raw);
}

// Tensor amax of the transformed tensor (and with kDual of the plain one),
// as per-workgroup partial maxima. The amax needs only whole 16-token column
// blocks, so its unit of work is shaped for the loads: a wave takes 32
// tokens x 256 columns (two 16-token steps, two 128-column halves with the
// MFMA lane layout), i.e. 512 contiguous bytes of each row where the
// quantize tile reads 256, which streams at the full read rate. Waves walk
// the units; as soon as a step and half is consumed, the same part of the
// wave's next unit is requested into its registers.
constexpr int kAmaxUnitRows = 32;
constexpr int kAmaxUnitCols = 256;
constexpr int64_t kAmaxUnitsPerBlock = 20;

struct AmaxUnit {
  int64_t r0;                // token of this lane's first row (step 0)
  int64_t c0;                // first of this lane's 8 columns (half 0)
  int steps;                 // steps inside the matrix (0..2), wave-uniform
  bool valid0, valid1;       // the lane's columns exist in half 0 / 1
};

__device__ __forceinline__ AmaxUnit locate_amax_unit(int64_t u, int64_t rows, int64_t cols) {
  AmaxUnit a;
  const int lane = threadIdx.x & 63;
  const int64_t units_c = (cols + kAmaxUnitCols - 1) / kAmaxUnitCols;
  const int64_t ur = u / units_c, uc = u - ur * units_c;
  const int64_t left = (rows - ur * kAmaxUnitRows) >> 4;
  a.steps = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left >= 2 ? 2 : static_cast<int>(left)));
  a.r0 = ur * kAmaxUnitRows + 4 * (lane >> 4);
  a.c0 = uc * kAmaxUnitCols + 8 * (lane & 15);
  a.valid0 = a.c0 < cols;
  a.valid1 = a.c0 + 128 < cols;
  return a;
}

// raw[4 (2 s + hc) + i] = token r0 + 16 s + i, columns c0 + 128 hc .. + 7;
// parts past the matrix read its first 8 values (never used).
__device__ __forceinline__ void load_amax_part(const uint16_t* __restrict__ x, int64_t ldx,
                                               const AmaxUnit& a, int s, int hc, uint4 (&raw)[16]) {
  const bool ok = (hc == 0 ? a.valid0 : a.valid1) && s < a.steps;
  const uint16_t* base = x + (ok ? (a.r0 + 16 * s) * ldx + a.c0 + 128 * hc : 0);
  const int64_t stride = ok ? ldx : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[4 * (2 * s + hc) + i] = load_stream(base + i * stride);
}

template <bool kDual>
__global__ __launch_bounds__(kThreads) void rht_amax_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, uint32_t sign_mask,
    int64_t units, uint32_t* __restrict__ partials, uint32_t* __restrict__ partials_plain) {
  __shared__ uint32_t lds4[kThreads / 64];
  __shared__ uint32_t lds4_plain[kThreads / 64];
  const bf16x4_t a = rht_a_operand(sign_mask);
  float m = 0.0f;
  uint32_t m_plain = 0;  // two packed 16-bit maxima of bf16 magnitudes
  const int64_t wave_stride = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  int64_t u = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) +
              __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  AmaxUnit cu = locate_amax_unit(u, rows, cols);
  uint4 raw[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) load_amax_part(x, ldx, cu, q >> 1, q & 1, raw);
  for (; u < units; u += wave_stride) {
    const AmaxUnit uc = cu;
    const bool has_next = u + wave_stride < units;
    if (has_next) cu = locate_amax_unit(u + wave_stride, rows, cols);
    float mt0 = 0.0f, mt1 = 0.0f;
    uint32_t mp0 = 0, mp1 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = q >> 1, hc = q & 1;
      if (s < uc.steps) {
        const uint4* rs = raw + 4 * q;
        uint32_t mp = hc ? mp1 : mp0;
        if constexpr (kDual) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mp = max_u16x2(mp, rs[i].x & 0x7FFF7FFFu);
            mp = max_u16x2(mp, rs[i].y & 0x7FFF7FFFu);
            mp = max_u16x2(mp, rs[i].z & 0x7FFF7FFFu);
            mp = max_u16x2(mp, rs[i].w & 0x7FFF7FFFu);
          }
        }
        float mt = hc ? mt1 : mt0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4_t o[4];
          if (h == 0) {
            o[0] = rht_mfma<0>(a, rs);
            o[1] = rht_mfma<1>(a, rs);
            o[2] = rht_mfma<2>(a, rs);
            o[3] = rht_mfma<3>(a, rs);
          } else {
            o[0] = rht_mfma<4>(a, rs);
            o[1] = rht_mfma<5>(a, rs);
            o[2] = rht_mfma<6>(a, rs);
            o[3] = rht_mfma<7>(a, rs);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            mt = max3_abs(mt, o[j][0], o[j][1]);
            mt = max3_abs(mt, o[j][2], o[j][3]);
          }
        }
        if (hc) { mt1 = mt; mp1 = mp; } else { mt0 = mt; mp0 = mp; }
      }
      if (has_next) load_amax_part(x, ldx, cu, s, hc, raw);
    }
    // parts whose columns are past the matrix transformed placeholder data
    if (uc.valid0) {
      m = max_of(m, mt0);
      if constexpr (kDual) m_plain = max_u16x2(m_plain, mp0);
    }
    if (uc.valid1) {
      m = max_of(m, mt1);
      if constexpr (kDual) m_plain = max_u16x2(m_plain, mp1);
    }
  }
  block_max_store(__float_as_uint(m), lds4, partials + blockIdx.x);
  if constexpr (kDual) {
    const uint32_t lo = m_plain & 0xFFFFu, hi = m_plain >> 16;
    block_max_store((lo > hi ? lo : hi) << 16, lds4_plain, partials_plain + blockIdx.x);
  }
}

// v kept in a register as it is: the compiler can no longer recompute it
// from its inputs at each use (which it otherwise does for cheap lane
// values, at a cost of several instructions per use in the loops below).
template <typename T>
__device__ __forceinline__ T pinned(T v) {
  asm("" : "+v"(v));
  return v;
}

// Codes of one column pair of this lane (4 tokens each): column q0 in the
// low 16 bits, q1 in the high ones (token i in nibble i of its half).
// mult0 / mult1 are the columns' block multipliers (0 for a zero scale
// byte, whose codes must be 0). For SR, wa / wb hold the random words of the
// two columns' 4 tokens (token i: word i / 2, half i % 2).
// any_zero (wave-uniform) says whether a multiplier of the wave is 0.
template <bool kSR>
__device__ __forceinline__ uint32_t pair_codes(const f32x4_t& o0, const f32x4_t& o1, float mult0,
                                               float mult1, uint32_t wa0, uint32_t wa1,
                                               uint32_t wb0, uint32_t wb1, bool any_zero) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i] = __fmul_rn(o0[i], mult0);
    y[4 + i] = __fmul_rn(o1[i], mult1);
  }
  uint32_t out;
  if constexpr (kSR) {
    out = pack8_sr(y, U4{wa0, wa1, wb0, wb1});
  } else {
    out = pack8_rn(y);
  }
  // a zero scale byte (multiplier 0) gives +-0 values, whose codes must be 0
  if (any_zero) {
    asm volatile("");  // keeps this a branch: not to be computed on every call
    const uint32_t keep = (mult0 != 0.0f ? 0x0000FFFFu : 0u) | (mult1 != 0.0f ? 0xFFFF0000u : 0u);
    out &= keep;
  }
  return out;
}

// One workgroup per 256 x 128 tile: the Hadamard 16x1 column copy of bf16
// x (tokens = rows), and with kDual the 1x16 round-to-nearest row copy from
// the same loads. Field use as quantize_kernel's kModeRHT (no kDual) and
// kModeRowRHT (kDual: the primary fields are the row copy's, the _t ones the
// Hadamard copy's).
// kWideG: group indices can exceed 32 bits (rows x cols >= 2^35), which
// takes the general Philox counter instead of the 32-bit one.
template <bool kDual, bool kSR, bool kWideG>
__global__ __launch_bounds__(kThreads) void rht_quantize_mfma_kernel(QuantParams p) {
  __shared__ __attribute__((aligned(16))) Staging st;
  __shared__ float rtab_h[128];
  __shared__ float rtab_r[kDual ? 128 : 1];
  const int64_t rows = p.rows, cols = p.cols;
  const int64_t ntiles = ((rows + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
  constexpr TileOrder kOrder = kDual ? TileOrder::kBand : TileOrder::kColMajor;
  const MfmaTile t = locate_mfma<kOrder>(xcd_tile(static_cast<int64_t>(blockIdx.x), ntiles), rows, cols);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, r = lane >> 4;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);

  // partial maxima first, then the tile: the reductions, the tables and the
  // barrier wait only for the partials
  const float* amax_in_h = kDual ? p.amax_in_t : p.amax_in;
  const bool reduce_h = amax_in_h == nullptr;
  const bool reduce_r = kDual && p.amax_in == nullptr;
  PartialWords pw_h{}, pw_r{};
  if (reduce_h) load_partials(kDual ? p.partials_t : p.partials, pw_h);
  if (reduce_r) load_partials(p.partials, pw_r);
  uint4 raw[16];
  load_mfma_raw(x, p.ldx, t, raw);
  const float amax_h = reduce_h ? reduce_loaded_partials(pw_h, p.n_partials) : *amax_in_h;
  const float s_h = tensor_scale_from_amax(amax_h);
  const ScaleDiv six_s_h = scale_div(__fmul_rn(6.0f, s_h));
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *(kDual ? p.tensor_scale_t : p.tensor_scale) = s_h;
    float* out = kDual ? p.amax_out_t : p.amax_out;
    if (out != nullptr) *out = amax_h;
    if (!(amax_h <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
  }
  fill_recip_table(rtab_h, s_h);
  ScaleDiv six_s_r = six_s_h;
  if constexpr (kDual) {
    const float amax_r = reduce_r ? reduce_loaded_partials(pw_r, p.n_partials) : *p.amax_in;
    const float s_r = tensor_scale_from_amax(amax_r);
    six_s_r = scale_div(__fmul_rn(6.0f, s_r));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *p.tensor_scale = s_r;
      if (p.amax_out != nullptr) *p.amax_out = amax_r;
      if (!(amax_r <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
    }
    fill_recip_table(rtab_r, s_r);
  }
  __syncthreads();

  const bf16x4_t a = rht_a_operand(p.sign_mask);
  const SrKey key = sr_key(p, kStreamCol);
  const int c_local0 = 8 * n;
  // Lane constants of the loop below. The Philox group of column c and
  // tokens t..t+7 is g = (c rows + t) / 8 = c rows / 8 + t / 8 (rows is a
  // multiple of 16), so each (step, column pair) adds a launch constant to
  // this lane's first group (column c0 + (r & 1), token 8 (r >> 1) of the
  // wave's first step).
  const uint64_t rows8 = static_cast<uint64_t>(rows) >> 3;
  const uint64_t g_lane = pinned(static_cast<uint64_t>(t.c0 + (r & 1)) * rows8 +
                                 static_cast<uint64_t>(t.tr * (kTileRows / 8) + 8 * wave + (r >> 1)));
  const uint32_t join_sel = pinned((r & 1) ? 0x07060302u : 0x05040100u);
  // st.col_scales index of this lane's column {0, 2, 1, 3}[r] (+ 4 h) and
  // step s: this base + 64 h + s
  const int scale_lane = pinned((c_local0 + ((r & 1) << 1 | (r >> 1))) * 16 + 4 * wave);
  // staged_code_offset(c_local0 + j0 + (r & 1), 32 wave + 8 s + 4 (r >> 1))
  // for j0 < 8 and s < 4: the column's granule swizzle is n & 7 and the
  // granule index 2 wave + (s >> 1), so the offset is one of two lane bases
  // plus 128 j0 + 8 (s & 1).
  const int lds_lane = (c_local0 + (r & 1)) * kLdsCodeStride + 4 * (r >> 1);
  const int lds_swz = ((2 * wave) ^ (n & 7)) << 4;
  const int lds_half[2] = {pinned(lds_lane + lds_swz), pinned(lds_lane + (lds_swz ^ 16))};
  // st.row_scales index of this lane's tokens (row copy, even lanes):
  // this base + 8 (16 s + i) for token i of step s
  const int row_scale_lane = pinned((64 * wave + 4 * r) * 8 + (n >> 1));
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s >= t.steps) break;  // wave-uniform
    const uint4* rs = raw + 4 * s;
    const int tok_step = 64 * wave + 16 * s;  // tile-local first token of the step
    if constexpr (kDual) {
      if (t.col_valid) {
        // 1x16 row blocks: this lane's 8 values of a token + lane ^ 1's 8
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w4[4] = {rs[i].x, rs[i].y, rs[i].z, rs[i].w};
          float x8[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x8[2 * k] = bf16_lo(w4[k]);
            x8[2 * k + 1] = bf16_hi(w4[k]);
          }
          // magnitudes: their bits order like their values
          const uint32_t mine = __float_as_uint(abs_max<8>(x8));
          const uint32_t other = swap_adjacent_lanes(mine);
          const BlockMult bs = block_mult(__uint_as_float(mine > other ? mine : other), six_s_r, rtab_r);
          float y[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(x8[k], bs.mult);
          uint32_t w = pack8_rn(y);
          if (__builtin_amdgcn_ballot_w64(bs.byte == 0u) != 0) {
            asm volatile("");  // a rare branch: zero scale bytes, whose codes must be 0
            w = (bs.byte == 0u) ? 0u : w;
          }
          const int64_t tok = t.r0 + 16 * s + i;
          *reinterpret_cast<uint32_t*>(p.q_row + tok * (cols >> 1) + (t.c0 >> 1)) = w;
          if ((n & 1) == 0) st.row_scales[row_scale_lane + (16 * s + i) * 8] = static_cast<uint8_t>(bs.byte);
        }
      }
    }
    // the Hadamard column copy, four columns at a time
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4_t o[4];
      if (h == 0) {
        rht_mfma4<0>(a, rs, o);
      } else {
        rht_mfma4<4>(a, rs, o);
      }
      // block maxima over the columns' 4 lanes (rows r of the lane grid):
      // after the two swaps, lane row r holds column {0, 2, 1, 3}[r] of the four
      const auto s01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(col_absmax(o[0])),
                                                        __float_as_uint(col_absmax(o[1])), false, false);
      const auto s23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(col_absmax(o[2])),
                                                        __float_as_uint(col_absmax(o[3])), false, false);
      const float p01 = max_of(__uint_as_float(s01[0]), __uint_as_float(s01[1]));
      const float p23 = max_of(__uint_as_float(s23[0]), __uint_as_float(s23[1]));
      const auto sq = __builtin_amdgcn_permlane16_swap(__float_as_uint(p01), __float_as_uint(p23), false, false);
      const float bmax = max_of(__uint_as_float(sq[0]), __uint_as_float(sq[1]));
      const BlockMult bm = block_mult(bmax, six_s_h, rtab_h);
      // column {0, 2, 1, 3}[r] + 4 h of this lane's eight
      if (t.col_valid) st.col_scales[scale_lane + 64 * h + s] = static_cast<uint8_t>(bm.byte);
      // every lane needs the multipliers of all four columns
      const uint32_t mb = __float_as_uint(bm.mult);
      // a zero multiplier (zero scale byte) anywhere in the wave: rare, so
      // its code masking runs behind a uniform branch
      const bool any_zero = __builtin_amdgcn_ballot_w64(bm.mult == 0.0f) != 0;
      const auto u = __builtin_amdgcn_permlane16_swap(mb, mb, false, false);  // [c0 c0 c1 c1], [c2 c2 c3 c3]
      const auto v01 = __builtin_amdgcn_permlane32_swap(u[0], u[0], false, false);
      const auto v23 = __builtin_amdgcn_permlane32_swap(u[1], u[1], false, false);
      const float mult[4] = {__uint_as_float(v01[0]), __uint_as_float(v01[1]), __uint_as_float(v23[0]),
                             __uint_as_float(v23[1])};
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        // column pair (4 h + 2 pr, 4 h + 2 pr + 1); the lane grid's rows r and
        // r ^ 1 hold tokens 0-3 and 4-7 of the same 8-token group
        const int j0 = 4 * h + 2 * pr;
        uint32_t wa0 = 0, wa1 = 0, wb0 = 0, wb1 = 0;
        if constexpr (kSR) {
          // the even row draws the group of column j0, the odd row that of
          // j0 + 1; two swaps hand each lane the words of its 4 tokens
          const uint64_t g = g_lane + static_cast<uint64_t>(j0) * rows8 + static_cast<uint64_t>(2 * s);
          U4 w;
          if constexpr (kWideG) {
            w = sr_words(key.k0, key.k1, g, key.offset, key.stream);
          } else {
            w = sr_words_fast(key.ps, static_cast<uint32_t>(g));
          }
          const auto e0 = __builtin_amdgcn_permlane16_swap(w.x, w.z, false, false);
          const auto e1 = __builtin_amdgcn_permlane16_swap(w.y, w.w, false, false);
          wa0 = e0[0];
          wb0 = e0[1];
          wa1 = e1[0];
          wb1 = e1[1];
        }
        const uint32_t codes = pair_codes<kSR>(o[2 * pr], o[2 * pr + 1], mult[2 * pr], mult[2 * pr + 1],
                                               wa0, wa1, wb0, wb1, any_zero);
        // join rows r and r ^ 1: the even row takes column j0's 8 tokens, the
        // odd row column j0 + 1's
        const auto jn = __builtin_amdgcn_permlane16_swap(codes, codes, false, false);
        const uint32_t dw = __builtin_amdgcn_perm(jn[1], jn[0], join_sel);
        if (t.col_valid) {
          *reinterpret_cast<uint32_t*>(st.codes + lds_half[s >> 1] + j0 * kLdsCodeStride + 8 * (s & 1)) = dw;
        }
      }
    }
  }
  __syncthreads();
  store_staged(st, p, t.tr, t.tc, kDual, true, true);
}

// The transformed values of bf16 x, as the kernels above compute them.
__global__ __launch_bounds__(kThreads) void rht_transform_mfma_kernel(const uint16_t* __restrict__ x,
                                                                      int64_t rows, int64_t cols,
                                                                      int64_t ldx, uint32_t sign_mask,
                                                                      float* __restrict__ out) {
  const MfmaTile t = locate_mfma(blockIdx.x, rows, cols);
  uint4 raw[16];
  load_mfma_raw(x, ldx, t, raw);
  const bf16x4_t a = rht_a_operand(sign_mask);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s >= t.steps) break;
    const uint4* rs = raw + 4 * s;
    f32x4_t o[8];
    o[0] = rht_mfma<0>(a, rs);
    o[1] = rht_mfma<1>(a, rs);
    o[2] = rht_mfma<2>(a, rs);
    o[3] = rht_mfma<3>(a, rs);
    o[4] = rht_mfma<4>(a, rs);
    o[5] = rht_mfma<5>(a, rs);
    o[6] = rht_mfma<6>(a, rs);
    o[7] = rht_mfma<7>(a, rs);
    if (t.col_valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4* dst = reinterpret_cast<float4*>(out + (t.r0 + 16 * s + i) * cols + t.c0);
        dst[0] = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
        dst[1] = make_float4(o[4][i], o[5][i], o[6][i], o[7][i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row copy only (1x16 blocks, no column copy): a streaming kernel. Thread
// (ty = tid / 32, tx = tid % 32) of workgroup (bx, by) owns the 32-value
// chunk 32 bx + tx of rows 8 by + ty, 8 (by + gridDim.y) + ty, ...: two
// whole 1x16 blocks in registers (no exchange between lanes), read as one
// contiguous 64-byte run (bf16), written as 16 bytes of codes and 2 scale
// bytes. A wave covers 1 KiB of two rows per load instruction, the loads of
// the next row are in flight while a row is quantized, and the workgroup
// needs LDS only for the reciprocal table.
// ---------------------------------------------------------------------------
constexpr int kRowChunk = 32;    // values per thread and row
constexpr int kRowGroups = 512;  // most workgroups along the rows

template <typename InT>
struct Chunk;

template <>
struct Chunk<uint16_t> {
  uint4 r[4];
  __device__ __forceinline__ float get(int j) const {
    const uint4& v = r[j >> 3];
    const int k = (j >> 1) & 3;
    const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};

template <>
struct Chunk<float> {
  float4 r[8];
  __device__ __forceinline__ float get(int j) const {
    const float4& v = r[j >> 2];
    return (j & 3) == 0 ? v.x : (j & 3) == 1 ? v.y : (j & 3) == 2 ? v.z : v.w;
  }
};

// Loads the chunk's first nblk (1 or 2) blocks; absent blocks read as zero.
template <typename InT>
__device__ __forceinline__ void load_chunk(const InT* __restrict__ src, int nblk, Chunk<InT>& c) {
  constexpr int kPerBlock = 32 / (16 / sizeof(InT)) / 2;  // 16-byte loads per 16 values
#pragma unroll
  for (int i = 0; i < 2 * kPerBlock; ++i) {
    const uint4 v = (i < nblk * kPerBlock) ? reinterpret_cast<const uint4*>(src)[i]
                                           : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (sizeof(InT) == 2) {
      c.r[i] = v;
    } else {
      c.r[i] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                           __uint_as_float(v.w));
    }
  }
}

template <typename InT, bool kSR>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(QuantParams p) {
  __shared__ float rtab[128];
  __shared__ float amax_lds;
  const int64_t rows = p.rows, cols = p.cols;
  const int64_t nblk_row = cols >> 4;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * 32 + tx;
  const int64_t c0 = chunk * kRowChunk;
  // blocks of this chunk that exist: 2, 1 (a row of 16 * odd values) or 0
  const int64_t left = nblk_row - 2 * chunk;
  const int nblk = left >= 2 ? 2 : (left > 0 ? static_cast<int>(left) : 0);
  const int64_t row_step = static_cast<int64_t>(gridDim.y) * 8;
  int64_t row = static_cast<int64_t>(blockIdx.y) * 8 + ty;
  const InT* x = static_cast<const InT*>(p.x);

  Chunk<InT> cur;
  if (row < rows) load_chunk<InT>(x + row * p.ldx + c0, nblk, cur);
  // the tensor amax from the partial maxima: one wave reduces, the others
  // read it after the barrier that also publishes the reciprocal table
  if (threadIdx.x < 64) {
    const float a = p.amax_in != nullptr ? *p.amax_in : reduce_partials(p.partials, p.n_partials);
    if (threadIdx.x == 0) amax_lds = a;
  }
  __syncthreads();
  const float amax = amax_lds;
  const float s = tensor_scale_from_amax(amax);
  const ScaleDiv six_s = scale_div(__fmul_rn(6.0f, s));
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    *p.tensor_scale = s;
    if (p.amax_out != nullptr) *p.amax_out = amax;
    if (!(amax <= 3.402823466e38f) && p.dev_status != nullptr) *p.dev_status = 1;
  }
  fill_recip_table(rtab, s);
  __syncthreads();
  if (nblk == 0) return;  // no barrier below

  // rows of 16 * even values keep 16-byte code and 2-byte scale stores aligned
  const bool wide_stores = (nblk_row & 1) == 0;
  const SrKey key = sr_key(p, kStreamRow);
  for (; row < rows; row += row_step) {
    Chunk<InT> nxt;
    const int64_t next = row + row_step;
    if (next < rows) load_chunk<InT>(x + next * p.ldx + c0, nblk, nxt);
    uint32_t w[4], sb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = cur.get(16 * b + j);
      const BlockMult bm = block_mult(abs_max<16>(v), six_s, rtab);
      float y[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) y[j] = __fmul_rn(v[j], bm.mult);
      if constexpr (kSR) {
        const uint64_t g = (static_cast<uint64_t>(row) * static_cast<uint64_t>(cols) +
                            static_cast<uint64_t>(c0 + 16 * b)) >> 3;
        w[2 * b] = pack8_sr(y, words_for(key, g));
        w[2 * b + 1] = pack8_sr(y + 8, words_for(key, g + 1));
      } else {
        w[2 * b] = pack8_rn(y);
        w[2 * b + 1] = pack8_rn(y + 8);
      }
      const uint32_t keep = (bm.byte == 0u) ? 0u : 0xFFFFFFFFu;
      w[2 * b] &= keep;
      w[2 * b + 1] &= keep;
      sb[b] = bm.byte;
    }
    uint8_t* qdst = p.q_row + row * (cols >> 1) + c0 / 2;
    uint8_t* sdst = p.s_row + row * nblk_row + 2 * chunk;
    if (wide_stores) {
      *reinterpret_cast<uint4*>(qdst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint16_t*>(sdst) = static_cast<uint16_t>(sb[0] | (sb[1] << 8));
    } else {
      *reinterpret_cast<uint2*>(qdst) = make_uint2(w[0], w[1]);
      sdst[0] = static_cast<uint8_t>(sb[0]);
      if (nblk == 2) {
        *reinterpret_cast<uint2*>(qdst + 8) = make_uint2(w[2], w[3]);
        sdst[1] = static_cast<uint8_t>(sb[1]);
      }
    }
    cur = nxt;
  }
}

template <typename InT, bool kSR>
void launch_rows(const QuantParams& p, hipStream_t stream) {
  const int64_t chunks = ((p.cols >> 4) + 1) / 2;
  const int64_t gx = (chunks + 31) / 32;
  int64_t gy = (p.rows + 7) / 8;
  if (gy > kRowGroups) gy = kRowGroups;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  quantize_rows_kernel<InT, kSR><<<grid, kThreads, 0, stream>>>(p);
}

template <typename InT, int kMode, bool kSR>
void launch_quant(const QuantParams& p, hipStream_t stream) {
  const int64_t tiles =
      ((p.rows + kTileRows - 1) / kTileRows) * ((p.cols + kTileCols - 1) / kTileCols);
  quantize_kernel<InT, kMode, kSR><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
}

// Launches the amax kernel for x; returns the number of partial maxima it
// writes (from ws + kPartialsOffset on), or -1 on a launch error.
// With dual (rht only) the maxima of the untransformed values follow, from
// ws + kPartialsOffset + kMaxPartials on.
// Workgroups of the amax kernel launch_amax picks for x, i.e. the number of
// partial maxima it writes (per set of maxima).
int64_t amax_workgroups(int64_t rows, int64_t cols, int64_t ldx, bool rht, int64_t elem_bytes) {
  if (!rht && ldx == cols) {
    const int64_t n = rows * cols;
    const int64_t per_block = static_cast<int64_t>(kThreads) * kFlatUnroll * (16 / elem_bytes);
    const int64_t g = (n + per_block - 1) / per_block;
    return g > kMaxPartials ? kMaxPartials : g;
  }
  if (rht && elem_bytes == 2) {
    // rht_amax_mfma_kernel: waves walk 32 x 256 units; about 20 units per
    // workgroup (5 per wave) measured faster than one unit per wave for the
    // 16384 x 5120 activation (2048 waves against 4096), and large tensors
    // keep kMaxTileBlocks workgroups
    const int64_t units = ((rows + kAmaxUnitRows - 1) / kAmaxUnitRows) *
                          ((cols + kAmaxUnitCols - 1) / kAmaxUnitCols);
    const int64_t g = (units + kAmaxUnitsPerBlock - 1) / kAmaxUnitsPerBlock;
    return g < kMaxTileBlocks ? g : kMaxTileBlocks;
  }
  const int64_t tiles = ((rows + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
  return tiles < kMaxTileBlocks ? tiles : kMaxTileBlocks;
}

template <typename InT>
int launch_amax(const InT* x, int64_t rows, int64_t cols, int64_t ldx, bool rht,
                uint32_t sign_mask, float* amax_ws, hipStream_t stream, bool dual = false) {
  uint32_t* partials = reinterpret_cast<uint32_t*>(amax_ws) + kPartialsOffset;
  uint32_t* partials_plain = partials + kMaxPartials;
  const int64_t g = amax_workgroups(rows, cols, ldx, rht, sizeof(InT));
  if (!rht && ldx == cols) {
    amax_flat_kernel<InT><<<static_cast<unsigned>(g), kThreads, 0, stream>>>(x, rows * cols, partials);
  } else {
    const int64_t tiles = ((rows + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
    const unsigned gg = static_cast<unsigned>(g);
    const bool ragged = (rows % 16) != 0;
    if (rht && sizeof(InT) == 2) {
      const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
      const int64_t units = ((rows + kAmaxUnitRows - 1) / kAmaxUnitRows) *
                            ((cols + kAmaxUnitCols - 1) / kAmaxUnitCols);
      if (dual) {
        rht_amax_mfma_kernel<true><<<gg, kThreads, 0, stream>>>(xb, rows, cols, ldx, sign_mask, units,
                                                                partials, partials_plain);
      } else {
        rht_amax_mfma_kernel<false><<<gg, kThreads, 0, stream>>>(xb, rows, cols, ldx, sign_mask, units,
                                                                 partials, nullptr);
      }
    } else if (rht && dual) {
      amax_tile_kernel<InT, true, false, true><<<gg, kThreads, 0, stream>>>(
          x, rows, cols, ldx, sign_mask, tiles, partials, partials_plain);
    } else if (rht) {
      amax_tile_kernel<InT, true, false><<<gg, kThreads, 0, stream>>>(x, rows, cols, ldx, sign_mask,
                                                                       tiles, partials, nullptr);
    } else if (ragged) {
      amax_tile_kernel<InT, false, true><<<gg, kThreads, 0, stream>>>(x, rows, cols, ldx, sign_mask,
                                                                       tiles, partials, nullptr);
    } else {
      amax_tile_kernel<InT, false, false><<<gg, kThreads, 0, stream>>>(x, rows, cols, ldx, sign_mask,
                                                                        tiles, partials, nullptr);
    }
  }
  return hipGetLastError() == hipSuccess ? static_cast<int>(g) : -1;
}

// The tile kernel serves every call with a column copy or 16x16 blocks; those
// require rows % 16 == 0 (ragged row counts reach only the row-copy kernel).
template <bool kDual, bool kSR>
void launch_rht_mfma(const QuantParams& p, hipStream_t stream) {
  const int64_t tiles =
      ((p.rows + kTileRows - 1) / kTileRows) * ((p.cols + kTileCols - 1) / kTileCols);
  if constexpr (kSR) {
    if (static_cast<uint64_t>(p.rows) * static_cast<uint64_t>(p.cols) >= (uint64_t(1) << 35)) {
      rht_quantize_mfma_kernel<kDual, true, true><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
      return;
    }
  }
  rht_quantize_mfma_kernel<kDual, kSR, false><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(p);
}

template <typename InT>
void dispatch_quant(const QuantParams& p, int mode, bool sr, hipStream_t stream) {
  if constexpr (sizeof(InT) == 2) {
    // bf16 Hadamard paths: the transform on the matrix cores
    if (mode == kModeRHT) {
      if (sr) launch_rht_mfma<false, true>(p, stream);
      else launch_rht_mfma<false, false>(p, stream);
      return;
    }
    if (mode == kModeRowRHT) {
      if (sr) launch_rht_mfma<true, true>(p, stream);
      else launch_rht_mfma<true, false>(p, stream);
      return;
    }
  }
  if (mode == kMode2D) {
    launch_quant<InT, kMode2D, false>(p, stream);
  } else if (mode == kModeRHT) {
    if constexpr (sizeof(InT) == 4) {
      if (sr) launch_quant<InT, kModeRHT, true>(p, stream);
      else launch_quant<InT, kModeRHT, false>(p, stream);
    }
  } else if (mode == kModeRowRHT) {
    if constexpr (sizeof(InT) == 4) {
      if (sr) launch_quant<InT, kModeRowRHT, true>(p, stream);
      else launch_quant<InT, kModeRowRHT, false>(p, stream);
    }
  } else {
    if (sr) launch_quant<InT, kMode1D, true>(p, stream);
    else launch_quant<InT, kMode1D, false>(p, stream);
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

int64_t quantize_workspace_floats(const QuantizeLaunch& q) {
  if (q.rows == 0 || q.cols == 0) return q.amax_in == nullptr ? (q.rht && q.row_too ? 2 : 1) : 0;
  if (q.amax_in != nullptr) return 0;
  const int64_t g = amax_workgroups(q.rows, q.cols, q.ldx, q.rht, q.x_bf16 ? 2 : 4);
  // the second set of maxima (the untransformed ones) starts kMaxPartials later
  return kPartialsOffset + ((q.rht && q.row_too) ? kMaxPartials : 0) + g;
}

int launch_quantize(const QuantizeLaunch& q, hipStream_t stream) {
  const bool bf16 = q.x_bf16;
  const bool dual = q.rht && q.row_too;
  if (q.rows == 0 || q.cols == 0) {
    empty_tensor_kernel<<<1, 64, 0, stream>>>(q.amax_in, q.amax_ws, q.tensor_scale, q.dev_status);
    if (dual) {
      empty_tensor_kernel<<<1, 64, 0, stream>>>(q.amax_in != nullptr ? q.amax_in + 1 : nullptr,
                                                q.amax_ws != nullptr ? q.amax_ws + 1 : nullptr,
                                                q.tensor_scale_t, q.dev_status);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  QuantParams p;
  p.amax_in = q.amax_in;
  p.partials = nullptr;
  p.n_partials = 0;
  p.amax_out = nullptr;
  p.amax_in_t = dual && q.amax_in != nullptr ? q.amax_in + 1 : nullptr;
  p.partials_t = nullptr;
  p.amax_out_t = nullptr;
  p.tensor_scale_t = q.tensor_scale_t;
  if (q.amax_in == nullptr) {
    const int n = bf16 ? launch_amax(static_cast<const uint16_t*>(q.x), q.rows, q.cols, q.ldx,
                                     q.rht, q.sign_mask, q.amax_ws, stream, dual)
                       : launch_amax(static_cast<const float*>(q.x), q.rows, q.cols, q.ldx,
                                     q.rht, q.sign_mask, q.amax_ws, stream, dual);
    if (n < 0) return -1;
    const uint32_t* base = reinterpret_cast<const uint32_t*>(q.amax_ws) + kPartialsOffset;
    p.n_partials = n;
    if (dual) {
      // the row copy: untransformed maxima, amax in ws[0]; the Hadamard copy:
      // transformed maxima, amax in ws[1]
      p.partials = base + kMaxPartials;
      p.amax_out = q.amax_ws;
      p.partials_t = base;
      p.amax_out_t = q.amax_ws + 1;
    } else {
      p.partials = base;
      p.amax_out = q.amax_ws;
    }
  }
  p.x = q.x;
  p.rows = q.rows;
  p.cols = q.cols;
  p.ldx = q.ldx;
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
  const int mode = dual ? kModeRowRHT : (q.rht ? kModeRHT : (q.block_2d ? kMode2D : kMode1D));
  if (mode == kMode1D && q.outputs == 1) {
    // the row copy alone streams through its own kernel
    if (bf16) {
      if (q.sr) launch_rows<uint16_t, true>(p, stream);
      else launch_rows<uint16_t, false>(p, stream);
    } else {
      if (q.sr) launch_rows<float, true>(p, stream);
      else launch_rows<float, false>(p, stream);
    }
  } else if (bf16) {
    dispatch_quant<uint16_t>(p, mode, q.sr, stream);
  } else {
    dispatch_quant<float>(p, mode, q.sr, stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4

namespace nvfp4 {

int launch_tensor_amax(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                       float* amax_ws, hipStream_t stream) {
  return x_bf16 ? launch_amax(static_cast<const uint16_t*>(x), rows, cols, ldx, false, 0u, amax_ws, stream)
                : launch_amax(static_cast<const float*>(x), rows, cols, ldx, false, 0u, amax_ws, stream);
}

int launch_rht_transform(const void* x, bool x_bf16, int64_t tokens, int64_t cols, int64_t ldx,
                         uint32_t sign_mask, float* out, hipStream_t stream) {
  if (tokens == 0 || cols == 0) return 0;
  const int64_t tiles = ((tokens + kTileRows - 1) / kTileRows) * ((cols + kTileCols - 1) / kTileCols);
  if (x_bf16) {
    rht_transform_mfma_kernel<<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(
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
