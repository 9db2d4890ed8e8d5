// Pieces shared by the GEMM kernels on 4-bit operands (NVFP4 and MXFP4):
// direct-to-LDS loads, the swizzled LDS code layout and the epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {
namespace gemm_common {

typedef float floatx16_t __attribute__((ext_vector_type(16)));

// Position (in 16-byte units) of code chunk c of LDS row r. The four 16-byte
// chunks of a 64-byte code row are XOR-swizzled by (r >> 1 ^ r >> 2) & 3, so
// both the DMA's contiguous writes and fragment reads of 16 (or 8)
// consecutive rows hit distinct banks.
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ (((r >> 1) ^ (r >> 2)) & 3); }

// One direct-to-LDS load: every lane fetches kBytes from its own global
// address and the wave's data lands in lane order at LDS byte address
// lds_addr (taken from M0, which needs one wait state after it is written).
// Written as inline assembly so that the compiler does not make unrelated LDS
// reads wait for it; the kernels wait for these loads themselves (vmcnt)
// before the barrier that hands a stage to the other waves.
template <int kBytes>
__device__ __forceinline__ void lds_dma(const uint8_t* gptr, uint32_t lds_addr) {
  if constexpr (kBytes == 16) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
  } else {
    static_assert(kBytes == 4, "4- or 16-byte loads");
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
  }
}

__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt immediate that waits for every vector memory load (vmcnt 0) and
// nothing else (expcnt and lgkmcnt fields at their maximum).
constexpr int kWaitVmcnt0 = 0x0F70;

// Scheduling hints (instruction classes of the gfx9 group scheduler).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;

// Two float32 -> two bf16 (round to nearest even; gfx950 converts a pair in
// one instruction), low half = a.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const bf16x2_t h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

// Stores of C. C is written once and not read back by the kernel, so its
// stores are nontemporal: they do not displace the operand panels that other
// workgroups of the same XCD still read from L2.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_c8(void* dst, uint32_t lo, uint32_t hi) {
  const u32x2_t v = {lo, hi};
  __builtin_nontemporal_store(v, static_cast<u32x2_t*>(dst));
}
__device__ __forceinline__ void store_c16(void* dst, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, static_cast<u32x4_t*>(dst));
}

// Epilogue of a wave's kT x kT accumulator tiles: C = acc * scale. The MFMAs
// took B as their first operand, so each accumulator tile is C^T in the MFMA
// output layout: lane l holds row l % 32 of the 32 x 32 tile and, in elements
// 4g .. 4g + 3, its four consecutive columns 8g + 4(l / 32) .. + 3. They
// leave as one 8-byte (bf16) or 16-byte (float32) store; ragged edges and
// unaligned rows fall back to element stores.
template <int kT, bool kBf16Out>
__device__ __forceinline__ void store_tile(const floatx16_t (&acc)[kT][kT], float scale, void* c,
                                           int64_t ldc, int64_t M, int64_t N, int64_t row0,
                                           int64_t col0, int lane) {
  const int row_l = lane & 31;
  const int col_l = (lane >> 5) * 4;
  const bool vec_ok = ((ldc & 3) == 0) &&
                      ((reinterpret_cast<uintptr_t>(c) & (kBf16Out ? 7u : 15u)) == 0);
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int64_t row = row0 + i * 32 + row_l;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < kT; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = col0 + j * 32 + 8 * g + col_l;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __fmul_rn(acc[i][j][4 * g + e], scale);
        if (vec_ok && col + 3 < N) {
          if constexpr (kBf16Out) {
            store_c8(static_cast<uint16_t*>(c) + row * ldc + col, f32x2_to_bf16x2(v[0], v[1]),
                     f32x2_to_bf16x2(v[2], v[3]));
          } else {
            store_c16(static_cast<float*>(c) + row * ldc + col, __float_as_uint(v[0]),
                      __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e < N) {
              if constexpr (kBf16Out) {
                static_cast<uint16_t*>(c)[row * ldc + col + e] =
                    static_cast<uint16_t>(f32x2_to_bf16x2(v[e], 0.0f) & 0xFFFFu);
              } else {
                static_cast<float*>(c)[row * ldc + col + e] = v[e];
              }
            }
          }
        }
      }
    }
  }
}

// LDS bytes store_tile_lds needs per wave (bf16 C: 128 rows of 272 bytes;
// float32 C: 64 rows of 528 bytes, two passes).
constexpr int kEpilogueRowBf16 = 128 * 2 + 16;
constexpr int kEpilogueRowF32 = 128 * 4 + 16;
constexpr int kEpilogueWaveBytes = 128 * kEpilogueRowBf16;  // >= 64 * kEpilogueRowF32
static_assert(64 * kEpilogueRowF32 <= kEpilogueWaveBytes, "float32 pass fits the bf16 region");

// Epilogue of a wave's 128 x 128 accumulator tile (kT = 4) staged through
// LDS: the wave writes its C values (times scale) row-major into its own
// LDS region (rows padded by 16 bytes), then stores whole rows with 16-byte
// nontemporal stores, so each store instruction writes complete 128-byte
// lines (8 of them) instead of 16-byte pieces of 32 rows. `region` is the wave's LDS
// region (kEpilogueWaveBytes, 16-byte aligned); the caller has finished all
// other use of it (a barrier after the last read and load). Only for a tile
// inside M x N with 16-byte aligned rows of C; others use store_tile.
template <bool kBf16Out>
__device__ __forceinline__ void store_tile_lds(const floatx16_t (&acc)[4][4], float scale, void* c, int64_t ldc,
                                               int64_t row0, int64_t col0, int lane, uint8_t* region) {
  const int row_l = lane & 31;
  const int col_l = (lane >> 5) * 4;
  constexpr int kPasses = kBf16Out ? 1 : 2;      // float32: row blocks 0-1, then 2-3
  constexpr int kRow = kBf16Out ? kEpilogueRowBf16 : kEpilogueRowF32;
  constexpr int kElem = kBf16Out ? 2 : 4;
  constexpr int kRowsPass = 128 / kPasses;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
    for (int ii = 0; ii < 4 / kPasses; ++ii) {
      const int i = pass * (4 / kPasses) + ii;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __fmul_rn(acc[i][j][4 * g + e], scale);
          uint8_t* dst = region + (ii * 32 + row_l) * kRow + (j * 32 + 8 * g + col_l) * kElem;
          if constexpr (kBf16Out) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
    }
    // the wave's own LDS writes are complete before it reads them back
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    constexpr int kChunks = 128 * kElem / 16;  // 16-byte chunks per row
    constexpr int kRowsPerStore = 64 / kChunks;
#pragma unroll
    for (int q = 0; q < kRowsPass / kRowsPerStore; ++q) {
      const int r = q * kRowsPerStore + lane / kChunks, ch = lane % kChunks;
      const uint4 v = *reinterpret_cast<const uint4*>(region + r * kRow + 16 * ch);
      uint8_t* out = static_cast<uint8_t*>(c) + ((row0 + pass * kRowsPass + r) * ldc + col0) * kElem + 16 * ch;
      store_c16(out, v.x, v.y, v.z, v.w);
    }
    if constexpr (kPasses > 1) {
      // the next pass overwrites the region: this pass's reads are done
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  }
}

// Workgroup b -> C tile (row-major tile index) for the 256 x 256 GEMM
// tiles. Workgroups are handed to the 8 XCDs in turn (b % 8), and each XCD
// has its own L2. When the tile grid divides into blocks of 32 tiles (4 tile
// rows x 8 tile columns, else 8 x 4), the 32 workgroups an XCD runs side by
// side take one block, so they read 12 operand panels between them (in
// row-major order about 13, spread over several panel rows and, started at
// different times, reused less from L2). Blocks are taken 8 at a time, one
// per XCD, in row-major block order; blocks past the last full set of 8
// follow in plain order. Other grids keep row-major order. A bijection on
// [0, tiles_m * tiles_n).
__device__ __forceinline__ int64_t tile_of(int64_t b, int64_t tiles_m, int64_t tiles_n) {
  int bh, lw;  // block height in tile rows; log2 of its width
  if ((tiles_m & 3) == 0 && (tiles_n & 7) == 0) {
    bh = 4;
    lw = 3;
  } else if ((tiles_m & 7) == 0 && (tiles_n & 3) == 0) {
    bh = 8;
    lw = 2;
  } else {
    return b;
  }
  const int64_t blocks_n = tiles_n >> lw;
  const int64_t blocks = (tiles_m / bh) * blocks_n;
  const int64_t full = blocks & ~static_cast<int64_t>(7);
  int64_t blk, i;
  if (b < full * 32) {
    const int64_t l = b >> 3;  // this XCD's l-th workgroup
    blk = (l >> 5) * 8 + (b & 7);
    i = l & 31;
  } else {
    blk = full + ((b - full * 32) >> 5);
    i = (b - full * 32) & 31;
  }
  const int64_t bm = blk / blocks_n, bn = blk - bm * blocks_n;
  return (bm * bh + (i >> lw)) * tiles_n + (bn << lw) + (i & ((1 << lw) - 1));
}

// Writes zeros to C (the K == 0 product).
__global__ void zero_output_kernel(void* c, int64_t M, int64_t N, int64_t ldc, bool bf16);

}  // namespace gemm_common
}  // namespace nvfp4
