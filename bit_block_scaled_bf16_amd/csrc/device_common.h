// Device-side building blocks of the NVFP4 kernels (gfx950).
//
// Number formats (gist.science summary of "Pretraining Large Language Models
// with NVFP4", Resumen técnico §2 "Formato NVFP4"): 4-bit E2M1 elements, E4M3
// block scales, an FP32 tensor scale. The exact rounding rules are the
// library's definitions stated in include/nvfp4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Scalars of the two-level scaling.
// ---------------------------------------------------------------------------

// Largest E2M1 magnitude times largest E4M3 value: the tensor amax maps to
// the top of both ranges.
constexpr float kTensorScaleDivisor = 2688.0f;
// Tensor scales below 2^-100 are replaced by 1 (the tensor quantizes to 0).
constexpr float kTensorScaleFloor = 7.888609052210118e-31f;  // 2^-100

// float32 tensor decode scale from the tensor amax.
__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
  float s = __fdiv_rn(amax, kTensorScaleDivisor);
  return (s < kTensorScaleFloor) ? 1.0f : s;  // also maps amax == 0 to 1
}

// E4M3FN byte nearest to t (t >= 0, finite), ties to even mantissa,
// saturating at 448 (0x7E). gfx950's converter rounds to nearest even into
// OCP E4M3FN, subnormals included, but gives NaN above 464, hence the clamp
// (checked against the CPU definition for every float32 near every E4M3
// value and midpoint).
__device__ __forceinline__ uint32_t e4m3_from_float(float t) {
  // t >= 0, whose bits order like its value: an integer minimum clamps it
  // (a NaN's bits lie above 448's, so a NaN clamps to 448 as with fminf)
  const uint32_t tb = __float_as_uint(t);
  const float c = __uint_as_float(tb < 0x43E00000u ? tb : 0x43E00000u);
  // old value 0 and second value +0, whose E4M3 byte is 0: bytes 1..3 of
  // the result are 0
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false));
}

// Value of an E4M3FN byte b in 0x00..0x7E, branch-free: b << 20 places the
// 4 exponent and 3 mantissa bits at the top of a float32 exponent / mantissa,
// which is the value times 2^-120 for normal bytes and, as a float32
// subnormal, m * 2^-129 = (m * 2^-9) * 2^-120 for subnormal ones; the
// multiply by 2^120 is exact (float32 subnormals are kept).
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  return __uint_as_float((b & 0x7Fu) << 20) * 0x1p120f;
}

// ---------------------------------------------------------------------------
// E2M1 rounding.
// ---------------------------------------------------------------------------

// Two round-to-nearest-even E2M1 codes (a in the low nibble, b in the high
// nibble) written into byte `sel` of `old`. gfx950's converter with scale
// 1.0 implements exactly the rounding of include/nvfp4.h: nearest, ties to
// the even code, saturation at 6, the sign bit of the input kept (checked
// against the CPU definition over every float near every tie, and by the
// parity tests).
template <int sel>
__device__ __forceinline__ uint32_t cvt_pk_e2m1_rn(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, sel);
}

// Eight RN codes packed into one 32-bit word, element j in nibble j.
__device__ __forceinline__ uint32_t pack8_rn(const float* y) {
  // the four converts write all four bytes; starting from a live value
  // instead of 0 saves a register move
  uint32_t w = __float_as_uint(y[0]);
  w = cvt_pk_e2m1_rn<0>(w, y[0], y[1]);
  w = cvt_pk_e2m1_rn<1>(w, y[2], y[3]);
  w = cvt_pk_e2m1_rn<2>(w, y[4], y[5]);
  w = cvt_pk_e2m1_rn<3>(w, y[6], y[7]);
  return w;
}

// Stochastic rounding of y to E2M1 from 16 random bits u16: with
// a = min(|y|, 6), lo the largest magnitude <= a and hi the next one, round
// up exactly when (a - lo) / (hi - lo) + u16 / 2^16 >= 1.
//
// Scaled by 2^-126, the E2M1 grid is float32's own bit layout: 1.0 becomes
// the smallest normal, the magnitudes below 1 fall in the subnormal range
// with its uniform spacing, and each binade above holds two grid points,
// like one mantissa bit. So the bits of z = y * 2^-126 rounded toward zero
// hold y's sign in bit 31, lo's code from bit 22 up and frac * 2^22 below:
// exactly for |y| >= 1 (a power-of-two scaling of a normal number), and as
// floor(|y| * 2^23) for |y| < 1 (toward zero onto the subnormal grid, which
// drops only bits below 2^-22 of a step). Adding u16 * 2^6 carries into bit
// 22 exactly when frac + u16 / 2^16 >= 1: u16 * 2^6 has no bits below 2^6,
// so the bits of frac * 2^22 below 2^6 cannot complete a carry. Clearing the
// fraction bits gives the chosen grid value times 2^-126 with y's sign; the
// round-to-nearest converter, told to scale by 2^126, encodes it exactly,
// and a value past 6 (|y| > 6) lands on 6 through its saturation.
//
// The toward-zero multiplies switch the wave's float32 rounding mode (MODE
// bits 1:0) around eight multiplies in one assembly block and restore round
// to nearest even, the kernels' mode, before the block ends; s_nop 1 gives
// the mode write two wait states before the VALU reads it.
__device__ __forceinline__ void scale_rz8(const float* y, uint32_t (&z)[8]) {
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_e64 %0, %8, %16\n\t"
      "v_mul_f32_e64 %1, %9, %16\n\t"
      "v_mul_f32_e64 %2, %10, %16\n\t"
      "v_mul_f32_e64 %3, %11, %16\n\t"
      "v_mul_f32_e64 %4, %12, %16\n\t"
      "v_mul_f32_e64 %5, %13, %16\n\t"
      "v_mul_f32_e64 %6, %14, %16\n\t"
      "v_mul_f32_e64 %7, %15, %16\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
      "s_nop 1"
      : "=&v"(z[0]), "=&v"(z[1]), "=&v"(z[2]), "=&v"(z[3]), "=&v"(z[4]), "=&v"(z[5]),
        "=&v"(z[6]), "=&v"(z[7])
      : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]),
        "s"(0x1p-126f));
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11).
// ---------------------------------------------------------------------------

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(uint32_t k0, uint32_t k1, U4 c) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c.z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    // three-way xors as one gfx950 v_bitop3_b32 each (truth table 0x96)
    c = U4{static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96)), lo1,
           static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96)), lo0};
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

// Random words for the 8 elements of group g (element 2i uses the low half
// of word i, element 2i+1 the high half).
__device__ __forceinline__ U4 sr_words(uint32_t k0, uint32_t k1, uint64_t g, uint32_t offset,
                                       uint32_t stream) {
  return philox4x32_10(k0, k1,
                       U4{static_cast<uint32_t>(g), static_cast<uint32_t>(g >> 32), offset, stream});
}

// Philox4x32-10 for the counters of stochastic rounding, (g, 0, offset,
// stream) with g < 2^32 (tensors of fewer than 2^35 elements): the first
// round's product M1 * offset and the second round's M0 * x1 are the same for
// every counter of a launch, so they are formed once, and a counter costs 18
// wide multiplies instead of 20. The words equal philox4x32_10's.
struct PhiloxSr {
  uint32_t k0, k1;   // key
  uint32_t x1;       // round 1 output word 0: hi(M1 offset) ^ k0
  uint32_t y1k;      // lo(M1 offset) ^ (k0 + W0), xored into round 2's word 0
  uint32_t z1k;      // stream ^ k1, xored into round 1's word 2
  uint32_t d_hi_k;   // hi(M0 x1) ^ (k1 + W1), xored into round 2's word 2
  uint32_t w2k;      // lo(M0 x1) ^ (k1 + 2 W1), xored into round 3's word 2
};

__device__ __forceinline__ PhiloxSr philox_sr_setup(uint32_t k0, uint32_t k1, uint32_t offset,
                                                    uint32_t stream) {
  PhiloxSr ps;
  ps.k0 = __builtin_amdgcn_readfirstlane(k0);
  ps.k1 = __builtin_amdgcn_readfirstlane(k1);
  const uint32_t off = __builtin_amdgcn_readfirstlane(offset);
  const uint64_t a = static_cast<uint64_t>(kPhiloxM1) * off;
  ps.x1 = static_cast<uint32_t>(a >> 32) ^ ps.k0;
  ps.y1k = static_cast<uint32_t>(a) ^ (ps.k0 + kPhiloxW0);
  ps.z1k = stream ^ ps.k1;
  const uint64_t d = static_cast<uint64_t>(kPhiloxM0) * ps.x1;
  ps.d_hi_k = static_cast<uint32_t>(d >> 32) ^ (ps.k1 + kPhiloxW1);
  ps.w2k = static_cast<uint32_t>(d) ^ (ps.k1 + 2u * kPhiloxW1);
  return ps;
}

__device__ __forceinline__ U4 sr_words_fast(const PhiloxSr& ps, uint32_t g) {
  // round 1: (hi(M1 off) ^ 0 ^ k0, lo(M1 off), hi(M0 g) ^ stream ^ k1, lo(M0 g))
  const uint64_t b = static_cast<uint64_t>(kPhiloxM0) * g;
  const uint32_t z1 = static_cast<uint32_t>(b >> 32) ^ ps.z1k, w1 = static_cast<uint32_t>(b);
  // round 2: word 0 from M1 z1, words 2 and 3 from M0 x1 (launch constants)
  const uint64_t c = static_cast<uint64_t>(kPhiloxM1) * z1;
  U4 r{static_cast<uint32_t>(c >> 32) ^ ps.y1k, static_cast<uint32_t>(c), w1 ^ ps.d_hi_k, 0u};
  // round 3: word 3 of round 2 is the launch constant lo(M0 x1)
  uint32_t k0 = ps.k0 + 2u * kPhiloxW0, k1 = ps.k1 + 2u * kPhiloxW1;
  {
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * r.x;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * r.z;
    r = U4{static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), r.y, k0, 0x96)),
           static_cast<uint32_t>(p1), static_cast<uint32_t>(p0 >> 32) ^ ps.w2k, static_cast<uint32_t>(p0)};
  }
#pragma unroll
  for (int round = 3; round < 10; ++round) {
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * r.x;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * r.z;
    r = U4{static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), r.y, k0, 0x96)),
           static_cast<uint32_t>(p1),
           static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), r.w, k1, 0x96)),
           static_cast<uint32_t>(p0)};
  }
  return r;
}

// z + u16 * 2^6, u16 the low (hi == 0) or high half of the random word w:
// one v_mad_u32_u16, which reads either half of its first source (op_sel).
__device__ __forceinline__ uint32_t sr_add(uint32_t z, uint32_t w, int hi) {
  uint32_t t;
  if (hi) {
    asm("v_mad_u32_u16 %0, %1, 64, %2 op_sel:[1,0,0,0]" : "=v"(t) : "v"(w), "v"(z));
  } else {
    asm("v_mad_u32_u16 %0, %1, 64, %2" : "=v"(t) : "v"(w), "v"(z));
  }
  return t;
}

// Eight SR codes for y[0..7] from one Philox block (element j in nibble j).
// The converter's scale operand acts as a power of two and divides: with
// scale 2^-126 it encodes the chosen grid value t * 2^126 directly, the
// subnormal t = 2^-127 (the value 0.5) included.
__device__ __forceinline__ uint32_t pack8_sr(const float* y, U4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t z[8];
  scale_rz8(y, z);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(sr_add(z[j], ws[j >> 1], j & 1) & 0xFFC00000u);
  uint32_t out = __float_as_uint(v[0]);  // every byte is written below
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[0], v[1], 0x1p-126f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[2], v[3], 0x1p-126f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[4], v[5], 0x1p-126f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[6], v[7], 0x1p-126f, 3);
  return out;
}

constexpr uint32_t kStreamRow = 0;
constexpr uint32_t kStreamCol = 1;

// ---------------------------------------------------------------------------
// Loads.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |x| as ordered integer bits (float32 layout): larger bits = larger |x|,
// NaN above infinity.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------------------
// 16-point Hadamard transform (Sylvester order) of the signed values, in
// float32 with a fixed butterfly order: pair distances 1, 2, 4, 8, each
// mapping (a, b) -> (a + b, a - b), then a multiply by 1/4 (exact).
// sign_mask bit i set means the input i is negated first.
// ---------------------------------------------------------------------------

// The signs as +-1.0 floats (the same for every column of a launch).
struct RhtSigns {
  float d[16];
};

__device__ __forceinline__ RhtSigns rht_signs(uint32_t sign_mask) {
  RhtSigns g;
#pragma unroll
  for (int i = 0; i < 16; ++i) g.d[i] = ((sign_mask >> i) & 1u) ? -1.0f : 1.0f;
  return g;
}

// The transform without the final 1/4. The signs ride on the first stage:
// t = d_b * b is exact and fma(d_a, a, +-t) rounds d_a a +- d_b b once, as
// the add of the negated values does.
__device__ __forceinline__ void rht16_unscaled(float* v, const RhtSigns& g) {
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const float t = __fmul_rn(g.d[i + 1], v[i + 1]);
    const float a = v[i];
    v[i] = __builtin_fmaf(g.d[i], a, t);
    v[i + 1] = __builtin_fmaf(g.d[i], a, -t);
  }
#pragma unroll
  for (int h = 2; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = __fadd_rn(a, b);
        v[i + h] = __fsub_rn(a, b);
      }
    }
  }
}

__device__ __forceinline__ void rht16(float* v, const RhtSigns& g) {
  rht16_unscaled(v, g);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __fmul_rn(v[i], 0.25f);
}

// Exchange with the neighbouring lane (lane ^ 1) through DPP.
__device__ __forceinline__ uint32_t swap_adjacent_lanes(uint32_t v) {
  // quad_perm [1, 0, 3, 2]
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
}

// Maximum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64));
    v = (o > v) ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Tensor amax workspace (floats): [0] receives the amax, the per-workgroup
// partial maxima of the amax kernels (float bits, which order like unsigned
// integers for non-negative values, NaN above infinity) start at
// kPartialsOffset.
// ---------------------------------------------------------------------------
constexpr int kPartialsOffset = 64;
constexpr int kMaxPartials = 1024;

// The tensor amax from n <= kMaxPartials partial maxima. Each wave reduces
// them on its own: 4 loads of 16 bytes per lane, all issued before the
// first is needed (entries past n hold stale values and are masked off,
// and the loads stay inside the workspace), then a wave maximum: no LDS, no
// barrier. The loads and the reduction are separate steps so that a kernel
// can issue its own loads in between and still wait for these alone
// (a wave's loads complete in the order they were issued).
struct PartialWords {
  uint4 b[kMaxPartials / 256];
};

__device__ __forceinline__ void load_partials(const uint32_t* __restrict__ partials, PartialWords& w) {
  const int lane = threadIdx.x & 63;
  const uint4* p4 = reinterpret_cast<const uint4*>(partials);
#pragma unroll
  for (int k = 0; k < kMaxPartials / 256; ++k) w.b[k] = p4[lane + 64 * k];
}

__device__ __forceinline__ float reduce_loaded_partials(const PartialWords& w, int n) {
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kMaxPartials / 256; ++k) {
    const int i = 4 * (lane + 64 * k);
    const uint32_t v[4] = {w.b[k].x, w.b[k].y, w.b[k].z, w.b[k].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t x = i + c < n ? v[c] : 0u;
      m = x > m ? x : m;
    }
  }
  return __uint_as_float(wave_max_u32(m));
}

__device__ __forceinline__ float reduce_partials(const uint32_t* __restrict__ partials, int n) {
  PartialWords w;
  load_partials(partials, w);
  return reduce_loaded_partials(w, n);
}

}  // namespace nvfp4
