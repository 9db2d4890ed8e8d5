/*
 * nvfp4.h -- C ABI of the NVFP4 quantizer and NVFP4 GEMM for AMD MI355X
 * (gfx950).
 *
 * NVFP4 stores a tensor as 4-bit E2M1 codes (two per byte), one E4M3 scale
 * byte per block of 16 elements (1x16, 16x1) or per 16x16 tile, and one FP32
 * tensor scale. The format and the training recipe come from NVIDIA's report
 * "Pretraining Large Language Models with NVFP4" as summarised on
 * gist.science (Resumen técnico §2: "Formato NVFP4" -- 16-element blocks, E4M3
 * block scale, FP32 tensor scale; "Transformadas de Hadamard Aleatorias
 * (RHT)" -- 16x16 Hadamard transform with a fixed random sign vector on the
 * weight-gradient inputs; "Escalado Bidimensional (2D) y Redondeo
 * Estocástico" -- 16x16 weight blocks, stochastic rounding of gradients;
 * "Precisión Mixta Selectiva" -- the GEMMs run on NVFP4 operands).
 *
 * Numerics (the pages give none; these are the library's definitions, all in
 * float32 with round-to-nearest-even unless stated):
 *   A   = max |x| over the tensor (after the transform on the RHT path)
 *   S   = A / 2688   (2688 = 6 * 448); S := 1 when A / 2688 < 2^-100
 *   per block: s_b = E4M3_rne_sat(a_b / (6 * S)); s_f = value(s_b)
 *              r = 1 / (s_f * S), or every code 0 when s_f == 0
 *   per element: y = x * r; q = E2M1 round-to-nearest-even (ties to the code
 *              with mantissa bit 0, |y| > 6 -> 6, sign bit of y kept), or
 *              stochastic: a = min(|y|, 6), lo <= a < hi the adjacent E2M1
 *              magnitudes (lo = hi = 6 when a = 6); round up to hi exactly
 *              when (a - lo) / (hi - lo) + u16 / 2^16 >= 1, compared exactly
 *              (the random fraction is added below the step and the sum
 *              truncated: up-probability floor(frac * 2^16) / 2^16); the
 *              sign bit of y is kept
 *   SR example: y = 2.5, u16 = 32767 -> code 0x4; u16 = 32768 -> code 0x5
 *   SR example: y = -0.75, u16 = 32767 -> code 0x9; u16 = 32768 -> code 0xA
 *   SR example: y = 0.25, u16 = 32767 -> code 0x0; u16 = 32768 -> code 0x1
 *   SR example: y = 6.0, u16 = 65535 -> code 0x7
 *   u16 for element e (row-major index of the stored matrix): Philox4x32-10
 *              with key (seed lo, seed hi), counter (e>>3 lo, e>>3 hi,
 *              offset, stream), word (e&7)>>1, half e&1 (0 = low 16 bits);
 *              stream 0 = row-blocked copy, 1 = column-blocked copy
 *   RHT of 16 consecutive tokens x of one column: x' = (1/4) H (d .* x),
 *              H the Sylvester 16x16 Hadamard matrix (H[i][j] =
 *              (-1)^popcount(i&j)), d_i = 1 - 2 * bit i of word 0 of
 *              Philox4x32-10(key = rht_seed, counter (0, 0, 0, 2))
 *   dequant:   x_hat = (e2m1(q) * s_f) * S
 *
 * Layouts (all row-major, dense, owned by the caller):
 *   codes: byte j of a row holds element 2j (low nibble) and 2j+1 (high).
 *   row-blocked copy of an R x C matrix:    codes [R][C/2], scales [R][C/16]
 *   column-blocked copy (16x1 blocks), stored as the quantized transpose:
 *                                            codes [C][R/2], scales [C][R/16]
 *   16x16 blocks: codes [R][C/2] and [C][R/2] (transposed), scale grid
 *                 [R/16][C/16] and its transpose [C/16][R/16].
 *
 * Conventions shared by every entry point:
 *   - Every pointer except the host-side ones named so is a DEVICE pointer
 *     owned by the caller; the library never allocates, frees or keeps
 *     pointers, and keeps no state between calls (thread-safe).
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *   - Argument errors are detected on the host before any HIP call and
 *     returned synchronously; nothing is enqueued then.
 *   - Device pointers must be 16-byte aligned; leading dimensions in
 *     elements must keep every row 16-byte aligned.
 *   - Data-dependent conditions never synchronise: a non-finite tensor amax
 *     stores 1 into *dev_status (when dev_status is not NULL); the outputs
 *     are then unspecified. The library never writes 0 there.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,  /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2, /* a size or leading dimension is invalid */
  NVFP4_ERR_ENUM = 3,  /* unknown enum value or unsupported combination */
  NVFP4_ERR_ALIGN = 4, /* a pointer or row is not 16-byte aligned */
  NVFP4_ERR_HIP = 5    /* a kernel launch failed (hipGetLastError) */
};

/* Element types of inputs and outputs. */
enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 };
/* Block shapes. */
enum { NVFP4_BLOCK_1D = 0, NVFP4_BLOCK_2D = 1 };
/* Rounding of the elements. */
enum { NVFP4_ROUND_RN = 0, NVFP4_ROUND_SR = 1 };
/* Output orientations (bit mask). */
enum { NVFP4_OUT_ROW = 1, NVFP4_OUT_COL = 2 };

/* Size of the amax workspace (amax_ws) of nvfp4_quantize and
 * nvfp4_rht_quantize. Its first float receives the tensor amax; the rest
 * holds per-workgroup partial maxima between the two kernels of a call and
 * needs no initial value. The library cannot check the size of a plain
 * pointer: a smaller buffer is written out of bounds. */
#define NVFP4_AMAX_WS_BYTES 16384

/*
 * nvfp4_quantize -- two-level NVFP4 quantization of an R x C matrix.
 * (gist.science summary, Resumen técnico §2 "Formato NVFP4"; for 16x16 blocks
 * §2 "Escalado Bidimensional (2D) y Redondeo Estocástico".)
 *
 *   x          [rows][ldx] input, x_dtype NVFP4_F32 or NVFP4_BF16.
 *   rows, cols  >= 0. cols % 16 == 0. rows % 16 == 0 when NVFP4_OUT_COL is
 *               requested or block == NVFP4_BLOCK_2D. rows == 0 or cols == 0
 *               is an empty tensor: only *tensor_scale (= 1) and amax_ws[0]
 *               (= 0) are written.
 *   ldx         >= cols.
 *   block       NVFP4_BLOCK_1D: row copy in 1x16 blocks along cols, column
 *               copy in 16x1 blocks along rows. NVFP4_BLOCK_2D: 16x16 tiles,
 *               one scale each; the column copy holds the transposed codes,
 *               which dequantize to exactly the transpose of the row copy.
 *   rounding    NVFP4_ROUND_RN or NVFP4_ROUND_SR (SR with BLOCK_2D is
 *               NVFP4_ERR_ENUM: the recipe rounds weights to nearest).
 *   seed, offset  Philox key and counter word 2 for SR (ignored for RN).
 *   outputs     non-empty mask of NVFP4_OUT_ROW / NVFP4_OUT_COL; both are
 *               produced from one read of x and share the tensor scale.
 *   amax_in     NULL, or 1 float: the tensor amax to use instead of
 *               computing it (e.g. from an earlier pass).
 *   amax_ws     NVFP4_AMAX_WS_BYTES of workspace, required when amax_in is
 *               NULL; amax_ws[0] holds the computed amax afterwards.
 *   q_row, s_row  row copy codes [rows][cols/2] and scales [rows][cols/16]
 *               (1D) or grid [rows/16][cols/16] (2D); required with OUT_ROW.
 *   q_col, s_col  column copy codes [cols][rows/2] and scales [cols][rows/16]
 *               (1D) or grid^T [cols/16][rows/16] (2D); required with OUT_COL.
 *   tensor_scale  out: 1 float, S (decode scale) for dequantize and GEMM.
 *   dev_status    NULL or 1 int32, set to 1 on a non-finite amax.
 */
int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                   int block, int rounding, uint64_t seed, uint32_t offset, int outputs,
                   const float* amax_in, float* amax_ws, uint8_t* q_row, uint8_t* s_row,
                   uint8_t* q_col, uint8_t* s_col, float* tensor_scale, int32_t* dev_status,
                   hipStream_t stream);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, hosts that
 * forbid allocation): the same arguments without amax_ws, the same outputs
 * bit for bit. The amax pass uses a workspace inside the library instead: a
 * static device array of NVFP4_AMAX_WS_BYTES (16 KiB) per GPU, held until
 * the process ends. Its device address is looked up on the first call on
 * each device (with that device current); no call allocates or frees
 * memory, or synchronises.
 *
 *   Every call on one GPU shares that GPU's workspace, and each call leaves
 *   its partial maxima in it (none needs an initial value). Calls whose work
 *   may overlap on one GPU (different streams, unordered host threads) race
 *   on it: order them on one stream. The workspace need does not grow with
 *   the tensor (at most NVFP4_AMAX_WS_BYTES for any shape nvfp4_quantize
 *   accepts); a call that would need more returns NVFP4_ERR_SHAPE. The
 *   tensor amax itself is not returned (tensor_scale is).
 *   Errors: those of nvfp4_quantize (amax_in == NULL is allowed), checked
 *   before any HIP call; NVFP4_ERR_HIP when the workspace's address cannot
 *   be found or a launch fails.
 */
int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                           int block, int rounding, uint64_t seed, uint32_t offset, int outputs,
                           const float* amax_in, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                           uint8_t* s_col, float* tensor_scale, int32_t* dev_status,
                           hipStream_t stream);

/*
 * nvfp4_rht_quantize -- weight-gradient operand path: 16-point random
 * Hadamard transform along the token dimension, then 16x1 NVFP4 blocks along
 * tokens, stored transposed so the token dimension is the GEMM K dimension.
 * (gist.science summary, Resumen técnico §2 "Transformadas de Hadamard
 * Aleatorias (RHT)" and "... Redondeo Estocástico"; news.hamidun.com,
 * "Cómo Funciona".)
 *
 *   x          [tokens][ldx], x_dtype NVFP4_F32 or NVFP4_BF16.
 *   tokens     >= 0, multiple of 16. cols >= 0, multiple of 16. ldx >= cols.
 *   rht_seed   selects the fixed sign vector d (same seed on both operands
 *              of one weight-gradient GEMM).
 *   rounding, seed, offset  as nvfp4_quantize (stream word 1).
 *   amax_in    NULL or 1 float: amax of the transformed tensor.
 *   amax_ws    NVFP4_AMAX_WS_BYTES of workspace, required when amax_in is
 *              NULL (amax_ws[0] holds the amax of the transformed tensor
 *              afterwards).
 *   q_t        codes [cols][tokens/2]; s_t scales [cols][tokens/16].
 *   tensor_scale, dev_status  as nvfp4_quantize.
 */
int nvfp4_rht_quantize(const void* x, int x_dtype, int64_t tokens, int64_t cols, int64_t ldx,
                       uint64_t rht_seed, int rounding, uint64_t seed, uint32_t offset,
                       const float* amax_in, float* amax_ws, uint8_t* q_t, uint8_t* s_t,
                       float* tensor_scale, int32_t* dev_status, hipStream_t stream);

/*
 * nvfp4_quantize_row_rht -- both NVFP4 copies of one activation from one
 * read: the 1x16 row copy (round to nearest, the forward operand) and the
 * Hadamard-transformed 16x1 column copy of nvfp4_rht_quantize (the
 * weight-gradient operand). Each copy has its own tensor amax and tensor
 * scale, so every output equals, bit for bit, that of nvfp4_quantize(block
 * 1D, RN, OUT_ROW) and of nvfp4_rht_quantize on the same x.
 * (gist.science summary, Resumen técnico §2 "Formato NVFP4" for the row
 * copy, "Transformadas de Hadamard Aleatorias (RHT)" for the column copy,
 * which the recipe applies only to the weight-gradient inputs.)
 *
 *   x, x_dtype, tokens, cols, ldx, rht_seed  as nvfp4_rht_quantize.
 *   rounding_t, seed, offset  rounding of the column copy (and its Philox key
 *              and counter word 2 for SR); the row copy always rounds to
 *              nearest.
 *   amax_in    NULL, or 2 floats: [0] the amax of x, [1] the amax of the
 *              transformed x.
 *   amax_ws    NVFP4_AMAX_WS_BYTES of workspace, required when amax_in is
 *              NULL; afterwards amax_ws[0] and amax_ws[1] hold the two
 *              amaxes in the order of amax_in.
 *   q_row, s_row  row copy: codes [tokens][cols/2], scales [tokens][cols/16].
 *   tensor_scale_row  out: 1 float, the row copy's S.
 *   q_t, s_t   column copy: codes [cols][tokens/2], scales [cols][tokens/16].
 *   tensor_scale_t    out: 1 float, the column copy's S.
 *   dev_status  as nvfp4_quantize (set on either non-finite amax).
 * tokens == 0 or cols == 0 writes only the two tensor scales (= 1) and
 * amax_ws[0..1] (= 0). All four output arrays are required otherwise.
 */
int nvfp4_quantize_row_rht(const void* x, int x_dtype, int64_t tokens, int64_t cols, int64_t ldx,
                           uint64_t rht_seed, int rounding_t, uint64_t seed, uint32_t offset,
                           const float* amax_in, float* amax_ws, uint8_t* q_row, uint8_t* s_row,
                           float* tensor_scale_row, uint8_t* q_t, uint8_t* s_t,
                           float* tensor_scale_t, int32_t* dev_status, hipStream_t stream);

/*
 * nvfp4_dequantize -- y = (e2m1(q) * s_f) * S for one stored orientation.
 * (Implied by the format, gist.science summary, Resumen técnico §2 "Formato
 * NVFP4".)
 *
 *   q          codes [rows][cols/2]; s scales [rows][cols/16] (BLOCK_1D) or
 *              [rows/16][cols/16] (BLOCK_2D, rows % 16 == 0).
 *   tensor_scale  1 float, S.
 *   rows, cols >= 0, cols % 16 == 0.
 *   out_dtype  NVFP4_F32, or NVFP4_BF16 (round to nearest even of the
 *              float32 value).
 *   y          [rows][ldy], ldy >= cols.
 */
int nvfp4_dequantize(const uint8_t* q, const uint8_t* s, const float* tensor_scale,
                     int64_t rows, int64_t cols, int block, int out_dtype, void* y, int64_t ldy,
                     hipStream_t stream);

/*
 * nvfp4_gemm -- C[M][N] = deq(A) . deq(B)^T with A [M][K] and B [N][K]
 * NVFP4 matrices blocked along K, float32 accumulation.
 * (gist.science summary, Resumen técnico §2 "Precisión Mixta Selectiva": the
 * linear-layer GEMMs run on NVFP4 operands.)
 *
 *   qa, sa, ta  A codes [M][K/2], scales [M][K/16] (a_block BLOCK_1D) or
 *               [M/16][K/16] (BLOCK_2D, M % 16 == 0), tensor scale (1 float).
 *   qb, sb, tb  B likewise with N.
 *   M, N >= 0; K >= 0, K % 16 == 0. K == 0 writes zeros.
 *   c           [M][ldc], ldc >= N; c_dtype NVFP4_BF16 (round to nearest
 *               even) or NVFP4_F32. C = (ta * tb) * sum_k a_k b_k, where
 *               a_k = e2m1 * s_f (exact), accumulated in float32. c needs
 *               only the alignment of its element type, and ldc any value
 *               >= N (the 16-byte rule does not apply to C).
 */
int nvfp4_gemm(const uint8_t* qa, const uint8_t* sa, const float* ta, int a_block,
               const uint8_t* qb, const uint8_t* sb, const float* tb, int b_block, int64_t M,
               int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, hipStream_t stream);

/* ---- Inspection hooks used by the parity tests ---- */

/*
 * nvfp4_philox_fill -- out[4g .. 4g+3] = Philox4x32-10(key = (seed lo,
 * seed hi), counter = (g lo, g hi, c2, c3)) for g in [0, n_groups): the same
 * device function the stochastic rounding uses. out holds 4 * n_groups
 * uint32. n_groups >= 0.
 */
int nvfp4_philox_fill(uint64_t seed, uint32_t c2, uint32_t c3, int64_t n_groups, uint32_t* out,
                      hipStream_t stream);

/*
 * nvfp4_rht_transform -- out[t][c] = the float32 transformed values that
 * nvfp4_rht_quantize quantizes (same device code), for inspection.
 * x as nvfp4_rht_quantize; out is dense [tokens][cols] float32.
 */
int nvfp4_rht_transform(const void* x, int x_dtype, int64_t tokens, int64_t cols, int64_t ldx,
                        uint64_t rht_seed, float* out, hipStream_t stream);

/*
 * nvfp4_rht_sign_mask -- host-only: bit i set means d_i = -1 for rht_seed.
 * Touches no device.
 */
uint32_t nvfp4_rht_sign_mask(uint64_t rht_seed);

/* Host-only: static description of a status code. */
const char* nvfp4_status_string(int status);

/* ------------------------------------------------------------------------
 * MXFP4, the comparison format (gist.science summary, Resumen técnico §2
 * "Formato NVFP4": blocks of 32 elements instead of 16; §1: coarser scale
 * factors). E2M1 codes packed as NVFP4's; one E8M0 scale byte b per 32
 * elements along a row, value 2^(b - 127), with b = max(floor(log2 amax) -
 * 2 + 127, 0) so the block amax maps into [4, 8); elements rounded to nearest
 * (ties to the even code, saturating at 6); no tensor scale. Non-finite
 * inputs give unspecified codes.
 * ------------------------------------------------------------------------ */

/*
 * mxfp4_quantize -- q [rows][cols/2] codes and s [rows][cols/32] E8M0 scale
 * bytes of x [rows][ldx] (NVFP4_F32 or NVFP4_BF16). rows, cols >= 0,
 * cols % 32 == 0, ldx >= cols, every row 16-byte aligned. One pass over x.
 */
int mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                   uint8_t* q, uint8_t* s, hipStream_t stream);

/*
 * mxfp4_dequantize -- y [rows][ldy] = e2m1(q) * 2^(b - 127), as float32 or
 * bf16 (exact in both). cols % 32 == 0, ldy >= cols.
 */
int mxfp4_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                     int out_dtype, void* y, int64_t ldy, hipStream_t stream);

/*
 * mxfp4_gemm -- C[M][N] = sum_k deq(A)[m][k] deq(B)[n][k] with A [M][K] and
 * B [N][K] in MXFP4 (codes qa/qb, scales sa/sb as mxfp4_quantize writes
 * them), float32 accumulation on gfx950's block-scaled FP4 MFMA, C in
 * c_dtype with leading dimension ldc >= N (element alignment suffices).
 * K % 128 == 0 (K == 0 writes zeros), M and N <= 2^30; operand pointers
 * 16-byte aligned.
 */
int mxfp4_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
               int64_t M, int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc,
               hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8, the baseline format (gist.science summary, Resumen técnico §1 and §4:
 * NVFP4 is measured against an FP8 run; deultimominuto.info, "Cómo funciona
 * NVFP4": E4M3 has 4 exponent and 3 mantissa bits). One E4M3FN byte per
 * element (bias 7, largest 448, no infinities) and one float32 decode scale
 * per tensor: S8 = fp32(amax / 448), replaced by 1 below 2^-100;
 * r = fp32(1 / S8); y = fp32(x * r); byte = E4M3FN nearest to |y|, ties to
 * the even mantissa, saturating at 448, with the sign bit of y (so -0.0
 * gives 0x80). Bytes 0x7F and 0xFF (NaN) are never produced. A non-finite
 * amax sets *dev_status = 1 (codes unspecified), as for nvfp4_quantize.
 * ------------------------------------------------------------------------ */

/*
 * fp8_quantize -- FP8 copies of x [rows][ldx] (NVFP4_F32 or NVFP4_BF16):
 *   outputs & NVFP4_OUT_ROW: q_row [rows][cols] (row-major bytes);
 *   outputs & NVFP4_OUT_COL: q_col [cols][rows], the same bytes transposed
 *     (the K-contiguous operand of the weight-gradient GEMM); needs
 *     rows % 16 == 0.
 * cols % 16 == 0, ldx >= cols, every row of x and both outputs 16-byte
 * aligned. amax_in / amax_ws / tensor_scale / dev_status as for
 * nvfp4_quantize (amax_ws: NVFP4_AMAX_WS_BYTES of device memory, amax_ws[0]
 * receives the amax); *tensor_scale receives S8. Two passes over x (amax,
 * then quantization) unless amax_in is given.
 */
int fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int outputs,
                 const float* amax_in, float* amax_ws, uint8_t* q_row, uint8_t* q_col,
                 float* tensor_scale, int32_t* dev_status, hipStream_t stream);

/*
 * fp8_dequantize -- y [rows][ldy] = fp32(e4m3(q) * S8) as float32, or its
 * round-to-nearest-even bf16, from q [rows][cols]. cols % 16 == 0,
 * ldy >= cols, 16-byte aligned rows.
 */
int fp8_dequantize(const uint8_t* q, const float* tensor_scale, int64_t rows, int64_t cols,
                   int out_dtype, void* y, int64_t ldy, hipStream_t stream);

/*
 * fp8_gemm -- C[M][N] = S8_a * S8_b * sum_k e4m3(qa[m][k]) e4m3(qb[n][k]),
 * both operands K-contiguous ([M][K] and [N][K] bytes, 16-byte aligned),
 * float32 accumulation on gfx950's FP8 MFMA (products exact), the scales
 * applied once in the epilogue; C in c_dtype with leading dimension
 * ldc >= N (element alignment suffices). ta / tb: device float32 decode
 * scales as fp8_quantize writes them. K % 64 == 0 (K == 0 writes zeros),
 * M and N <= 2^30.
 */
int fp8_gemm(const uint8_t* qa, const float* ta, const uint8_t* qb, const float* tb, int64_t M,
             int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Streaming references (measurement, not part of the format): plain
 * hand-written streams over device memory, 16-byte nontemporal loads, 8 per
 * thread in flight, timed beside the quantizers to show the read and copy
 * rates the memory system gives a kernel with no arithmetic.
 * ------------------------------------------------------------------------ */

/* Words of the checksum buffer of nvfp4_stream_read. */
#define NVFP4_STREAM_SINK_WORDS 1024

/*
 * nvfp4_stream_read -- reads bytes of src (bytes % 16 == 0, src 16-byte
 * aligned) and writes the XOR of the 32-bit words each workgroup read into
 * sink[0 .. g), g = min(NVFP4_STREAM_SINK_WORDS, ceil(bytes / 32768)); sink
 * holds NVFP4_STREAM_SINK_WORDS uint32. The XOR of sink[0 .. g) is the XOR of
 * all 32-bit words of src. bytes == 0 writes nothing.
 */
int nvfp4_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * nvfp4_stream_copy -- dst[0 .. bytes) = src[0 .. bytes) (bytes % 16 == 0,
 * both 16-byte aligned, not overlapping).
 */
int nvfp4_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
