// C ABI of the NVFP4 library: host-side argument checking, then the kernel
// launchers. Every argument error is found here, before any HIP call, so the
// error paths need no GPU. The library keeps no state and never allocates.
#include <stdint.h>

#include "../../include/nvfp4.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int d) { return d == NVFP4_F32 || d == NVFP4_BF16; }

int64_t dtype_size(int d) { return d == NVFP4_F32 ? 4 : 2; }

// Checks an input matrix [rows][ldx] of dtype d with 16-aligned rows.
int check_input(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx) {
  if (!valid_dtype(dtype)) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || (cols % 16) != 0 || ldx < cols) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (x == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(x) || ((ldx * dtype_size(dtype)) % 16) != 0) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// Tensors larger than this are split by the caller (the kernels index tiles
// with 32-bit grid coordinates).
constexpr int64_t kMaxElements = int64_t(1) << 40;
// Rows of either operand of the MXFP4 and FP8 GEMMs (their loads index rows
// with 32-bit integers).
constexpr int64_t kMaxBlockGemmRows = int64_t(1) << 30;

// The argument checks of nvfp4_quantize; fills q when they pass. With
// ws_required, amax_ws must be given when amax_in is not (the no-allocation
// variant brings its own workspace and passes amax_ws = NULL).
int check_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int block,
                   int rounding, uint64_t seed, uint32_t offset, int outputs,
                   const float* amax_in, float* amax_ws, bool ws_required, uint8_t* q_row,
                   uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* tensor_scale,
                   int32_t* dev_status, nvfp4::QuantizeLaunch& q) {
  if (block != NVFP4_BLOCK_1D && block != NVFP4_BLOCK_2D) return NVFP4_ERR_ENUM;
  if (rounding != NVFP4_ROUND_RN && rounding != NVFP4_ROUND_SR) return NVFP4_ERR_ENUM;
  if (outputs < 1 || outputs > 3) return NVFP4_ERR_ENUM;
  if (block == NVFP4_BLOCK_2D && rounding == NVFP4_ROUND_SR) return NVFP4_ERR_ENUM;
  int rc = check_input(x, x_dtype, rows, cols, ldx);
  if (rc != NVFP4_OK) return rc;
  const bool out_row = (outputs & NVFP4_OUT_ROW) != 0, out_col = (outputs & NVFP4_OUT_COL) != 0;
  if ((out_col || block == NVFP4_BLOCK_2D) && (rows % 16) != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > kMaxElements / rows) return NVFP4_ERR_SHAPE;
  if (tensor_scale == nullptr) return NVFP4_ERR_NULL;
  if (ws_required && amax_in == nullptr && amax_ws == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(tensor_scale) || (amax_in && !aligned16(amax_in)) ||
      (amax_ws && !aligned16(amax_ws)) || (dev_status && !aligned16(dev_status)))
    return NVFP4_ERR_ALIGN;
  const bool empty = rows == 0 || cols == 0;
  if (!empty) {
    if (out_row && (q_row == nullptr || s_row == nullptr)) return NVFP4_ERR_NULL;
    if (out_col && (q_col == nullptr || s_col == nullptr)) return NVFP4_ERR_NULL;
    if ((out_row && (!aligned16(q_row) || !aligned16(s_row))) ||
        (out_col && (!aligned16(q_col) || !aligned16(s_col))))
      return NVFP4_ERR_ALIGN;
  }
  q.x = x;
  q.x_bf16 = x_dtype == NVFP4_BF16;
  q.rows = rows;
  q.cols = cols;
  q.ldx = ldx;
  q.block_2d = block == NVFP4_BLOCK_2D;
  q.rht = false;
  q.sr = rounding == NVFP4_ROUND_SR;
  q.seed = seed;
  q.offset = offset;
  q.sign_mask = 0;
  q.outputs = outputs;
  q.amax_in = amax_in;
  q.amax_ws = amax_ws;
  q.q_row = q_row;
  q.s_row = s_row;
  q.q_col = q_col;
  q.s_col = s_col;
  q.tensor_scale = tensor_scale;
  q.dev_status = dev_status;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

uint32_t nvfp4_rht_sign_mask(uint64_t rht_seed) {
  const uint32_t ctr[4] = {0u, 0u, 0u, 2u};
  uint32_t out[4];
  nvfp4::philox4x32_10_host(static_cast<uint32_t>(rht_seed), static_cast<uint32_t>(rht_seed >> 32),
                            ctr, out);
  return out[0] & 0xFFFFu;
}

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid size or leading dimension";
    case NVFP4_ERR_ENUM: return "unknown enum value or unsupported combination";
    case NVFP4_ERR_ALIGN: return "pointer or row not 16-byte aligned";
    case NVFP4_ERR_HIP: return "kernel launch failed";
    default: return "unknown status";
  }
}

int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int block,
                   int rounding, uint64_t seed, uint32_t offset, int outputs, const float* amax_in,
                   float* amax_ws, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                   float* tensor_scale, int32_t* dev_status, hipStream_t stream) {
  nvfp4::QuantizeLaunch q{};
  int rc = check_quantize(x, x_dtype, rows, cols, ldx, block, rounding, seed, offset, outputs,
                          amax_in, amax_ws, true, q_row, s_row, q_col, s_col, tensor_scale,
                          dev_status, q);
  if (rc != NVFP4_OK) return rc;
  return nvfp4::launch_quantize(q, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                           int block, int rounding, uint64_t seed, uint32_t offset, int outputs,
                           const float* amax_in, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                           uint8_t* s_col, float* tensor_scale, int32_t* dev_status,
                           hipStream_t stream) {
  nvfp4::QuantizeLaunch q{};
  int rc = check_quantize(x, x_dtype, rows, cols, ldx, block, rounding, seed, offset, outputs,
                          amax_in, nullptr, false, q_row, s_row, q_col, s_col, tensor_scale,
                          dev_status, q);
  if (rc != NVFP4_OK) return rc;
  if (amax_in == nullptr) {
    int64_t floats = 0;
    float* ws = nvfp4::static_amax_workspace(&floats);
    if (ws == nullptr) return NVFP4_ERR_HIP;
    q.amax_ws = ws;
    if (nvfp4::quantize_workspace_floats(q) > floats) return NVFP4_ERR_SHAPE;
  }
  return nvfp4::launch_quantize(q, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_rht_quantize(const void* x, int x_dtype, int64_t tokens, int64_t cols, int64_t ldx,
                       uint64_t rht_seed, int rounding, uint64_t seed, uint32_t offset,
                       const float* amax_in, float* amax_ws, uint8_t* q_t, uint8_t* s_t,
                       float* tensor_scale, int32_t* dev_status, hipStream_t stream) {
  if (rounding != NVFP4_ROUND_RN && rounding != NVFP4_ROUND_SR) return NVFP4_ERR_ENUM;
  int rc = check_input(x, x_dtype, tokens, cols, ldx);
  if (rc != NVFP4_OK) return rc;
  if ((tokens % 16) != 0) return NVFP4_ERR_SHAPE;
  if (tokens > 0 && cols > kMaxElements / tokens) return NVFP4_ERR_SHAPE;
  if (tensor_scale == nullptr) return NVFP4_ERR_NULL;
  if (amax_in == nullptr && amax_ws == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(tensor_scale) || (amax_in && !aligned16(amax_in)) ||
      (amax_ws && !aligned16(amax_ws)) || (dev_status && !aligned16(dev_status)))
    return NVFP4_ERR_ALIGN;
  const bool empty = tokens == 0 || cols == 0;
  if (!empty) {
    if (q_t == nullptr || s_t == nullptr) return NVFP4_ERR_NULL;
    if (!aligned16(q_t) || !aligned16(s_t)) return NVFP4_ERR_ALIGN;
  }
  nvfp4::QuantizeLaunch q{};
  q.x = x;
  q.x_bf16 = x_dtype == NVFP4_BF16;
  q.rows = tokens;
  q.cols = cols;
  q.ldx = ldx;
  q.block_2d = false;
  q.rht = true;
  q.sr = rounding == NVFP4_ROUND_SR;
  q.seed = seed;
  q.offset = offset;
  q.sign_mask = nvfp4_rht_sign_mask(rht_seed);
  q.outputs = NVFP4_OUT_COL;
  q.amax_in = amax_in;
  q.amax_ws = amax_ws;
  q.q_col = q_t;
  q.s_col = s_t;
  q.tensor_scale = tensor_scale;
  q.dev_status = dev_status;
  return nvfp4::launch_quantize(q, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_quantize_row_rht(const void* x, int x_dtype, int64_t tokens, int64_t cols, int64_t ldx,
                           uint64_t rht_seed, int rounding_t, uint64_t seed, uint32_t offset,
                           const float* amax_in, float* amax_ws, uint8_t* q_row, uint8_t* s_row,
                           float* tensor_scale_row, uint8_t* q_t, uint8_t* s_t,
                           float* tensor_scale_t, int32_t* dev_status, hipStream_t stream) {
  if (rounding_t != NVFP4_ROUND_RN && rounding_t != NVFP4_ROUND_SR) return NVFP4_ERR_ENUM;
  int rc = check_input(x, x_dtype, tokens, cols, ldx);
  if (rc != NVFP4_OK) return rc;
  if ((tokens % 16) != 0) return NVFP4_ERR_SHAPE;
  if (tokens > 0 && cols > kMaxElements / tokens) return NVFP4_ERR_SHAPE;
  if (tensor_scale_row == nullptr || tensor_scale_t == nullptr) return NVFP4_ERR_NULL;
  if (amax_in == nullptr && amax_ws == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(tensor_scale_row) || !aligned16(tensor_scale_t) ||
      (amax_in && !aligned16(amax_in)) || (amax_ws && !aligned16(amax_ws)) ||
      (dev_status && !aligned16(dev_status)))
    return NVFP4_ERR_ALIGN;
  const bool empty = tokens == 0 || cols == 0;
  if (!empty) {
    if (q_row == nullptr || s_row == nullptr || q_t == nullptr || s_t == nullptr)
      return NVFP4_ERR_NULL;
    if (!aligned16(q_row) || !aligned16(s_row) || !aligned16(q_t) || !aligned16(s_t))
      return NVFP4_ERR_ALIGN;
  }
  nvfp4::QuantizeLaunch q{};
  q.x = x;
  q.x_bf16 = x_dtype == NVFP4_BF16;
  q.rows = tokens;
  q.cols = cols;
  q.ldx = ldx;
  q.block_2d = false;
  q.rht = true;
  q.row_too = true;
  q.sr = rounding_t == NVFP4_ROUND_SR;
  q.seed = seed;
  q.offset = offset;
  q.sign_mask = nvfp4_rht_sign_mask(rht_seed);
  q.outputs = NVFP4_OUT_ROW | NVFP4_OUT_COL;
  q.amax_in = amax_in;
  q.amax_ws = amax_ws;
  q.q_row = q_row;
  q.s_row = s_row;
  q.q_col = q_t;
  q.s_col = s_t;
  q.tensor_scale = tensor_scale_row;
  q.tensor_scale_t = tensor_scale_t;
  q.dev_status = dev_status;
  return nvfp4::launch_quantize(q, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_dequantize(const uint8_t* q, const uint8_t* s, const float* tensor_scale, int64_t rows,
                     int64_t cols, int block, int out_dtype, void* y, int64_t ldy,
                     hipStream_t stream) {
  if (block != NVFP4_BLOCK_1D && block != NVFP4_BLOCK_2D) return NVFP4_ERR_ENUM;
  if (!valid_dtype(out_dtype)) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || (cols % 16) != 0 || ldy < cols) return NVFP4_ERR_SHAPE;
  if (block == NVFP4_BLOCK_2D && (rows % 16) != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (rows > kMaxElements / cols) return NVFP4_ERR_SHAPE;
  if (q == nullptr || s == nullptr || tensor_scale == nullptr || y == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(q) || !aligned16(s) || !aligned16(tensor_scale) || !aligned16(y) ||
      ((ldy * dtype_size(out_dtype)) % 16) != 0)
    return NVFP4_ERR_ALIGN;
  return nvfp4::launch_dequantize(q, s, tensor_scale, rows, cols, block == NVFP4_BLOCK_2D,
                                  out_dtype == NVFP4_BF16, y, ldy, stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int nvfp4_gemm(const uint8_t* qa, const uint8_t* sa, const float* ta, int a_block,
               const uint8_t* qb, const uint8_t* sb, const float* tb, int b_block, int64_t M,
               int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, hipStream_t stream) {
  if ((a_block != NVFP4_BLOCK_1D && a_block != NVFP4_BLOCK_2D) ||
      (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D) || !valid_dtype(c_dtype))
    return NVFP4_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || (K % 16) != 0 || ldc < N) return NVFP4_ERR_SHAPE;
  if ((a_block == NVFP4_BLOCK_2D && (M % 16) != 0) || (b_block == NVFP4_BLOCK_2D && (N % 16) != 0))
    return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (M > kMaxElements / N || (K > 0 && (M > kMaxElements / K || N > kMaxElements / K)))
    return NVFP4_ERR_SHAPE;
  if (c == nullptr || ta == nullptr || tb == nullptr) return NVFP4_ERR_NULL;
  if (K > 0 && (qa == nullptr || sa == nullptr || qb == nullptr || sb == nullptr))
    return NVFP4_ERR_NULL;
  // C is written element by element: natural alignment of its type suffices
  if ((reinterpret_cast<uintptr_t>(c) % static_cast<uintptr_t>(dtype_size(c_dtype))) != 0 ||
      !aligned16(ta) || !aligned16(tb))
    return NVFP4_ERR_ALIGN;
  if (K > 0 && (!aligned16(qa) || !aligned16(sa) || !aligned16(qb) || !aligned16(sb)))
    return NVFP4_ERR_ALIGN;
  nvfp4::GemmLaunch g{};
  g.qa = qa;
  g.sa = sa;
  g.ta = ta;
  g.a_2d = a_block == NVFP4_BLOCK_2D;
  g.qb = qb;
  g.sb = sb;
  g.tb = tb;
  g.b_2d = b_block == NVFP4_BLOCK_2D;
  g.M = M;
  g.N = N;
  g.K = K;
  g.c = c;
  g.c_bf16 = c_dtype == NVFP4_BF16;
  g.ldc = ldc;
  return nvfp4::launch_gemm(g, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_philox_fill(uint64_t seed, uint32_t c2, uint32_t c3, int64_t n_groups, uint32_t* out,
                      hipStream_t stream) {
  if (n_groups < 0 || n_groups > (int64_t(1) << 36)) return NVFP4_ERR_SHAPE;
  if (n_groups == 0) return NVFP4_OK;
  if (out == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(out)) return NVFP4_ERR_ALIGN;
  return nvfp4::launch_philox_fill(seed, c2, c3, n_groups, out, stream) == 0 ? NVFP4_OK
                                                                             : NVFP4_ERR_HIP;
}

int nvfp4_rht_transform(const void* x, int x_dtype, int64_t tokens, int64_t cols, int64_t ldx,
                        uint64_t rht_seed, float* out, hipStream_t stream) {
  int rc = check_input(x, x_dtype, tokens, cols, ldx);
  if (rc != NVFP4_OK) return rc;
  if ((tokens % 16) != 0) return NVFP4_ERR_SHAPE;
  if (tokens == 0 || cols == 0) return NVFP4_OK;
  if (tokens > kMaxElements / cols) return NVFP4_ERR_SHAPE;
  if (out == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(out)) return NVFP4_ERR_ALIGN;
  return nvfp4::launch_rht_transform(x, x_dtype == NVFP4_BF16, tokens, cols, ldx,
                                     nvfp4_rht_sign_mask(rht_seed), out, stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                   uint8_t* q, uint8_t* s, hipStream_t stream) {
  int rc = check_input(x, x_dtype, rows, cols, ldx);
  if (rc != NVFP4_OK) return rc;
  if ((cols % 32) != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (rows > kMaxElements / cols) return NVFP4_ERR_SHAPE;
  if (q == nullptr || s == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(q) || !aligned16(s)) return NVFP4_ERR_ALIGN;
  return nvfp4::launch_mx_quantize(x, x_dtype == NVFP4_BF16, rows, cols, ldx, q, s, stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int mxfp4_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                     int out_dtype, void* y, int64_t ldy, hipStream_t stream) {
  if (!valid_dtype(out_dtype)) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || (cols % 32) != 0 || ldy < cols) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (rows > kMaxElements / cols) return NVFP4_ERR_SHAPE;
  if (q == nullptr || s == nullptr || y == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(q) || !aligned16(s) || !aligned16(y) || ((ldy * dtype_size(out_dtype)) % 16) != 0)
    return NVFP4_ERR_ALIGN;
  return nvfp4::launch_mx_dequantize(q, s, rows, cols, out_dtype == NVFP4_BF16, y, ldy, stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int mxfp4_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
               int64_t M, int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc,
               hipStream_t stream) {
  if (!valid_dtype(c_dtype)) return NVFP4_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || (K % 128) != 0 || ldc < N) return NVFP4_ERR_SHAPE;
  if (M > kMaxBlockGemmRows || N > kMaxBlockGemmRows) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (M > kMaxElements / N || (K > 0 && (M > kMaxElements / K || N > kMaxElements / K)))
    return NVFP4_ERR_SHAPE;
  if (c == nullptr) return NVFP4_ERR_NULL;
  if (K > 0 && (qa == nullptr || sa == nullptr || qb == nullptr || sb == nullptr))
    return NVFP4_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(c) % static_cast<uintptr_t>(dtype_size(c_dtype))) != 0)
    return NVFP4_ERR_ALIGN;
  if (K > 0 && (!aligned16(qa) || !aligned16(sa) || !aligned16(qb) || !aligned16(sb)))
    return NVFP4_ERR_ALIGN;
  return nvfp4::launch_mx_gemm(qa, sa, qb, sb, M, N, K, c, c_dtype == NVFP4_BF16, ldc, stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int outputs,
                 const float* amax_in, float* amax_ws, uint8_t* q_row, uint8_t* q_col,
                 float* tensor_scale, int32_t* dev_status, hipStream_t stream) {
  if (outputs < 1 || outputs > 3) return NVFP4_ERR_ENUM;
  int rc = check_input(x, x_dtype, rows, cols, ldx);
  if (rc != NVFP4_OK) return rc;
  const bool out_row = (outputs & NVFP4_OUT_ROW) != 0, out_col = (outputs & NVFP4_OUT_COL) != 0;
  if (out_col && (rows % 16) != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > kMaxElements / rows) return NVFP4_ERR_SHAPE;
  if (tensor_scale == nullptr) return NVFP4_ERR_NULL;
  if (amax_in == nullptr && amax_ws == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(tensor_scale) || (amax_in && !aligned16(amax_in)) ||
      (amax_ws && !aligned16(amax_ws)) || (dev_status && !aligned16(dev_status)))
    return NVFP4_ERR_ALIGN;
  if (rows > 0 && cols > 0) {
    if ((out_row && q_row == nullptr) || (out_col && q_col == nullptr)) return NVFP4_ERR_NULL;
    if ((out_row && !aligned16(q_row)) || (out_col && !aligned16(q_col))) return NVFP4_ERR_ALIGN;
  }
  nvfp4::Fp8QuantizeLaunch q;
  q.x = x;
  q.x_bf16 = x_dtype == NVFP4_BF16;
  q.rows = rows;
  q.cols = cols;
  q.ldx = ldx;
  q.outputs = outputs;
  q.amax_in = amax_in;
  q.amax_ws = amax_ws;
  q.q_row = q_row;
  q.q_col = q_col;
  q.tensor_scale = tensor_scale;
  q.dev_status = dev_status;
  return nvfp4::launch_fp8_quantize(q, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int fp8_dequantize(const uint8_t* q, const float* tensor_scale, int64_t rows, int64_t cols,
                   int out_dtype, void* y, int64_t ldy, hipStream_t stream) {
  if (!valid_dtype(out_dtype)) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || (cols % 16) != 0 || ldy < cols) return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (rows > kMaxElements / cols) return NVFP4_ERR_SHAPE;
  if (q == nullptr || tensor_scale == nullptr || y == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(q) || !aligned16(y) || ((ldy * dtype_size(out_dtype)) % 16) != 0)
    return NVFP4_ERR_ALIGN;
  return nvfp4::launch_fp8_dequantize(q, tensor_scale, rows, cols, out_dtype == NVFP4_BF16, y, ldy,
                                      stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int fp8_gemm(const uint8_t* qa, const float* ta, const uint8_t* qb, const float* tb, int64_t M,
             int64_t N, int64_t K, void* c, int c_dtype, int64_t ldc, hipStream_t stream) {
  if (!valid_dtype(c_dtype)) return NVFP4_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || (K % 64) != 0 || ldc < N) return NVFP4_ERR_SHAPE;
  if (M > kMaxBlockGemmRows || N > kMaxBlockGemmRows) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (M > kMaxElements / N || (K > 0 && (M > kMaxElements / K || N > kMaxElements / K)))
    return NVFP4_ERR_SHAPE;
  if (c == nullptr) return NVFP4_ERR_NULL;
  if (K > 0 && (qa == nullptr || qb == nullptr || ta == nullptr || tb == nullptr))
    return NVFP4_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(c) % static_cast<uintptr_t>(dtype_size(c_dtype))) != 0)
    return NVFP4_ERR_ALIGN;
  if (K > 0 && (!aligned16(qa) || !aligned16(qb))) return NVFP4_ERR_ALIGN;
  return nvfp4::launch_fp8_gemm(qa, ta, qb, tb, M, N, K, c, c_dtype == NVFP4_BF16, ldc, stream) == 0
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

int nvfp4_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes < 0 || (bytes % 16) != 0) return NVFP4_ERR_SHAPE;
  if (bytes == 0) return NVFP4_OK;
  if (src == nullptr || sink == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return NVFP4_ERR_ALIGN;
  return nvfp4::launch_stream_read(src, bytes, sink, stream) > 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (bytes < 0 || (bytes % 16) != 0) return NVFP4_ERR_SHAPE;
  if (bytes == 0) return NVFP4_OK;
  if (src == nullptr || dst == nullptr) return NVFP4_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return NVFP4_ERR_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + static_cast<uintptr_t>(bytes) && b < a + static_cast<uintptr_t>(bytes))
    return NVFP4_ERR_SHAPE;  // overlapping buffers
  return nvfp4::launch_stream_copy(src, dst, bytes, stream) == 0 ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"

namespace nvfp4 {

// Philox4x32-10 (Salmon et al., SC'11), host copy of the device function
// used for the Hadamard sign vector.
void philox4x32_10_host(uint32_t k0, uint32_t k1, const uint32_t ctr[4], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * x2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ x1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ x3 ^ k1;
    x1 = static_cast<uint32_t>(p1);
    x3 = static_cast<uint32_t>(p0);
    x0 = n0;
    x2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

}  // namespace nvfp4
