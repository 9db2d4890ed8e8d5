// Internal interface between the C ABI (argument checking, abi.cpp) and the
// kernel launchers (*.hip). Arguments reaching a launcher are already valid.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace nvfp4 {

struct QuantizeLaunch {
  const void* x;
  bool x_bf16;
  int64_t rows, cols, ldx;  // for the RHT path rows are tokens
  bool block_2d;
  bool rht;
  bool sr;
  uint64_t seed;
  uint32_t offset;
  uint32_t sign_mask;  // RHT signs (bit i: d_i = -1)
  int outputs;         // 1 = row copy, 2 = column copy (RHT path: column copy)
  bool row_too;        // RHT path: also the 1x16 row copy (round to nearest) with its
                       // own tensor scale; amax_in then holds 2 floats (row, Hadamard)
  const float* amax_in;
  float* amax_ws;
  uint8_t *q_row, *s_row, *q_col, *s_col;
  float* tensor_scale;    // the row copy's (or the only) tensor scale
  float* tensor_scale_t;  // with row_too: the Hadamard column copy's tensor scale
  int32_t* dev_status;
};

// Each returns 0, or -1 when a launch failed.
int launch_quantize(const QuantizeLaunch& q, hipStream_t stream);

// Floats of amax_ws (from its start) that launch_quantize(q) writes or reads.
int64_t quantize_workspace_floats(const QuantizeLaunch& q);

// The library's own amax workspace on the current device (a static device
// array; see noalloc.hip), or NULL when its address cannot be found.
// *floats receives its size in floats.
float* static_amax_workspace(int64_t* floats);

int launch_dequantize(const uint8_t* q, const uint8_t* s, const float* tensor_scale, int64_t rows,
                      int64_t cols, bool block_2d, bool out_bf16, void* y, int64_t ldy,
                      hipStream_t stream);

struct GemmLaunch {
  const uint8_t *qa, *sa;
  const float* ta;
  bool a_2d;
  const uint8_t *qb, *sb;
  const float* tb;
  bool b_2d;
  int64_t M, N, K;
  void* c;
  bool c_bf16;
  int64_t ldc;
};

int launch_gemm(const GemmLaunch& g, hipStream_t stream);

// Compute units of the current device (queried once per device; 0 if the
// query fails).
int device_compute_units();

// MXFP4 (comparison format).
int launch_mx_quantize(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                       uint8_t* q, uint8_t* s, hipStream_t stream);
int launch_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                         bool out_bf16, void* y, int64_t ldy, hipStream_t stream);
int launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                   int64_t M, int64_t N, int64_t K, void* c, bool c_bf16, int64_t ldc,
                   hipStream_t stream);

// Per-workgroup partial maxima of |x| (no transform) into amax_ws from
// kPartialsOffset on; returns their count (> 0), or -1 on a launch error.
// rows and cols are > 0.
int launch_tensor_amax(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                       float* amax_ws, hipStream_t stream);

// FP8 (E4M3, one scale per tensor; the baseline format).
struct Fp8QuantizeLaunch {
  const void* x;
  bool x_bf16;
  int64_t rows, cols, ldx;
  int outputs;  // bit 0: row copy [rows][cols], bit 1: column copy [cols][rows]
  const float* amax_in;
  float* amax_ws;
  uint8_t *q_row, *q_col;
  float* tensor_scale;
  int32_t* dev_status;
};
int launch_fp8_quantize(const Fp8QuantizeLaunch& q, hipStream_t stream);
int launch_fp8_dequantize(const uint8_t* q, const float* tensor_scale, int64_t rows, int64_t cols,
                          bool out_bf16, void* y, int64_t ldy, hipStream_t stream);
int launch_fp8_gemm(const uint8_t* qa, const float* ta, const uint8_t* qb, const float* tb,
                    int64_t M, int64_t N, int64_t K, void* c, bool c_bf16, int64_t ldc,
                    hipStream_t stream);

int launch_philox_fill(uint64_t seed, uint32_t c2, uint32_t c3, int64_t n_groups, uint32_t* out,
                       hipStream_t stream);

int launch_rht_transform(const void* x, bool x_bf16, int64_t tokens, int64_t cols, int64_t ldx,
                         uint32_t sign_mask, float* out, hipStream_t stream);

// Streaming references (stream.hip). launch_stream_read returns the number
// of checksum words written (workgroups), or -1 on a launch error.
int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
int launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

// Host-side Philox4x32-10 (same definition as the device function).
void philox4x32_10_host(uint32_t k0, uint32_t k1, const uint32_t ctr[4], uint32_t out[4]);

}  // namespace nvfp4
