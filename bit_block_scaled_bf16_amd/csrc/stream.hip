// Streaming reference kernels: the read and copy rates a plain, hand-written
// stream reaches on this GPU, measured beside the quantizers so that their
// fractions of the 8 TB/s peak can be read against what the memory system
// delivers to a kernel with no arithmetic at all.
//
// Both use 16-byte nontemporal loads, 8 in flight per thread, and a
// grid-stride loop. The read kernel folds what it reads into one XOR
// checksum per workgroup (a real output, so no load can be dropped).
#include <hip/hip_runtime.h>

#include "launch.h"
#include "nvfp4.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int64_t kCopyGroups = 4096;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                               int64_t n, uint32_t* __restrict__ sink) {
  __shared__ uint32_t lds[kThreads / 64];
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n;
       base += stride) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      r[u] = i < n ? load_nt(src + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off, 64));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = lds[0] ^ lds[1] ^ lds[2] ^ lds[3];
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n;
       base += stride) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n) r[u] = load_nt(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n) dst[i] = r[u];
    }
  }
}

}  // namespace

int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n = bytes / 16;
  const int64_t per_group = static_cast<int64_t>(kThreads) * kUnroll;
  int64_t groups = (n + per_group - 1) / per_group;
  if (groups > NVFP4_STREAM_SINK_WORDS) groups = NVFP4_STREAM_SINK_WORDS;
  stream_read_kernel<<<static_cast<unsigned>(groups), kThreads, 0, stream>>>(
      static_cast<const uint4*>(src), n, sink);
  return hipGetLastError() == hipSuccess ? static_cast<int>(groups) : -1;
}

int launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16;
  const int64_t per_group = static_cast<int64_t>(kThreads) * kUnroll;
  int64_t groups = (n + per_group - 1) / per_group;
  if (groups > kCopyGroups) groups = kCopyGroups;
  stream_copy_kernel<<<static_cast<unsigned>(groups), kThreads, 0, stream>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nvfp4
