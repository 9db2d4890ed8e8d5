// A fixed amax workspace inside the library, for callers that cannot
// allocate device memory (code under stream capture, serving loops, hosts
// that forbid allocation): nvfp4_quantize_noalloc passes it where
// nvfp4_quantize takes the caller's amax_ws.
//
// The workspace is a static device array, so each GPU the library runs on
// holds one copy of it, at its own address, until the process ends. Host
// code must not pass the array's name to a kernel (on the host it names a
// stand-in, not device memory): its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
//
// Every call on one GPU shares that GPU's copy and leaves its partial maxima
// behind. Nothing in it needs an initial value (each call writes the
// partial maxima it reads, in stream order), but calls whose work overlaps
// on one GPU (different streams, or several host threads without ordering)
// race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "nvfp4.h"

namespace nvfp4 {
namespace {

constexpr int64_t kScratchFloats = NVFP4_AMAX_WS_BYTES / 4;  // 16 KiB per device

static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices];  // device address of scratch, per device (NULL: not yet looked up)

}  // namespace

float* static_amax_workspace(int64_t* floats) {
  *floats = kScratchFloats;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  return g_scratch_ptr[dev];
}

}  // namespace nvfp4
