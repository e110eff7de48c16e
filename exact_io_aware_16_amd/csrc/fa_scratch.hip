// Device-resident scratch of the allocation-free backward (fa_bwd_noalloc).
//
// The backward needs two float32 per query row between its kernels
// (scale * D_i and L_i log2(e)).  fa_bwd takes that buffer from the caller;
// fa_bwd_noalloc uses this file-scope array instead, so the call allocates
// nothing.  Every GPU the library runs on holds its own copy of the array
// (it lives until the process ends); its address on the current device is
// looked up once per device with hipGetSymbolAddress and cached.  In host
// code the array's name is only a host-side handle: kernels receive the
// looked-up device address, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_launch.h"

namespace fa {

// 16 MiB: two floats for each of up to 2^21 query rows (B * H * N).
constexpr size_t kScratchFloats = size_t(1) << 22;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
float* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

size_t scratch_floats() { return kScratchFloats; }

hipError_t scratch_on_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace fa
