// Stand-ins for the kernel launchers of libfa.so, linked with the C ABI
// (fa_api.cpp) into a host-only program built under AddressSanitizer and
// UndefinedBehaviorSanitizer.  No GPU is involved: every launcher counts its
// call and launches nothing, so a call that gets past the argument checks
// returns FA_ERR_HIP.  Test infrastructure only.
#include "fa_launch.h"

int g_launches = 0;

namespace fa {

hipError_t launch_fwd_bf16(const void*, const void*, const void*, float*, float*, int, int, int, int, int, int, int,
                           float*, float, const Dropout*, const Seqs*, hipStream_t, const Strides*) {
  ++g_launches;
  return hipErrorNotSupported;
}

hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, int, int, int, float, int,
                          hipStream_t) {
  ++g_launches;
  return hipErrorNotSupported;
}

hipError_t launch_bwd_dq_bf16(const void*, const void*, const void*, const void*, const float*, const float*, float*,
                              int, int, int, int, float, int, const Dropout*, const Seqs*, hipStream_t,
                              const Strides*) {
  ++g_launches;
  return hipErrorNotSupported;
}

hipError_t launch_bwd_prep(const void*, const float*, const float*, float*, int, int, int, float, hipStream_t) {
  ++g_launches;
  return hipErrorNotSupported;
}

hipError_t launch_bwd_dkdv(const void*, const void*, const void*, const void*, const float*, float*, float*, int, int,
                           int, int, float, int, const Dropout*, const Seqs*, hipStream_t, const Strides*) {
  ++g_launches;
  return hipErrorNotSupported;
}

hipError_t launch_bwd_bf16(const void*, const void*, const void*, const float*, const float*, const void*, float*,
                           float*, float*, float*, int, int, int, int, float, int, const Dropout*, const Seqs*,
                           hipStream_t, const Strides*) {
  ++g_launches;
  return hipErrorNotSupported;
}

// The number of key ranges: the request itself (the library's own choice
// depends on the kernels' tiling, which this program does not build).
int fwd_splitkv_resolve(int, int, int, int, int, int n_splits) { return n_splits < 1 ? 4 : n_splits; }

// The documented capacity of the allocation-free backward: 2^21 query rows,
// two floats each.
size_t scratch_floats() { return size_t(1) << 22; }

hipError_t scratch_on_current_device(float** out) {
  ++g_launches;
  *out = nullptr;
  return hipErrorNotSupported;
}

}  // namespace fa
