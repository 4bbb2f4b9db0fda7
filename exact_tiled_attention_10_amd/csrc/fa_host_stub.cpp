// Stand-ins for the device side of libfa.so, for a host-only build of the C
// ABI layer (fa_api.cpp + fa_plan.cpp) under the address and undefined-
// behaviour sanitizers on a machine without a GPU.  Every launcher reports
// that it cannot run; the argument checks, size queries and plans are the
// real ones.  Never part of libfa.so.
#include "fa_internal.h"

namespace fa {

int device_cus() { return 256; }

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNotSupported;
}

hipError_t launch_fwd_bf16_kv(const void*, const void*, const void*, void*, float*, void*, int,
                              int, int, int, int, bool, float, const FwdPlan&, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_fwd_fp8(const void*, const void*, const void*, void*, float*, int, int, int,
                          bool, float, float, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, int, int, int,
                          bool, float, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_bwd_pre(const void*, const void*, const float*, void*, int, int, int,
                          hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_bwd_main(const void*, const void*, const void*, const void*, void*, void*,
                           void*, int, int, int, int, int, int, bool, float, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_zero_bf16(void*, void*, size_t, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_bwd_finalize(const void*, const void*, const void*, const void*, void*,
                               const void*, int, int, int, int, int, bool, float, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fa
