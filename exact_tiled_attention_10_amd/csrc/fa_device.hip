// Per-device state of the library: the compute-unit count the launch plans
// size their grids by, and the static scratch buffer of the no-allocation
// backward entry point (fa_bwd_noalloc).
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kMaxDevices = 64;

// The scratch of fa_bwd_noalloc: device memory the library owns, one copy per
// GPU (each device that loads the library holds it until the process ends).
// In host code `scratch` names a host-side stand-in, not device memory: the
// only way host code reaches the array is through the per-device address
// static_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mu;
int g_cus[kMaxDevices];
void* g_scratch[kMaxDevices];

}  // namespace

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev] == nullptr) {
    // once per device, with that device current: its own copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace fa
