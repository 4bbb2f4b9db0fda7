// Per-device state of the library: the compute-unit count the launch plans
// size their grids by.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
int g_cus[kMaxDevices];

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

}  // namespace fa
