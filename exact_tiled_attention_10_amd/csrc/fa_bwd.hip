#include "fa_common.h"
#include "fa_internal.h"
namespace fa {
size_t bwd_workspace_bytes(int BH, int N, int d) {
  size_t dbytes = ((size_t)BH * N * 4 + 255) / 256 * 256;
  return dbytes + (size_t)BH * N * d * 4;
}
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const void*,
                           const float*, void*, void*, void*, void*, int, int, int, bool, float,
                           hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace fa
