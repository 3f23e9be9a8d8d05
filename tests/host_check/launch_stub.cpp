// Stub launchers and runtime calls for the host-only sanitizer build of
// qmat_api.cpp: each launcher records that it was reached and succeeds.
#include <hip/hip_runtime.h>

#include "qmat_launch.hpp"

int g_launches = 0;

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = const_cast<void*>(symbol);
  return hipSuccess;
}

namespace qmat {
hipError_t launch_quantize(int, const float*, void*, int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_kv_write(int, const float*, const float*, void*, int64_t, int64_t,
                           hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gemv(int, const void*, const float*, float*, int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gemv_batch(int, const GemvJob*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gemm_small(int, const void*, const void*, float*, int64_t, int64_t, int64_t,
                             hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gemm(int, const void*, const void*, float*, int64_t, int64_t, int64_t, float*,
                       hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace qmat
