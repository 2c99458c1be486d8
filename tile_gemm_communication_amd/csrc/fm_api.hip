// fm_api.cpp -- version, status strings and cached device properties.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fm_common.hpp"

namespace fm {

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace fm

extern "C" int fm_version(void) { return 100; }

extern "C" const char* fm_status_str(fm_status_t s) {
  switch (s) {
    case FM_OK: return "FM_OK";
    case FM_ERR_INVALID_ARG: return "FM_ERR_INVALID_ARG";
    case FM_ERR_UNSUPPORTED: return "FM_ERR_UNSUPPORTED";
    case FM_ERR_HIP: return "FM_ERR_HIP";
    case FM_ERR_TIMEOUT: return "FM_ERR_TIMEOUT";
  }
  return "FM_ERR_UNKNOWN";
}
