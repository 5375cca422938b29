// Library-wide entry points: error messages, version, device properties.
#include <hip/hip_runtime.h>

#include <atomic>

#include "device.hpp"

namespace pagedkv {

std::string& last_error() {
  static thread_local std::string msg;
  return msg;
}

int device_cus(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not yet queried
  int dev = 0;
  PA_HIP_CHECK(hipGetDevice(&dev));
  if (dev >= 0 && dev < kMaxDevices) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return PA_OK;
    }
  }
  int c = 0;
  PA_HIP_CHECK(hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev));
  if (c <= 0) return fail(PA_EHIP, "device %d reports %d compute units", dev, c);
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return PA_OK;
}

}  // namespace pagedkv

extern "C" const char* pa_last_error(void) { return pagedkv::last_error().c_str(); }

extern "C" int pa_version(void) { return 100; }
