// Library-wide entry points: error messages, version, device properties.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>

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

namespace {
std::atomic<int> g_debug{-1};  // -1: not yet read from the environment
}

bool debug_checks() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("PA_DEBUG_CHECKS");
    v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, v, std::memory_order_relaxed);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v == 1;
}

int check_slots(const int64_t* slots, int32_t n, int64_t num_slots, hipStream_t stream) {
  std::vector<int64_t> h;
  int rc = fetch(h, slots, (size_t)n, stream);
  if (rc != PA_OK) return rc;
  std::vector<std::pair<int64_t, int32_t>> in;
  for (int32_t i = 0; i < n; ++i)
    if (h[i] >= 0 && h[i] < num_slots) in.emplace_back(h[i], i);
  std::sort(in.begin(), in.end());
  for (size_t k = 1; k < in.size(); ++k)
    if (in[k].first == in[k - 1].first)
      return fail(PA_EINVAL, "debug check: slot %lld given to tokens %d and %d",
                  (long long)in[k].first, in[k - 1].second, in[k].second);
  return PA_OK;
}

int check_pairs(const int32_t* pairs, int32_t n, int32_t num_blocks, hipStream_t stream) {
  std::vector<int32_t> h;
  int rc = fetch(h, pairs, 2 * (size_t)n, stream);
  if (rc != PA_OK) return rc;
  std::vector<int32_t> role(num_blocks, 0);  // bit 0: a source, bit 1: a destination
  for (int32_t i = 0; i < n; ++i) {
    const int32_t src = h[2 * i], dst = h[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;  // skipped
    if (role[dst] & 2)
      return fail(PA_EINVAL, "debug check: block %d is the destination of two pairs", dst);
    if ((role[dst] & 1) || (role[src] & 2) || src == dst)
      return fail(PA_EINVAL, "debug check: pair %d (%d -> %d) copies from or into a block "
                  "another pair writes or reads", i, src, dst);
    role[src] |= 1;
    role[dst] |= 2;
  }
  return PA_OK;
}

}  // namespace pagedkv

extern "C" int pa_set_debug_checks(int32_t on) {
  pagedkv::g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
  return pagedkv::ok();
}

extern "C" int pa_debug_checks(void) { return pagedkv::debug_checks() ? 1 : 0; }

extern "C" const char* pa_last_error(void) { return pagedkv::last_error().c_str(); }

extern "C" int pa_version(void) { return 100; }
