// Status codes and the per-thread error message shared by every entry point.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pagedkv.h"

namespace pagedkv {

std::string& last_error();

// Record a message for pa_last_error() and return `code`.
inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error() = buf;
  return code;
}

inline int ok() {
  last_error().clear();
  return PA_OK;
}

}  // namespace pagedkv

namespace pagedkv {

// Host re-checks of the promises the device entry points rely on (distinct slots, copy
// pairs disjoint from their sources, share groups whose members' tables agree): on when
// the environment variable PA_DEBUG_CHECKS is set to a value other than 0 when the library
// first checks, or after pa_set_debug_checks(1). Each check copies the device arrays it
// needs to the host (ordered on the call's stream, which it waits for).
bool debug_checks();

}  // namespace pagedkv
