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
