// Host-side helpers shared by the library's translation units (no device code).
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "cb.h"

namespace cb {

// Per-thread message behind cb_last_error().
std::string& last_error();

inline void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error() = buf;
}

template <typename... Args>
inline int fail(int status, const char* fmt, Args... args) {
  set_error(fmt, args...);
  return status;
}

}  // namespace cb
