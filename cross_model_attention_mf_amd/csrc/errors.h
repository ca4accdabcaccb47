// Per-thread error message of the last failing call.
#pragma once

#include <stdarg.h>
#include <stdio.h>

#include "mapflow.h"

namespace mf {

inline char* error_buffer() {
  static thread_local char buf[512];
  return buf;
}

inline void clear_error() { error_buffer()[0] = 0; }

inline mf_status fail(mf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(error_buffer(), 512, fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace mf
