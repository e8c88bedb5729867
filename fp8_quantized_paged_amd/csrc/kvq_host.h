// Host-side helpers shared by the kvq entry points: error reporting and argument
// checks.  Nothing here touches the device.
#pragma once

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "kvq.h"

namespace kvq {

// Records a formatted message for kvq_last_error() and returns `st`.
kvq_status fail(kvq_status st, const char* fmt, ...);
void clear_error();

inline bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
inline bool supported_group(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}

// Checks the fields of a cache descriptor that every call relies on.
kvq_status check_cache(const kvq_cache_desc* c);

}  // namespace kvq
