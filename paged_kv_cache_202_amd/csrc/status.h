// Error reporting shared by the allocator and the device entry points.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pagedkv.h"

namespace pkv {

// Thread-local text of the last error; returned by paged_kv_last_error().
std::string &last_error();

// Record a formatted message and return `code` (so callers can `return fail(...)`).
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pkv
