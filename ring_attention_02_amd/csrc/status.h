// Internal status / error-string helpers shared by the library's sources.
#pragma once
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/ringattn.h"

namespace ringattn {

// Records a formatted detail string for cp_last_error() and returns `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's detail string and returns CP_OK.
int32_t ok();

}  // namespace ringattn

#define RA_CHECK(cond, code, ...)                  \
  do {                                             \
    if (!(cond)) return ringattn::fail(code, __VA_ARGS__); \
  } while (0)
