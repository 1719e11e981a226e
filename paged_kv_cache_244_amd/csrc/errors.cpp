#include "errors.h"

#include <cstdio>

#include "pagedkv.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace pkv {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error; }
