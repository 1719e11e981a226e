#include "errors.h"

#include <cstdio>

#include "pagedkv.h"

namespace {
thread_local char g_last_error[512] = "";
thread_local pkv::CallTiming g_call_timing;
}

namespace pkv {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

CallTiming& call_timing() { return g_call_timing; }

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error; }

extern "C" int pkv_time_next_call(void* start_event, void* stop_event) {
  pkv::call_timing() = pkv::CallTiming{start_event, stop_event};
  return PKV_OK;
}
