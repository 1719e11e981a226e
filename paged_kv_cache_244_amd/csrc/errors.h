// Thread-local error text behind pkv_last_error().
#pragma once

#include <cstdarg>

namespace pkv {

// Formats the message, stores it for pkv_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Events set by pkv_time_next_call for the next device call on this thread
// (hipEvent_t as void*): its first kernel records `start` when it starts, every
// kernel records `stop` when it ends.
struct CallTiming {
  void* start = nullptr;
  void* stop = nullptr;
};
CallTiming& call_timing();

// Declared at the top of every C entry point that launches kernels: the
// events set for "the next call" are consumed by that call, whatever path it
// returns through.
struct TimedCall {
  TimedCall() = default;
  TimedCall(const TimedCall&) = delete;
  TimedCall& operator=(const TimedCall&) = delete;
  ~TimedCall() { call_timing() = CallTiming{}; }
};

}  // namespace pkv
