// Thread-local error text behind pkv_last_error().
#pragma once

#include <cstdarg>

namespace pkv {

// Formats the message, stores it for pkv_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pkv
