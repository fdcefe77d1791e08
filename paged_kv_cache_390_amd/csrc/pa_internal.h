// Internal helpers shared by the library's translation units (not part of
// the C ABI).
#pragma once

#include <cstdarg>

namespace pa {

// Record a message for pa_last_error() on the calling thread.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Record a message and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear the calling thread's message.
void clear_error();

}  // namespace pa
