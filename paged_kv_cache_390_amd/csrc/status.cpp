// Thread-local error reporting behind pa_last_error().
#include <cstdarg>
#include <cstdio>

#include "pa.h"
#include "pa_internal.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace pa {

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_msg; }
