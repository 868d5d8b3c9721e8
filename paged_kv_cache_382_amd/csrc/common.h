// Shared helpers of the C ABI: thread-local error text and status returns.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"

namespace pa {

std::string& error_text();

// Record a message for pa_last_error() and return `status`.
inline pa_status fail(pa_status status, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

inline pa_status fail(pa_status status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    error_text() = buf;
    return status;
}

inline pa_status ok() {
    error_text().clear();
    return PA_OK;
}

}  // namespace pa
