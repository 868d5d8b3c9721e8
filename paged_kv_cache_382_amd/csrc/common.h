// Shared helpers of the C ABI: thread-local error text and status returns.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <exception>
#include <new>

#include "pa.h"

namespace pa {

constexpr size_t kErrorChars = 512;
// The calling thread's last error message (a fixed buffer: reporting an error
// never allocates).
char* error_text();

// Record a message for pa_last_error() and return `status`.
inline pa_status fail(pa_status status, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

inline pa_status fail(pa_status status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(error_text(), kErrorChars, fmt, ap);
    va_end(ap);
    return status;
}

inline pa_status ok() {
    error_text()[0] = '\0';
    return PA_OK;
}

// Run an entry point's body; any C++ exception (host memory exhausted, or
// anything unexpected) becomes PA_ERR_HOST, so none crosses the C ABI.
template <class F>
pa_status guard(const char* fn, F&& body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(PA_ERR_HOST, "%s: out of host memory", fn);
    } catch (const std::exception& e) {
        return fail(PA_ERR_HOST, "%s: %s", fn, e.what());
    } catch (...) {
        return fail(PA_ERR_HOST, "%s: unexpected exception", fn);
    }
}

}  // namespace pa
