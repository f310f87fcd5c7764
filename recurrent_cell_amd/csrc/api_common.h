// Host-side helpers shared by the C-ABI translation units of libcfc.so: the
// per-thread last-error text, error returns and argument-overlap checks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/cfc.h"

namespace cfc_host {

// One text per thread for the whole library (cfc_last_error returns it).
inline std::string& last_error()
{
    static thread_local std::string s;
    return s;
}

inline int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    last_error() = buf;
    return code;
}

inline int hip_fail(hipError_t e, const char* what)
{
    return fail(CFC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

struct Span {
    const void* p;
    size_t bytes;
};

inline bool overlap(Span a, Span b)
{
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

inline Span span(const void* p, int64_t n) { return Span{p, (size_t)(n > 0 ? n : 0) * sizeof(float)}; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace cfc_host

#define CFC_HIP(call, what)                                        \
    do {                                                           \
        hipError_t e_ = (call);                                    \
        if (e_ != hipSuccess) return cfc_host::hip_fail(e_, what); \
    } while (0)
