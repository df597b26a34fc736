// sft_internal.h -- helpers shared by the library's translation units
// (error channel and argument checks).  Not part of the public ABI.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "sft.h"

namespace sft {

// Records the message of a failure for sft_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message at the start of a call.
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace sft

#define SFT_CHECK(cond, code, ...)               \
    do {                                         \
        if (!(cond))                             \
            return ::sft::fail((code), __VA_ARGS__); \
    } while (0)
