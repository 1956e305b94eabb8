// Host-side helpers shared by the C ABI sources.
#pragma once

namespace sv {

// Record a printf-style message for spec_verify_last_error() (thread-local)
// and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace sv
