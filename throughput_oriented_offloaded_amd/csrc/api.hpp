// Helpers shared by the files that define the C entry points (runtime.hip,
// policy.hip). Hidden: none of these is exported from the library.
#pragma once

#include <new>

#include "../../include/tod.h"

// Records a printf-style message as the calling thread's last error (what
// last_error() returns) and returns code. Writes a fixed thread-local buffer:
// it never allocates and never throws.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// TOD_OK when init_model accepts the pair; otherwise TOD_EINVAL with the first
// violated rule recorded. Checks the configurations only: no device call, no
// allocation.
int check_config(const tod_model_config *cfg, const tod_run_config *run);

// Runs the body of a C entry point so that no C++ exception crosses the C ABI:
// std::bad_alloc (a host container or new that ran out of memory) becomes
// TOD_ENOMEM, anything else TOD_EHIP, each with a message naming the entry point.
template <class F>
int guard(const char *fn, F &&body) noexcept
{
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return fail(TOD_ENOMEM, "%s: out of host memory", fn);
    } catch (...) {
        return fail(TOD_EHIP, "%s: unexpected internal error", fn);
    }
}
