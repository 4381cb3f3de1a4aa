// Helpers shared by the files that define the C entry points (runtime.hip,
// policy.hip). Hidden: none of these is exported from the library.
#pragma once

#include "../../include/tod.h"

// Records a printf-style message as the calling thread's last error (what
// last_error() returns) and returns code.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// TOD_OK when init_model accepts the pair; otherwise TOD_EINVAL with the first
// violated rule recorded. Checks the configurations only: no device call, no
// allocation.
int check_config(const tod_model_config *cfg, const tod_run_config *run);
