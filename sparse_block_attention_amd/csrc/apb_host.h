// Host-only helpers of the C ABI: argument checks and the per-thread error text.
// No HIP types here, so validate.cpp also builds with a plain C++ compiler.
#pragma once

#include <stdint.h>

#include "apb.h"

namespace apb_host {

// Records a message for apb_last_error() and returns `st`.
apb_status fail(apb_status st, const char *fmt, ...);
void clear_error();

bool aligned16(const void *p);

// Full check of a problem description (also used by apb_validate_problem).
apb_status check_problem(const apb_problem *pr);

// q heads of each kv head in ascending order: out[h * g + j] = j-th q head of
// kv head h.  The problem must already have passed check_problem.
void slot_table(const apb_problem *pr, uint8_t *out /* [n_q_heads] */);

}  // namespace apb_host
