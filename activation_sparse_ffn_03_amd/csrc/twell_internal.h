// Internal entry points shared between the C ABI source files.
#pragma once

#include <stddef.h>

#include "../../include/twell.h"

namespace twell {

// Record `why` as the calling thread's last error message and return `st`.
twell_status set_error(twell_status st, const char* why);

// twell_ffn_forward with two extra switches: `use_side` false enqueues every
// kernel on `stream` in order (no side stream is created or used);
// `validate_only` checks every argument and returns without enqueuing.
twell_status ffn_forward_call(const twell_dims* dims, twell_dtype dtype, const void* x, const void* w_gate_t,
                              const float* t, const twell_pack* pack, const void* w_up_t, const void* w_down,
                              float* y, float* a_save, void* ws, size_t ws_bytes, void* gate_ws, size_t gate_ws_bytes,
                              bool use_side, bool validate_only, void* stream);

}  // namespace twell
