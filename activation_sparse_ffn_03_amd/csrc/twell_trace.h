// Optional per-kernel tracing: when enabled through the C ABI, every kernel
// launch of the library is bracketed by HIP events recorded on its stream.
#pragma once

#include <hip/hip_runtime.h>

namespace twell {

bool trace_on();
void trace_begin(hipStream_t s, const char* name);
void trace_end(hipStream_t s);

// Launch a kernel bracketed by trace events (no-ops when tracing is off).
#define TWELL_LAUNCH(name, kernel, grid, block, lds, stream, ...)        \
  do {                                                                  \
    ::twell::trace_begin((stream), (name));                             \
    kernel<<<(grid), (block), (lds), (stream)>>>(__VA_ARGS__);          \
    ::twell::trace_end((stream));                                       \
  } while (0)

}  // namespace twell
