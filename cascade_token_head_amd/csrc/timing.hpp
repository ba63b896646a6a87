// Optional per-kernel timing with HIP events on the launching stream.
// Off unless switched on through spatten_debug_timing(); when on, every
// kernel launch is bracketed by two events and durations are aggregated
// per kernel name by spatten_debug_kernel_times().
#pragma once

#include <hip/hip_runtime.h>

namespace spatten {

extern bool g_timing;
void timing_mark(const char* name, hipStream_t stream, bool begin);

}  // namespace spatten

#define SPATTEN_TIMED(name, stream, ...)                         \
  do {                                                           \
    if (::spatten::g_timing) ::spatten::timing_mark(name, stream, true);  \
    __VA_ARGS__;                                                 \
    if (::spatten::g_timing) ::spatten::timing_mark(name, stream, false); \
  } while (0)
