// trace.hpp -- opt-in per-kernel timing with HIP events (internal).
//
// While tracing is enabled (attn_trace_enable), every kernel the library
// launches is bracketed by two HIP events recorded on the launch stream;
// attn_trace_collect reads them back.  When tracing is off a launch costs one
// relaxed atomic load more than a plain launch.
#pragma once

#include <hip/hip_runtime.h>

namespace lcattn {

bool trace_on();
int trace_begin(const char* name, hipStream_t stream);  // slot, or -1 when full
void trace_end(int slot, hipStream_t stream);

}  // namespace lcattn

// hipLaunchKernelGGL with optional event bracketing.  KERNEL must be
// parenthesised when it has template arguments.
#define LCATTN_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                  \
  do {                                                                               \
    const int lcattn_slot_ = lcattn::trace_on() ? lcattn::trace_begin(NAME, STREAM) : -1; \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);              \
    if (lcattn_slot_ >= 0) lcattn::trace_end(lcattn_slot_, STREAM);                   \
  } while (0)
