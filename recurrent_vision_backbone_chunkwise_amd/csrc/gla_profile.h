// Optional per-kernel timing with HIP events (see gtr_gla_profile_begin/end).
#pragma once

#include <hip/hip_runtime_api.h>

namespace gtr {

enum KernelId : int { kKernelSegState = 0, kKernelSegScan = 1, kKernelSegOut = 2, kNumKernels = 3 };

// Records an event on `stream` before (start = true) or after a kernel launch
// while profiling is on and the stream is not being captured.  No-op otherwise.
void profile_mark(int kernel, hipStream_t stream, bool start);

}  // namespace gtr
