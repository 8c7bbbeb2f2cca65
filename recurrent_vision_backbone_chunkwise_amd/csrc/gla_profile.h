// Optional per-kernel timing with HIP events (see gtr_gla_profile_begin/end).
#pragma once

#include <hip/hip_runtime_api.h>

namespace gtr {

enum KernelId : int {
  kKernelSegState = 0,
  kKernelSegScan = 1,
  kKernelSegOut = 2,
  kKernelFused = 3,
  kKernelSwigluIn = 4,   // Spatial SwiGLU input projection (library GEMM)
  kKernelSwigluMix = 5,  // depthwise 3x3 + SiLU gate
  kKernelSwigluOut = 6,  // output projection (library GEMM)
  kKernelBwdDqk = 7,     // backward chunk kernel (dq, dk)
  kKernelBwdDgate = 8,   // gate gradient (running sums from the dk pass's chunk totals)
  kKernelBwdDs0 = 9,     // gradient of the initial state
  kNumKernels = 10
};

// While profiling is on and `stream` is not being captured, creates a pair of
// events for the next launch of `kernel` (to be passed to hipExtLaunchKernelGGL,
// which timestamps the dispatch itself) and returns true.  Otherwise returns
// false and leaves both events null.
bool profile_events(int kernel, hipStream_t stream, hipEvent_t *start, hipEvent_t *stop);

// Records start/stop on `stream` around work enqueued between the two calls
// (library calls that do not take events themselves); no-ops while off.
struct ProfileScope {
  ProfileScope(int kernel, hipStream_t stream);
  ~ProfileScope();
  hipStream_t stream;
  hipEvent_t start, stop;
};

}  // namespace gtr
