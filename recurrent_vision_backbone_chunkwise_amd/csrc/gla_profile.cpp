// Per-kernel timing with HIP events on the launch stream.  Off unless
// gtr_gla_profile_begin() was called; events are never recorded while the
// stream is being captured into a graph.

#include "gla_profile.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "gtr_gla.h"

namespace gtr {
namespace {

struct Mark {
  int kernel;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Mark> g_marks;

const char *kNames[kNumKernels] = {"gla_seg_state",  "gla_seg_scan",  "gla_seg_out",    "gla_fused",
                                   "swiglu_gemm_in", "swiglu_mix",    "swiglu_gemm_out", "gla_bwd_dqk",
                                   "gla_bwd_dgate",  "gla_bwd_ds0"};

}  // namespace

bool profile_events(int kernel, hipStream_t stream, hipEvent_t *start, hipEvent_t *stop) {
  *start = nullptr;
  *stop = nullptr;
  if (!g_on.load(std::memory_order_relaxed)) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return false;
  }
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
    (void)hipGetLastError();
    if (a) (void)hipEventDestroy(a);
    return false;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  g_marks.push_back({kernel, a, b});
  *start = a;
  *stop = b;
  return true;
}

ProfileScope::ProfileScope(int kernel, hipStream_t s) : stream(s) {
  if (profile_events(kernel, s, &start, &stop)) (void)hipEventRecord(start, s);
}
ProfileScope::~ProfileScope() {
  if (stop) (void)hipEventRecord(stop, stream);
}

}  // namespace gtr

extern "C" {

void gtr_gla_profile_begin(void) {
  std::lock_guard<std::mutex> lock(gtr::g_mu);
  gtr::g_marks.clear();
  gtr::g_on.store(true);
}

int gtr_gla_profile_end(double *total_ms, int *launches, int max_kernels) {
  std::lock_guard<std::mutex> lock(gtr::g_mu);
  gtr::g_on.store(false);
  const int n = max_kernels < gtr::kNumKernels ? max_kernels : gtr::kNumKernels;
  for (int i = 0; i < n; ++i) {
    if (total_ms) total_ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  int rc = GTR_OK;
  for (const auto &m : gtr::g_marks) {
    float ms = 0.f;
    if (hipEventSynchronize(m.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, m.start, m.stop) != hipSuccess) {
      (void)hipGetLastError();
      rc = GTR_ERR_LAUNCH;
    } else if (m.kernel < n) {
      if (total_ms) total_ms[m.kernel] += ms;
      if (launches) launches[m.kernel] += 1;
    }
    (void)hipEventDestroy(m.start);
    (void)hipEventDestroy(m.stop);
  }
  gtr::g_marks.clear();
  return rc == GTR_OK ? gtr::kNumKernels : rc;
}

const char *gtr_gla_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < gtr::kNumKernels) ? gtr::kNames[kernel] : "";
}

}  // extern "C"
