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
hipEvent_t g_pending[kNumKernels] = {};

const char *kNames[kNumKernels] = {"gla_seg_state", "gla_seg_scan", "gla_seg_out"};

}  // namespace

void profile_mark(int kernel, hipStream_t stream, bool start) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  (void)hipEventRecord(ev, stream);
  if (start) {
    g_pending[kernel] = ev;
  } else if (g_pending[kernel]) {
    g_marks.push_back({kernel, g_pending[kernel], ev});
    g_pending[kernel] = nullptr;
  } else {
    (void)hipEventDestroy(ev);
  }
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
  for (auto &e : gtr::g_pending) {
    if (e) (void)hipEventDestroy(e);
    e = nullptr;
  }
  return rc == GTR_OK ? gtr::kNumKernels : rc;
}

const char *gtr_gla_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < gtr::kNumKernels) ? gtr::kNames[kernel] : "";
}

}  // extern "C"
