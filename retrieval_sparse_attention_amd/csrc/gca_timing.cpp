// Per-kernel HIP event timing.  Off by default; when on, every kernel launch of
// the library is bracketed by two events recorded on the launch stream, and
// gca_timing_collect() turns the recorded pairs into per-kernel sums.

#include <mutex>
#include <vector>

#include "gca.h"
#include "gca_launch.h"

namespace gca {
namespace {

struct Pending {
  int kid;
  hipEvent_t a, b;
};

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  double total_ms[kNumKernels] = {};
  int64_t launches[kNumKernels] = {};
};

TimingState& state() {
  static TimingState* s = new TimingState();  // lives until process exit
  return *s;
}

hipEvent_t take_event(TimingState& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* kNames[kNumKernels] = {"scan_topk", "topk_merge", "forward",
                                   "reverse_index", "backward_q", "backward_kv",
                                   "gather_kv", "swa_forward", "swa_backward_q",
                                   "swa_backward_kv", "topk_merge_forward"};

}  // namespace

KernelTimer::KernelTimer(int kernel_id, hipStream_t stream) : kid_(kernel_id), stream_(stream) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on) return;
  start_ = take_event(s);
  if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
    s.pool.push_back(start_);
    start_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  hipEvent_t end = take_event(s);
  if (end && hipEventRecord(end, stream_) == hipSuccess) {
    s.pending.push_back({kid_, start_, end});
  } else {
    s.pool.push_back(start_);
    if (end) s.pool.push_back(end);
  }
}

}  // namespace gca

extern "C" {

int gca_num_kernels(void) { return gca::kNumKernels; }

const char* gca_kernel_name(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= gca::kNumKernels) return "";
  return gca::kNames[kernel_id];
}

gca_status gca_timing_enable(int on) {
  gca::TimingState& s = gca::state();
  std::lock_guard<std::mutex> g(s.mu);
  s.on = on != 0;
  return GCA_OK;
}

gca_status gca_timing_collect(double* total_ms, int64_t* launches) {
  gca::TimingState& s = gca::state();
  std::lock_guard<std::mutex> g(s.mu);
  gca_status st = GCA_OK;
  for (const gca::Pending& p : s.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess)
      st = GCA_ERR_DEVICE;
    s.total_ms[p.kid] += ms;
    s.launches[p.kid] += 1;
    s.pool.push_back(p.a);
    s.pool.push_back(p.b);
  }
  s.pending.clear();
  for (int k = 0; k < gca::kNumKernels; ++k) {
    if (total_ms) total_ms[k] = s.total_ms[k];
    if (launches) launches[k] = s.launches[k];
    s.total_ms[k] = 0.0;
    s.launches[k] = 0;
  }
  return st;
}

}  // extern "C"
