// timing.hip -- opt-in per-kernel timing with HIP events on the launch stream.
//
// When enabled, every kernel launch of the entry points is bracketed by two
// hipEvents recorded on the caller's stream; pdr_splat_timing_read waits for
// them and accumulates the elapsed milliseconds per kernel class.  Events are
// pooled and reused; nothing is recorded while timing is off.
#include <mutex>
#include <vector>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

namespace pdr {

namespace {

struct Pending {
  int kid;
  hipEvent_t a, b;
};

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double ms[PDR_KERNEL_COUNT] = {};
  long long count[PDR_KERNEL_COUNT] = {};
  hipEvent_t open[PDR_KERNEL_COUNT] = {};
};

TimingState &state() {
  static TimingState s;
  return s;
}

hipEvent_t take_event(TimingState &s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void timing_begin(int kid, hipStream_t st) {
  TimingState &s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on) return;
  hipEvent_t e = take_event(s);
  if (e && hipEventRecord(e, st) == hipSuccess) s.open[kid] = e;
}

void timing_end(int kid, hipStream_t st) {
  TimingState &s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on || !s.open[kid]) return;
  hipEvent_t e = take_event(s);
  if (e && hipEventRecord(e, st) == hipSuccess) s.pending.push_back({kid, s.open[kid], e});
  s.open[kid] = nullptr;
}

}  // namespace pdr

using namespace pdr;

extern "C" {

int pdr_splat_timing(int enable) {
  TimingState &s = state();
  std::lock_guard<std::mutex> g(s.mu);
  int prev = s.on ? 1 : 0;
  s.on = enable != 0;
  return prev;
}

int pdr_splat_timing_read(double *total_ms, long long *launches, int reset) {
  TimingState &s = state();
  std::lock_guard<std::mutex> g(s.mu);
  int rc = PDR_OK;
  for (const Pending &p : s.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
      rc = PDR_ERR_HIP;
    } else {
      s.ms[p.kid] += ms;
      s.count[p.kid] += 1;
    }
    s.pool.push_back(p.a);
    s.pool.push_back(p.b);
  }
  s.pending.clear();
  for (int k = 0; k < PDR_KERNEL_COUNT; ++k) {
    if (total_ms) total_ms[k] = s.ms[k];
    if (launches) launches[k] = s.count[k];
    if (reset) {
      s.ms[k] = 0.0;
      s.count[k] = 0;
    }
  }
  return rc;
}

const char *pdr_splat_kernel_name(int id) {
  static const char *names[PDR_KERNEL_COUNT] = {
      "preprocess", "bin_count", "scan", "bin_write",
      "forward_raster", "zero_verify", "backward_raster", "finalize",
      "loss_fwd", "loss_bwd", "loss_reduce", "grid_init", "activate", "activate_bwd"};
  return (id >= 0 && id < PDR_KERNEL_COUNT) ? names[id] : "unknown";
}

}  // extern "C"
