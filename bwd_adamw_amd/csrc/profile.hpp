// Opt-in launch timing for diagnostics (lora_profile_begin/end).
//
// While a profile is open, every kernel launch of the library carries a pair
// of HIP events that the launch's dispatch packet timestamps (start and end of
// the kernel, on the launch's own stream); closing the profile waits for the
// device and aggregates elapsed times per (kernel, shape).  Each record carries the launch's algorithmic flops and bytes so a
// caller can place it on the roofline.  Closed (the default) it costs one
// branch per launch.  Not thread-safe: one profiling caller at a time.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <string.h>

#include <vector>

#include "../../include/lora.h"

namespace lora {
namespace prof {

struct Rec {
  const char* name;
  int64_t M, N, K;
  double flops, bytes;
  int ev;   // index of the start event; ev + 1 is the stop event
};

struct State {
  bool on = false;
  std::vector<hipEvent_t> events;
  std::vector<Rec> recs;
  size_t used = 0;
};

inline State& state() {
  static State s;
  return s;
}

// Events for one launch: both null unless a profile is open.  The kernel is
// launched with hipExtLaunchKernelGGL, which timestamps the dispatch packet
// itself, so the elapsed time is the kernel's own execution time.
class Scope {
 public:
  Scope(const char* name, int64_t M, int64_t N, int64_t K, double flops, double bytes)
      : a_(nullptr), b_(nullptr) {
    State& s = state();
    if (!s.on || s.used + 2 > s.events.size()) return;
    const int idx = (int)s.used;
    s.used += 2;
    s.recs.push_back({name, M, N, K, flops, bytes, idx});
    a_ = s.events[idx];
    b_ = s.events[idx + 1];
  }
  hipEvent_t start() const { return a_; }
  hipEvent_t stop() const { return b_; }

 private:
  hipEvent_t a_, b_;
};

}  // namespace prof
}  // namespace lora
