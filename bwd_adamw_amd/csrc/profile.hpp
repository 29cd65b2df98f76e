// Opt-in launch timing for diagnostics (lora_profile_begin/end).
//
// While a profile is open, every kernel launch of the library is bracketed
// by a pair of HIP events recorded on the launch's own stream; closing the
// profile waits for the device and aggregates elapsed times per (kernel,
// shape).  Each record carries the launch's algorithmic flops and bytes so a
// caller can place it on the roofline.  Closed (the default) it costs one
// branch per launch.  Not thread-safe: one profiling caller at a time.
#pragma once
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

class Scope {
 public:
  Scope(hipStream_t st, const char* name, int64_t M, int64_t N, int64_t K, double flops,
        double bytes)
      : st_(st), idx_(-1) {
    State& s = state();
    if (!s.on || s.used + 2 > s.events.size()) return;
    idx_ = (int)s.used;
    s.used += 2;
    s.recs.push_back({name, M, N, K, flops, bytes, idx_});
    (void)hipEventRecord(s.events[idx_], st_);
  }
  ~Scope() {
    if (idx_ >= 0) (void)hipEventRecord(state().events[idx_ + 1], st_);
  }

 private:
  hipStream_t st_;
  int idx_;
};

}  // namespace prof
}  // namespace lora
