// Every kernel of the library is launched through here: on the caller's
// stream, with the profile's packet-timestamp events when one is open
// (profile.hpp).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "profile.hpp"

namespace lora {

template <typename F, typename... Args>
void launch_n(F kern, dim3 grid, unsigned threads, hipStream_t st, const prof::Scope& ps,
              Args... args) {
  hipExtLaunchKernelGGL(kern, grid, dim3(threads), 0, st, ps.start(), ps.stop(), 0, args...);
}
template <typename F, typename... Args>
void launch(F kern, dim3 grid, hipStream_t st, const prof::Scope& ps, Args... args) {
  launch_n(kern, grid, 256u, st, ps, args...);
}

}  // namespace lora
