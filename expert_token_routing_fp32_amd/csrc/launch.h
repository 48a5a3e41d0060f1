// Kernel launch with optional dispatch-timestamped events.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <utility>

namespace moek {

// With an event, hipExtLaunchKernelGGL records e0 at the dispatch's start and
// e1 at its end (no marker packets); without one the plain launch is used,
// so untimed calls take the ordinary launch path.
template <typename... P, typename... A>
inline void launch_timed(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1, A&&... args) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0, std::forward<A>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, std::forward<A>(args)...);
}

}  // namespace moek
