// Kernel launch helper. A launch made while the timing hook is armed for it
// (see smoe_trace_kernel) carries the caller's start/stop events on the
// dispatch itself (hipExtLaunchKernelGGL), so the events bracket the kernel's
// execution rather than the queue around it.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace smoe {

struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// events for the launches made by this thread while set (see TracedLaunch)
extern thread_local LaunchEvents t_launch_events;

template <typename... Args, typename K>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  if (t_launch_events.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t_launch_events.start,
                          t_launch_events.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

template <typename... Args, typename K>
hipError_t launch_kernel_lds(K kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t s,
                             Args... args) {
  if (t_launch_events.start)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t_launch_events.start,
                          t_launch_events.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}

// Takes the armed events when the hook is armed for `kernel` (disarming it)
// and attaches them to the launches made in this scope.
bool trace_take(int kernel, hipEvent_t* start, hipEvent_t* stop);

struct TracedLaunch {
  explicit TracedLaunch(int kernel) {
    hipEvent_t a, b;
    if (trace_take(kernel, &a, &b)) t_launch_events = LaunchEvents{a, b};
  }
  ~TracedLaunch() { t_launch_events = LaunchEvents{}; }
  TracedLaunch(const TracedLaunch&) = delete;
  TracedLaunch& operator=(const TracedLaunch&) = delete;
};

}  // namespace smoe
