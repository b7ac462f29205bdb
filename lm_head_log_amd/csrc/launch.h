// launch.h - kernel launches that report their own status.
//
// hipGetLastError() after a launch also reports a failure of any earlier HIP
// call made on the thread, including the caller's own; hipLaunchKernel
// returns the status of this launch alone. The arguments are converted to
// the kernel's parameter types and passed by address, as the runtime expects.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace lmh_launch {

template <typename... KArgs, typename... Args, size_t... I>
hipError_t launch_with(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                       std::index_sequence<I...>, Args&&... args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)] = {static_cast<void*>(&std::get<I>(vals))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, s);
}

// Launches kernel k on stream s; returns the launch's own hipError_t.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "one argument per kernel parameter");
  static_assert(sizeof...(KArgs) > 0, "kernels take arguments");
  return launch_with(k, grid, block, s, std::index_sequence_for<KArgs...>{},
                     std::forward<Args>(args)...);
}

}  // namespace lmh_launch
