// launch.hpp -- kernel launch that reports its own status.
//
// Every launcher returns the status of the launch it made, taken from the
// launch call itself: the thread's last-error state (which earlier, unrelated
// HIP calls of the process may have left set) is neither read nor cleared.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace w4a16 {

// Launch kern<<<grid, block, lds, stream>>>(args...), each argument converted
// to the kernel's parameter type; returns hipLaunchKernel's status.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> vals(static_cast<P>(std::forward<A>(args))...);
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, lds, stream);
      },
      vals);
}

}  // namespace w4a16
