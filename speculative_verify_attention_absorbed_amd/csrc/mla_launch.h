// Kernel launch with the launch call's own status (HIP sources only).
//
// hipLaunchKernel returns the error of this launch itself; the thread's
// sticky last-error state, which may hold an unrelated earlier failure (for
// example one left by another library on the same thread), is neither read
// nor cleared.
#ifndef MLA_LAUNCH_H
#define MLA_LAUNCH_H

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

#include "mla_verify.h"

namespace mla {

template <typename Tuple, size_t... I>
inline int launch_tuple(const void* kernel, dim3 grid, dim3 block, unsigned smem, hipStream_t stream,
                        Tuple& args, std::index_sequence<I...>) {
  void* argv[] = {static_cast<void*>(&std::get<I>(args))..., nullptr};
  return hipLaunchKernel(kernel, grid, block, argv, smem, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Launches `kernel` with `args` converted to its parameter types; returns
// MLA_OK, or MLA_ERR_HIP when the launch is rejected.
template <typename... KArgs, typename... Args>
inline int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned smem, hipStream_t stream,
                  Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  return launch_tuple(reinterpret_cast<const void*>(kernel), grid, block, smem, stream, vals,
                      std::index_sequence_for<KArgs...>{});
}

}  // namespace mla

#endif
