// Kernel launches with their own status, shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "mla_post.h"

namespace mla_dev {

// The HIP error string of the last failed launch on this thread
// (mla_post_last_hip_error).
inline thread_local std::string g_hip_error;

inline int launched(hipError_t e) {
  if (e != hipSuccess) {
    g_hip_error = hipGetErrorString(e);
    return MLA_POST_ELAUNCH;
  }
  return MLA_POST_OK;
}

template <class T>
struct same_type {
  using type = T;
};

// Enqueue kernel k and report this launch's own status: hipLaunchKernel
// returns the error of this launch, so an error left pending by an earlier
// HIP call (the caller's, or a device query) is neither taken for it nor
// cleared. The arguments are converted to the kernel's parameter types
// before their addresses are taken.
template <typename... P>
int launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t stream, typename same_type<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return launched(hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, stream));
}

}  // namespace mla_dev
