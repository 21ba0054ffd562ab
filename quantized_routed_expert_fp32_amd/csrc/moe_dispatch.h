// Kernel launch with optional dispatch timing (HIP sources only).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace moe {

// Launches kernel k; when ev is given, ev[i] / ev[i + 1] (each may be NULL)
// take the dispatch's own start and end times (hipExtLaunchKernelGGL), so the
// events time the kernel alone, not the queue around it.
template <typename K, typename... Args>
inline void launch_k(K k, dim3 grid, dim3 block, uint32_t shm, hipStream_t s, hipEvent_t* ev, int i,
                     Args... args) {
  if (ev && (ev[i] || ev[i + 1]))
    hipExtLaunchKernelGGL(k, grid, block, shm, s, ev[i], ev[i + 1], 0, args...);
  else
    hipLaunchKernelGGL(k, grid, block, shm, s, args...);
}

}  // namespace moe
