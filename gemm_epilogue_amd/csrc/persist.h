// Grid-wide barrier for the library's persistent (cooperative) kernels.
//
// A counter in device memory that every block increments once per barrier
// and polls until it reaches (barriers so far) x (blocks).  The launch is
// cooperative, so all blocks are resident; the poll is still bounded, and a
// block that gives up sets the error word, which makes every other block
// give up at its next barrier too.
//
// Ordering: the block's own stores are complete at its workgroup barrier,
// one agent-scope release fence writes the XCD's L2 back before the
// arrival, the poll itself is a relaxed agent-scope load (it goes past the
// non-coherent L2 without invalidating it), and one agent-scope acquire
// fence after the wait invalidates stale lines before the block reads what
// other blocks wrote.  An acquire load inside the poll loop would invalidate
// the L2 on every iteration, under the feet of the blocks still computing.
#pragma once

#include <hip/hip_runtime.h>

namespace ge {

constexpr int kGridSpinLimit = 1 << 22;  // polls of about 64 cycles each before giving up

// the counter must start at zero at the launch; returns false when the
// barrier timed out (or another block reported that)
__device__ __forceinline__ bool grid_barrier(unsigned *count, unsigned target, unsigned *err) {
  __shared__ int grid_barrier_ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int good = 1, spins = 0;
    while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > kGridSpinLimit ||
          ((spins & 63) == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        good = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    grid_barrier_ok = good;
  }
  __syncthreads();
  return grid_barrier_ok != 0;
}

}  // namespace ge
