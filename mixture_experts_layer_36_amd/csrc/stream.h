// Helpers of the streaming kernels that read x (routing and the router's
// weight gradient): the LDS size that bounds their residency, and a barrier
// that lets global loads stay in flight across it.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

// LDS bytes of one compute unit
constexpr int kLdsPerCu = 160 * 1024;

// A workgroup barrier that orders LDS traffic only: outstanding global loads
// stay in flight across it (a plain __syncthreads waits for them as well).
__device__ __forceinline__ void lds_only_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moe
