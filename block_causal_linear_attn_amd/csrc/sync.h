// sync.h -- flag hand-off between the work items of one launch.
//
// A producer item publishes a 64-bit flag equal to the launch's epoch (a
// value the host never reuses) once its global stores are complete; a
// consumer polls the flag with device-scope atomic loads (which bypass the
// CU's L1) and then reads the data.  With publish() and wait_all(), producer
// and consumer run on the same XCD (their block ids are equal modulo 8), so
// the data itself passes through that XCD's L2: a store counts as complete
// (vmcnt reaches zero) once the L2 has taken it.  A hand-off between XCDs
// takes publish_release() and wait_all_acquire(), whose agent-scope fences
// write back the producer's L2 and invalidate the consumer's caches; each
// costs microseconds, so they are kept off serial chains.  Waits are
// bounded: after kSpinLimit polls a wait gives up, sets *err and continues,
// so a launch always finishes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linscan {

constexpr int kSpinLimit = 1 << 22;

// All of this workgroup's global stores are complete; then *flag = epoch.
__device__ __forceinline__ void publish(uint64_t* flag, uint64_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns once flags[0 .. n) all equal epoch (or a wait timed out).
__device__ __forceinline__ void wait_all(const uint64_t* flags, int n, uint64_t epoch, uint32_t* err) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int spins = 0;
    while (__hip_atomic_load(&flags[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      if (++spins > kSpinLimit) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// publish() for a consumer that may run on another XCD: a release fence at
// agent scope (the XCD's L2 is written back) before the flag.
__device__ __forceinline__ void publish_release(uint64_t* flag, uint64_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// wait_all() for data a producer on another XCD published with
// publish_release(): the first wave takes an acquire fence at agent scope
// (the CU's L1 and the XCD's L2 drop stale lines), and a barrier orders the
// other waves' loads after it.
__device__ __forceinline__ void wait_all_acquire(const uint64_t* flags, int n, uint64_t epoch, uint32_t* err) {
  wait_all(flags, n, epoch, err);
  if (threadIdx.x < 64) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
}

}  // namespace linscan
