// kq_split.hpp — how the K parts of a split output tile meet (the W4A4 product and
// the product with the quantizer in its prologue).
//
// Each part of a tile, when its K range is done, adds 1 to the tile's flag word
// (bits 0-7 count arrivals).  Every part but the last to arrive stores its fp32
// sums in its own slot of the workspace, waits until they are visible to the
// device and adds kSplitReady (bits 8-15 count the stored parts); the last waits
// for parts - 1 stored parts, which come from workgroups already running that
// wait for nothing, adds every part's sums in part order and writes the tile, and
// puts the flag back to 0 for the next call.  No workgroup waits for one that may
// not have started, whatever the order workgroups run in.  The sums move as
// device-coherent (sc1) buffer stores and loads, the form of agent-scope relaxed
// atomics, so they need no cache write-back or invalidation (which would also drop
// the other workgroups' operands from the XCD's L2).  Included by the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

constexpr uint32_t kSplitReady = 256u;
constexpr int kSplitCoherent = 16;  // buffer cache policy sc1

// Adds this part's arrival (thread 0; `arrival` a workgroup-shared word) and
// returns, to every thread, whether it is the last part of the tile to arrive.
__device__ __forceinline__ bool split_arrive_last(uint32_t* flag, uint32_t parts, uint32_t& arrival) {
  if (threadIdx.x == 0) arrival = __hip_atomic_fetch_add(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return (__builtin_amdgcn_readfirstlane(arrival) & 0xFFu) + 1u >= parts;
}

// After every thread has stored its sums (kSplitCoherent buffer stores): once
// every wave's stores are visible device-wide, count the part as stored.
__device__ __forceinline__ void split_publish(uint32_t* flag) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(flag, kSplitReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last part: waits (bounded) for the other parts' stored sums, then resets the
// flag for the next call.
__device__ __forceinline__ void split_wait_reset(uint32_t* flag, uint32_t parts) {
  if (threadIdx.x == 0) {
    // bounded: the other parts have arrived and only store their sums before counting
    for (uint32_t n = 0; n < (1u << 26); ++n) {
      if (((__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 8) & 0xFFu) + 1u >= parts)
        break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kq
