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

#include <climits>

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

// Which tiles an XCD takes.  Workgroups go to the 8 XCDs round-robin by index and a
// tile's parts run on workgroups p n8 + t (n8 a multiple of 8), so the tiles t = x,
// x + 8, ... are XCD x's.  They are made the x-th run of an order that goes down
// bands of band_rows tile rows column by column, so each XCD's tiles form one
// compact block of the tile grid and share their operand rows in its L2.  The map is
// a bijection onto the tiles_m x tiles_n grid (ntiles = tiles_m tiles_n).
__device__ __forceinline__ void split_tile(uint32_t t, uint32_t ntiles, uint32_t tiles_n, uint32_t band_rows,
                                           uint32_t& tm, uint32_t& tn) {
  const uint32_t x = t & 7u, u = t >> 3, r8 = ntiles & 7u;
  const uint32_t j = x * (ntiles >> 3) + (x < r8 ? x : r8) + u;  // position in the order
  const uint32_t tiles_m = ntiles / tiles_n, span = band_rows * tiles_n;
  const uint32_t band = j / span, within = j - band * span;
  const uint32_t left = tiles_m - band * band_rows;
  const uint32_t rows_b = left < band_rows ? left : band_rows;  // rows in this band
  tn = within / rows_b;
  tm = band * band_rows + (within - tn * rows_b);
}

// The band height for split_tile: the one whose runs of ceil(ntiles / 8) tiles span
// the fewest tile rows plus columns (1024 x 3072 x 12288 in 256 x 256 tiles: an XCD's
// 6 tiles as 2 x 3 instead of 4 rows x 3 columns, 50.1-50.8 -> 47.2-47.4 us).
inline uint32_t split_band_rows(int64_t ntiles, int64_t tiles_n) {
  const int64_t tiles_m = ntiles / tiles_n, k = (ntiles + 7) / 8;
  int64_t best = 1, cost = INT64_MAX;
  for (int64_t r = 1; r <= tiles_m && r <= k; ++r) {
    const int64_t c = r + (k + r - 1) / r;
    if (c < cost) {
      cost = c;
      best = r;
    }
  }
  return (uint32_t)best;
}

}  // namespace kq
