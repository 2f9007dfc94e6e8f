// kq_bench_stream.hip — the quantizer's memory traffic without its arithmetic
// (64 B read, 16 B + 1 B written per 32-element bf16 unit), for the practical HBM
// ceiling reported beside the quantizer's time.  Several access designs, so that
// the ceiling is the best of them rather than one kernel's: one unit per lane in a
// grid-stride loop; two units per lane with both loads issued before any store; a
// lane walking its units with the next two in flight; and the read-only and
// write-only halves of the traffic.  Declared in include/kq_bench.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_bench.h"

namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_unit(const uint8_t* __restrict__ x, uint32_t u) {
  const u32x4* p = reinterpret_cast<const u32x4*>(x + (uint64_t)u * 64);
  return p[0] ^ p[1] ^ p[2] ^ p[3];
}

// 16 code bytes and one scale byte per unit, derived from the input so the reads
// cannot be dropped (the values mean nothing)
__device__ __forceinline__ void store_unit(uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                           uint32_t u, u32x4 w) {
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(q + (uint64_t)u * 16));
  __builtin_nontemporal_store((uint8_t)(w.x ^ w.y ^ w.z ^ w.w), s + u);
}

__global__ __launch_bounds__(kThreads) void stream_kernel(const uint8_t* __restrict__ x,
                                                          uint32_t units,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
  const uint32_t lanes = gridDim.x * kThreads;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += lanes)
    store_unit(q, s, u, load_unit(x, u));
}

// two units per lane (u and u + lanes), both loads before either store
__global__ __launch_bounds__(kThreads) void stream_pair_kernel(const uint8_t* __restrict__ x,
                                                               uint32_t units,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ s) {
  const uint32_t lanes = gridDim.x * kThreads;
  const uint32_t last = units - 1;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += 2 * lanes) {
    const uint32_t u2 = u + lanes;
    const u32x4 a = load_unit(x, u), b = load_unit(x, u2 < last ? u2 : last);
    store_unit(q, s, u, a);
    if (u2 < units) store_unit(q, s, u2, b);
  }
}

// a lane walks u, u + lanes, ... with the next two units' loads in flight (loads
// past the end re-read the last unit)
__global__ __launch_bounds__(kThreads) void stream_ring_kernel(const uint8_t* __restrict__ x,
                                                               uint32_t units,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ s) {
  const uint32_t lanes = gridDim.x * kThreads;
  const uint32_t last = units - 1;
  uint32_t u = blockIdx.x * kThreads + threadIdx.x;
  if (u > last) return;
  auto clamp = [&](uint32_t v) { return v < last ? v : last; };
  u32x4 r0 = load_unit(x, clamp(u)), r1 = load_unit(x, clamp(u + lanes));
  for (;;) {
    const u32x4 a = r0;
    r0 = load_unit(x, clamp(u + 2 * lanes));
    store_unit(q, s, u, a);
    u += lanes;
    if (u > last) return;
    const u32x4 b = r1;
    r1 = load_unit(x, clamp(u + 2 * lanes));
    store_unit(q, s, u, b);
    u += lanes;
    if (u > last) return;
  }
}

// the read half alone: every unit read once, one byte written per lane at the end
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint8_t* __restrict__ x,
                                                               uint32_t units,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ s) {
  const uint32_t lanes = gridDim.x * kThreads;
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (uint32_t u = g; u < units; u += lanes) acc ^= load_unit(x, u);
  if (g < units) s[g] = (uint8_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

// the write half alone: 16 + 1 bytes per unit from the unit index
__global__ __launch_bounds__(kThreads) void stream_write_kernel(const uint8_t* __restrict__ x,
                                                                uint32_t units,
                                                                uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ s) {
  const uint32_t lanes = gridDim.x * kThreads;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += lanes) {
    const u32x4 w = {u, u * 3u, u * 5u, u * 7u};
    store_unit(q, s, u, w);
  }
}

}  // namespace

extern "C" int kq_bench_stream_design(const void* x, int64_t units, uint8_t* q, uint8_t* s,
                                      int grid, int design, void* stream) {
  if (units < 0 || units >= (int64_t(1) << 30) || grid < 1 || grid > 65535) return -2;
  if (design < KQB_LANE || design > KQB_WRITE) return -2;
  if (units == 0) return 0;
  if (!x || !q || !s) return -1;
  if (((uintptr_t)x & 15) || ((uintptr_t)q & 15)) return -3;
  void (*k)(const uint8_t*, uint32_t, uint8_t*, uint8_t*) =
      design == KQB_LANE   ? stream_kernel
      : design == KQB_PAIR ? stream_pair_kernel
      : design == KQB_RING ? stream_ring_kernel
      : design == KQB_READ ? stream_read_kernel
                           : stream_write_kernel;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint8_t*)x, (uint32_t)units, q, s);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int kq_bench_stream(const void* x, int64_t units, uint8_t* q, uint8_t* s, int grid,
                               void* stream) {
  return kq_bench_stream_design(x, units, q, s, grid, KQB_LANE, stream);
}
