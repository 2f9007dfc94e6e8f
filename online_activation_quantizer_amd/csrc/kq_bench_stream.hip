// kq_bench_stream.hip — the quantizer's memory traffic without its arithmetic
// (64 B read, 17 B written per 32-element bf16 unit), for the practical HBM
// ceiling reported beside the quantizer's time.  Declared in include/kq_bench.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_bench.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_kernel(const uint4* __restrict__ x,
                                                          uint32_t units,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t lanes = gridDim.x * kThreads;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += lanes) {
    const uint4* p = x + (uint64_t)u * 4;
    const uint4 a = p[0], b = p[1], c = p[2], d = p[3];
    const u32x4 w = {a.x ^ b.x ^ c.x ^ d.x, a.y ^ b.y ^ c.y ^ d.y, a.z ^ b.z ^ c.z ^ d.z,
                     a.w ^ b.w ^ c.w ^ d.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(q + (uint64_t)u * 16));
    __builtin_nontemporal_store((uint8_t)(w.x ^ w.y ^ w.z ^ w.w), s + u);
  }
}

}  // namespace

extern "C" int kq_bench_stream(const void* x, int64_t units, uint8_t* q, uint8_t* s, int grid,
                               void* stream) {
  if (units < 0 || units >= (int64_t(1) << 31) || grid < 1 || grid > 65535) return -2;
  if (units == 0) return 0;
  if (!x || !q || !s) return -1;
  if (((uintptr_t)x & 15) || ((uintptr_t)q & 15)) return -3;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4*)x, (uint32_t)units, q, s);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
