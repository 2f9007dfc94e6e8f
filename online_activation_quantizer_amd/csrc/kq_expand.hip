// kq_expand.hip — expand factor parameters (l, u, v) into a dense 32x32 block
// transform T_b = F1 (x) F2 (x) F3 (x) F4 (x) F5 (KroQuant researchpod summary,
// method paragraph), with F = L*U = [[u, v], [l*u, l*v + 1/u]].  Entry (i, j) is the
// product over k of F_k[bit(4-k) of i][bit(4-k) of j], computed in fp32.
// The bf16x3 format additionally splits each fp32 entry into three bf16 parts
// hi + mid + lo that sum to it exactly, for the matrix-core variant.  The 2x2
// format writes the five factors F_k themselves, row-major.
#include "kq_device.hpp"
#include "kq_launch.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void expand_kernel(const float* __restrict__ params,
                                                          int64_t nb, void* __restrict__ out) {
  const int64_t b = blockIdx.x;
  const int e = blockIdx.y * kThreads + threadIdx.x;  // 0..1023
  const int i = e >> 5, j = e & 31;
  const float* p = params + b * 15;
  float t = 1.0f;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const float l = p[3 * k], u = p[3 * k + 1], v = p[3 * k + 2];
    const int r = (i >> (4 - k)) & 1, c = (j >> (4 - k)) & 1;
    const float f = r == 0 ? (c == 0 ? u : v) : (c == 0 ? l * u : l * v + 1.0f / u);
    t *= f;
  }
  const int64_t o = b * 1024 + e;
  if (FMT == 1) {
    static_cast<float*>(out)[o] = t;
  } else {
    uint16_t* h = static_cast<uint16_t*>(out);
    const uint16_t hi = bf16_rne_bits(t);
    const float r1 = t - __uint_as_float((uint32_t)hi << 16);
    const uint16_t mid = bf16_rne_bits(r1);
    const float r2 = r1 - __uint_as_float((uint32_t)mid << 16);
    const uint16_t lo = bf16_rne_bits(r2);
    h[o] = hi;
    h[nb * 1024 + o] = mid;
    h[2 * nb * 1024 + o] = lo;
  }
}

// One thread per (block, factor): F = L U = [[u, v], [l u, l v + 1/u]] (IEEE quotient).
__global__ __launch_bounds__(kThreads) void factors_kernel(const float* __restrict__ params,
                                                          int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // block * 5 + factor
  if (i >= n) return;
  const float l = params[3 * i], u = params[3 * i + 1], v = params[3 * i + 2];
  float4 f;
  f.x = u;
  f.y = v;
  f.z = l * u;
  f.w = l * v + 1.0f / u;
  reinterpret_cast<float4*>(out)[i] = f;
}

}  // namespace

hipError_t launch_expand(const float* params, int64_t nb, int tfmt, void* out, void* stream) {
  if (tfmt == 3) {
    const int64_t n = nb * 5;
    hipLaunchKernelGGL(factors_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, params, n, static_cast<float*>(out));
    return hipGetLastError();
  }
  const dim3 grid((unsigned)nb, 1024 / kThreads);
  if (tfmt == 1)
    hipLaunchKernelGGL((expand_kernel<1>), grid, dim3(kThreads), 0, (hipStream_t)stream, params,
                       nb, out);
  else
    hipLaunchKernelGGL((expand_kernel<2>), grid, dim3(kThreads), 0, (hipStream_t)stream, params,
                       nb, out);
  return hipGetLastError();
}

}  // namespace kq
