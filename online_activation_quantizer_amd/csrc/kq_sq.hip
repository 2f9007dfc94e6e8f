// kq_sq.hip — SmoothQuant baseline on the same memory skeleton as the
// butterfly kernel: per-channel multiply y_c = x_c * mult_c (mult = 1/s_c, the
// per-channel smoothing the KroQuant abstract compares against), then the same
// MXFP4 encode and stores.  Each lane keeps its block's 32 multipliers in VGPRs
// (128 B per lane against the 60 B of factors the butterfly kernel reads: the
// parameter count difference the KroQuant abstract points out).
#include "kq_device.hpp"
#include "kq_launch.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

template <int DT, bool WRITE_Y>
__global__ __launch_bounds__(kThreads) void sq_kernel(
    const void* __restrict__ x, int64_t rows, uint32_t nb, int64_t ldx, uint32_t tstep,
    const float* __restrict__ mult, uint8_t* __restrict__ q, int64_t ldq,
    uint8_t* __restrict__ s, int64_t lds, float* __restrict__ y, int64_t ldy) {
  const uint32_t gtid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t b = gtid % nb;
  const int64_t t = gtid / nb;
  if (t >= rows) return;
  // multiplier loads first: they complete before the rows
  float4 mr[8];
  {
    const float4* mp = reinterpret_cast<const float4*>(mult + (size_t)b * kBlk);
#pragma unroll
    for (int k = 0; k < 8; ++k) mr[k] = mp[k];
  }
  __builtin_amdgcn_sched_barrier(0);
  float m[kBlk];
  for_each_row<DT, kRowDepth>(
      x, rows, ldx, b * kBlk, t, tstep,
      [&] {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          m[4 * k] = mr[k].x;
          m[4 * k + 1] = mr[k].y;
          m[4 * k + 2] = mr[k].z;
          m[4 * k + 3] = mr[k].w;
        }
      },
      [&](float (&v)[kBlk], int64_t r) {
#pragma unroll
        for (int i = 0; i < kBlk; ++i) v[i] *= m[i];
        if (WRITE_Y) store_y(y + r * ldy + b * kBlk, v);
        encode_store(v, q + r * ldq + b * (kBlk / 2), s + r * lds + b);
      });
}

template <int DT, bool WRITE_Y>
hipError_t launch_t(const LaunchArgs& a) {
  uint32_t tstep = 0;
  const int64_t grid = grid_for_units(a.rows, a.nb, a.cus, kBlocksPerCU, &tstep);
  hipLaunchKernelGGL((sq_kernel<DT, WRITE_Y>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)a.stream, a.x, a.rows, (uint32_t)a.nb, a.ldx, tstep,
                     (const float*)a.t, a.q, a.ldq, a.s, a.lds, a.y, a.ldy);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sq(const LaunchArgs& a) {
  if (a.dtype == DT_BF16) return a.y ? launch_t<DT_BF16, true>(a) : launch_t<DT_BF16, false>(a);
  return a.y ? launch_t<DT_FP32, true>(a) : launch_t<DT_FP32, false>(a);
}

}  // namespace kq
