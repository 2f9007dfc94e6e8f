// kq_sq.hip — SmoothQuant baseline on the same memory skeleton as the
// butterfly kernel: per-channel multiply y_c = x_c * mult_c (mult = 1/s_c, the
// per-channel smoothing the KroQuant abstract compares against), then the same
// MXFP4 encode and stores.  Each lane keeps its block's 32 multipliers in VGPRs
// (128 B per lane against the 60 B of factors the butterfly kernel reads: the
// parameter count difference the KroQuant abstract points out); a workgroup
// fetches its blocks' multipliers once into LDS and its lanes read them there.
#include "kq_device.hpp"
#include "kq_launch.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

template <int DT, bool WRITE_Y>
__global__ __launch_bounds__(kThreads) void sq_kernel(
    const uint8_t* __restrict__ x, uint32_t rows, uint32_t nb, uint32_t ldx, uint32_t tstep,
    const float* __restrict__ mult, uint8_t* __restrict__ q, uint32_t ldq,
    uint8_t* __restrict__ s, uint32_t lds, float* __restrict__ y, uint32_t ldy) {
  const uint32_t gtid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t b = gtid % nb;
  const uint32_t t = gtid / nb;  // lanes with t >= rows take part in the set-up only
  // the multipliers of the workgroup's blocks: its 256 lanes cover min(nb, 256)
  // consecutive blocks (mod nb) starting at b0
  __shared__ float4 sm[kThreads * 8];
  const uint32_t nblk = nb < (uint32_t)kThreads ? nb : (uint32_t)kThreads;
  const uint32_t b0 = nb <= (uint32_t)kThreads ? 0u : (blockIdx.x * kThreads) % nb;
  float m[kBlk];
  uint8_t* const qcol = q + b * (kBlk / 2);
  uint8_t* const scol = s + b;
  uint8_t* const ycol = reinterpret_cast<uint8_t*>(y) + b * kBlk * 4;
  const uint32_t n4 = nblk * 8u;
  // (a register-friendly vector type: an array of HIP's float4 struct shared by the
  // two set-up steps is kept in scratch memory)
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4 tmp[8];
  for_each_row<DT>(
      x + (size_t)b * kBlk * (DT == DT_BF16 ? 2 : 4), rows, ldx, t, tstep,
      [&] {
        // before the first row: the workgroup's multipliers, on their way to LDS (8
        // loads per thread; indices past the slice re-read its last chunk)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t f = threadIdx.x + kThreads * k;
          f = f < n4 ? f : n4 - 1u;
          uint32_t gb = b0 + f / 8u;
          gb = gb >= nb ? gb - nb : gb;
          tmp[k] = reinterpret_cast<const f32x4*>(mult)[(size_t)gb * 8u + (f & 7u)];
        }
      },
      [&] {
        // while the first row is in flight: the multipliers into LDS, one barrier, and
        // each lane reads its block's 32 (9.53 -> 9.18 us at 4608 x 3072 against 32
        // multipliers loaded by every lane)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t f = threadIdx.x + kThreads * k;
          if (f < n4) sm[f] = make_float4(tmp[k].x, tmp[k].y, tmp[k].z, tmp[k].w);
        }
        __syncthreads();
        // the lane's block in the slice: b itself when the workgroup covers every
        // block, else its offset from b0 (the lane's index, below 256)
        const uint32_t lb = nb <= (uint32_t)kThreads ? b : (b + nb - b0) % nb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float4 mr = sm[lb * 8u + k];
          m[4 * k] = mr.x;
          m[4 * k + 1] = mr.y;
          m[4 * k + 2] = mr.z;
          m[4 * k + 3] = mr.w;
        }
      },
      [&](float (&v)[kBlk], uint32_t r) {
#pragma unroll
        for (int i = 0; i < kBlk; ++i) v[i] *= m[i];
        if (WRITE_Y) store_y(reinterpret_cast<float*>(ycol + (uint64_t)r * ldy), v);
        encode_store(v, qcol + (uint64_t)r * ldq, scol + (uint64_t)r * lds);
      });
}

template <int DT, bool WRITE_Y>
hipError_t launch_t(const LaunchArgs& a) {
  uint32_t tstep = 0;
  const int64_t grid = grid_for_units(a.rows, a.nb, a.cus, kBlocksPerCU, &tstep);
  const int64_t esz = DT == DT_BF16 ? 2 : 4;
  hipLaunchKernelGGL((sq_kernel<DT, WRITE_Y>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint8_t*)a.x, (uint32_t)a.rows,
                     (uint32_t)a.nb, (uint32_t)(a.ldx * esz), tstep, (const float*)a.t, a.q,
                     (uint32_t)a.ldq, a.s, (uint32_t)a.lds, a.y, (uint32_t)(a.ldy * 4));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sq(const LaunchArgs& a) {
  if (a.dtype == DT_BF16) return a.y ? launch_t<DT_BF16, true>(a) : launch_t<DT_BF16, false>(a);
  return a.y ? launch_t<DT_FP32, true>(a) : launch_t<DT_FP32, false>(a);
}

}  // namespace kq
