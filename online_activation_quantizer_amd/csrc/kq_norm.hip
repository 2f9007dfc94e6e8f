// kq_norm.hip — LayerNorm + adaptive-norm modulation fused ahead of the block
// transform and the MXFP4 encoder (gfx950).
//
// The normalization layers between DiT blocks are what force the transform to
// run online (KroQuant abstract); fusing them means the activations are read once,
// before normalization, instead of being normalized, written and read again.  Per
// row t:  mu and the biased variance over the d channels, rstd = 1/sqrt(var + eps),
//   h = (x - mu) * rstd * (1 + scale[g]) + shift[g],   g = t / rows_per_sample,
// then y_b = T_b h_b per 32-channel block and the MXFP4 encoding of y.
//
// One wave owns one row at a time (rows in a grid-stride loop).  Pass 1 reads the
// row (lane l takes blocks l, l + 64, ...) and computes each block's mean (pairwise
// sum) and sum of squared deviations from it; blocks, then lanes (a butterfly of
// lane exchanges), are merged with the pairwise update of Chan, Golub and LeVeque
// (count, mean, M2), which keeps the statistics accurate to a few ulps whatever
// the row's mean and outliers.  Pass 2 reads the row again (it was just read: the re-read is served by
// the cache, not by HBM), normalizes, modulates, applies the factored transform
// from the block's factors and encodes.  HBM traffic stays the quantizer's
// 2.53125 B per element (plus the modulation vectors, shared by all rows of a
// sample).
#include "kq_device.hpp"
#include "kq_factors.hpp"
#include "kq_launch.hpp"

namespace kq {
namespace {

// Running statistics of a set of values: count, mean, sum of squared deviations.
struct Moments {
  float n, mean, m2;
};

// Merge of two sets (Chan, Golub and LeVeque's pairwise update).
__device__ __forceinline__ Moments merge(const Moments& a, const Moments& b) {
  const float n = a.n + b.n;
  if (n == 0.0f) return a;
  const float delta = b.mean - a.mean;
  const float wb = b.n / n;
  return {n, __builtin_fmaf(delta, wb, a.mean), a.m2 + b.m2 + delta * delta * (a.n * wb)};
}

// Moments of one block's 32 values: pairwise sum for the mean, then the squared
// deviations from it.
__device__ __forceinline__ Moments block_moments(const float (&v)[kBlk]) {
  float t[kBlk / 2];
#pragma unroll
  for (int i = 0; i < kBlk / 2; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = kBlk / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  const float mean = t[0] * (1.0f / kBlk);
  float m2 = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    const float dv = v[i] - mean;
    m2 = __builtin_fmaf(dv, dv, m2);
  }
  return {(float)kBlk, mean, m2};
}

__device__ __forceinline__ Moments wave_merge(Moments m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const Moments o = {__shfl_xor(m.n, off), __shfl_xor(m.mean, off), __shfl_xor(m.m2, off)};
    // both lanes of a pair merge in the same order so they end with equal values
    m = (threadIdx.x & off) ? merge(o, m) : merge(m, o);
  }
  return m;
}

template <int DT, bool MOD, bool WRITE_Y>
__global__ __launch_bounds__(kThreads) void norm_kernel(
    const uint8_t* __restrict__ x, uint32_t rows, uint32_t nb, uint32_t ldx,
    const float* __restrict__ shift, const float* __restrict__ scale, uint32_t rows_per_sample,
    float eps, float inv_d, const float* __restrict__ params, uint8_t* __restrict__ q,
    uint32_t ldq, uint8_t* __restrict__ s, uint32_t lds, float* __restrict__ y, uint32_t ldy) {
  // pitches in bytes; one wave per row
  constexpr uint32_t kBlkBytes = kBlk * (DT == DT_BF16 ? 2 : 4);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  const uint64_t d = (uint64_t)nb * kBlk;
  for (uint32_t r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < rows; r += nwaves) {
    const uint8_t* xr = x + (uint64_t)r * ldx;
    Moments m = {0.0f, 0.0f, 0.0f};
    for (uint32_t b = lane; b < nb; b += 64) {
      float v[kBlk];
      unpack(load_raw<DT>(xr + (uint64_t)b * kBlkBytes), v);
      m = merge(m, block_moments(v));
    }
    m = wave_merge(m);
    const float mean = m.mean;
    const float var = m.m2 * inv_d;
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);
    const uint64_t g = r / rows_per_sample;
    for (uint32_t b = lane; b < nb; b += 64) {
      const BlockParams bp = load_params(params, b);
      float v[kBlk];
      unpack(load_raw<DT>(xr + (uint64_t)b * kBlkBytes), v);
      BlockConsts c;
      make_consts<false>(bp, c);
      if (MOD) {
        const float4* sc4 = reinterpret_cast<const float4*>(scale + g * d + (uint64_t)b * kBlk);
        const float4* sh4 = reinterpret_cast<const float4*>(shift + g * d + (uint64_t)b * kBlk);
#pragma unroll
        for (int k = 0; k < kBlk / 4; ++k) {
          const float4 a = sc4[k], o = sh4[k];
          const float av[4] = {a.x, a.y, a.z, a.w}, ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float hn = (v[4 * k + j] - mean) * rstd;
            v[4 * k + j] = __builtin_fmaf(hn, 1.0f + av[j], ov[j]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kBlk; ++i) v[i] = (v[i] - mean) * rstd;
      }
      transform<false>(v, c);
      if (WRITE_Y)
        store_y(reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(y) + (uint64_t)r * ldy) + b * kBlk, v);
      encode_store(v, q + (uint64_t)r * ldq + b * (kBlk / 2), s + (uint64_t)r * lds + b);
    }
  }
}

template <int DT, bool MOD, bool WRITE_Y>
hipError_t launch_t(const NormArgs& n) {
  const LaunchArgs& a = n.a;
  const int64_t waves_per_wg = kThreads / 64;
  int64_t grid = (int64_t)a.cus * kNormBlocksPerCU;
  const int64_t need = (a.rows + waves_per_wg - 1) / waves_per_wg;
  if (grid > need) grid = need;
  const int64_t esz = DT == DT_BF16 ? 2 : 4;
  hipLaunchKernelGGL((norm_kernel<DT, MOD, WRITE_Y>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint8_t*)a.x, (uint32_t)a.rows, (uint32_t)a.nb,
                     (uint32_t)(a.ldx * esz), n.shift, n.scale, (uint32_t)n.rows_per_sample, n.eps,
                     (float)(1.0 / (double)a.d), (const float*)a.t, a.q, (uint32_t)a.ldq, a.s,
                     (uint32_t)a.lds, a.y, (uint32_t)(a.ldy * 4));
  return hipGetLastError();
}

template <bool MOD>
hipError_t launch_mod(const NormArgs& n) {
  if (n.a.dtype == DT_BF16)
    return n.a.y ? launch_t<DT_BF16, MOD, true>(n) : launch_t<DT_BF16, MOD, false>(n);
  return n.a.y ? launch_t<DT_FP32, MOD, true>(n) : launch_t<DT_FP32, MOD, false>(n);
}

}  // namespace

hipError_t launch_norm(const NormArgs& n) {
  return n.shift ? launch_mod<true>(n) : launch_mod<false>(n);
}

}  // namespace kq
