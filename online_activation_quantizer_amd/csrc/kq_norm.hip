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
// Mapping.  A row is handled by H = ceil(nb / 32) half waves, one lane per block
// (lanes past nb idle), and a workgroup holds R = max(1, 256 / 32H) row slots
// packed back to back, so every lane keeps one block for the whole kernel.  Each
// lane carries two rows at a time, slot s of rows rbase + s and rbase + R + s, and
// walks on with a stride of 2R x gridDim.x: the two rows' reductions share their
// LDS round trips and barriers, and their arithmetic fills each other's waits.
// The lane's factors and shift are requested before its first rows (vector loads
// complete in issue order, so constants requested after the rows could only be
// built once the rows had arrived), and each pair of rows is loaded after the
// previous pair is stored.
//
// Statistics, in two passes over the rows held in registers: the row sum (each
// lane's block by pairwise addition, the 32 lanes of a half wave by a butterfly of
// lane exchanges, the H half-wave partials of a row through LDS in a fixed order)
// gives the mean; then the same reduction of the squared deviations from it gives
// the variance.  Deterministic, and accurate whatever the row's mean; the
// deviations are reused as the transform's input.
//
// Arithmetic.  With T_b = (kron L)(kron S) diag(d) and h = n * a + sh, where
// n = (x - mu) * rstd and a = 1 + scale:
//     y = rstd * (kron L)(kron S) diag(d * a) (x - mu) + T_b sh,
// so the modulation folds into the transform's diagonal (e = d * a) and a constant
// c = T_b sh, both computed once per lane and sample.  Per element that is one
// subtraction more and one fma (y = rstd * z + c) than the quantizer alone.
//
// Traffic: the quantizer's 2.53125 B per element plus the modulation vectors,
// read once per lane and sample.
#include "kq_device.hpp"
#include "kq_factors.hpp"
#include "kq_launch.hpp"

namespace kq {
namespace {

// Pairwise sum of one block's 32 values.
__device__ __forceinline__ float block_sum(const float (&v)[kBlk]) {
  float t[kBlk / 2];
#pragma unroll
  for (int i = 0; i < kBlk / 2; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = kBlk / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// v + the value DPP control CTRL moves into this lane (quad permutations and row
// mirrors within rows of 16 lanes, a row's last lane broadcast to the next row);
// rows outside ROW_MASK keep v.  One v_add_f32_dpp.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                  ROW_MASK, 0xF, false));
}

// Sum over the 32 lanes of a half wave: exchanges with the partner lane in the quad
// (xor 1, xor 2) and the mirrored lane in the half row and in the row leave every
// lane of a row with the row's total; the first row's total is then added into the
// second row (row broadcast), and lane 31 (63) holds the half wave's total, which
// every lane of that half reads.  One summation order for all 32 lanes.
__device__ __forceinline__ float half_sum(float v) {
  v = add_dpp<0xB1>(v);         // quad_perm [1,0,3,2]
  v = add_dpp<0x4E>(v);         // quad_perm [2,3,0,1]
  v = add_dpp<0x141>(v);        // row_half_mirror
  v = add_dpp<0x140>(v);        // row_mirror
  v = add_dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  return (threadIdx.x & 32u) ? t1 : t0;
}

constexpr uint32_t kMaxNormHalves = 16;  // half waves per workgroup (512 threads: d <= 16384)

template <int DT, bool MOD, bool WRITE_Y>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void norm_kernel(
    const uint8_t* __restrict__ x, uint32_t rows, uint32_t nb, uint32_t ldx,
    const float* __restrict__ shift, const float* __restrict__ scale, uint32_t rows_per_sample,
    float eps, float inv_d, const float* __restrict__ params, uint8_t* __restrict__ q,
    uint32_t ldq, uint8_t* __restrict__ s, uint32_t lds, float* __restrict__ y, uint32_t ldy,
    uint32_t H, uint32_t R) {
  // pitches in bytes; a row takes H half waves (32 H >= nb lanes), R row slots per
  // workgroup, blockDim.x = 32 H R rounded up to whole waves
  constexpr uint32_t kBlkBytes = kBlk * (DT == DT_BF16 ? 2 : 4);
  const uint32_t L = 32u * H;
  const uint32_t half = threadIdx.x >> 5;
  const uint32_t slot0 = threadIdx.x / L, b = threadIdx.x - slot0 * L;
  const bool active = slot0 < R && b < nb;
  const uint32_t slot = slot0 < R ? slot0 : R - 1;
  const uint32_t bb = b < nb ? b : nb - 1;  // idle lanes shadow a real block, store nothing
  const uint32_t last = rows - 1;
  const uint64_t d = (uint64_t)nb * kBlk;
  const uint8_t* const xcol = x + (uint64_t)bb * kBlkBytes;

  // half-wave partials of the two rows, two buffers (consecutive reductions
  // alternate, so a fast wave never overwrites partials a slow one still reads)
  __shared__ float part[2][2 * kMaxNormHalves];
  // the lane's rows: rbase + slot and rbase + R + slot, rbase advancing by 2R x
  // gridDim.x; the workgroup iterates while its first row exists, so every wave
  // reaches every barrier (rows past the end are clamped and not stored)
  uint32_t rbase = blockIdx.x * 2u * R;
  if (rbase > last) return;  // uniform over the workgroup
  const uint32_t rstep = gridDim.x * 2u * R;
  auto row_ptr = [&](uint32_t r) { return xcol + (uint64_t)(r < last ? r : last) * ldx; };
  // per-lane constants: shear coefficients, the modulated diagonal e and c = T_b shift
  // (rebuilt from the factors whenever the lane's row moves to another sample)
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  BlockConsts k;
  float cvec[kBlk];
  uint64_t cur_g = ~0ull;
  BlockParams bp;
  // the sample's factors and shift (straight into cvec), requested ...
  auto request_sample = [&](uint64_t g) {
    bp = load_params(params, bb);
    if (MOD) {
      const f32x4* o4 = reinterpret_cast<const f32x4*>(shift + g * d + (uint64_t)bb * kBlk);
#pragma unroll
      for (int j = 0; j < kBlk / 4; ++j) {
        const f32x4 o = o4[j];
        cvec[4 * j + 0] = o.x;
        cvec[4 * j + 1] = o.y;
        cvec[4 * j + 2] = o.z;
        cvec[4 * j + 3] = o.w;
      }
    }
  };
  // ... then turned into the constants; the scale is read four values at a time
  auto build_sample = [&](uint64_t g) {
    make_consts<false>(bp, k);
    if (MOD) {
      transform<false>(cvec, k);  // c = T_b shift, with the unmodulated diagonal
      const f32x4* a4 = reinterpret_cast<const f32x4*>(scale + g * d + (uint64_t)bb * kBlk);
#pragma unroll
      for (int j = 0; j < kBlk / 4; ++j) {
        const f32x4 a = a4[j];
        k.d[4 * j + 0] *= 1.0f + a.x;
        k.d[4 * j + 1] *= 1.0f + a.y;
        k.d[4 * j + 2] *= 1.0f + a.z;
        k.d[4 * j + 3] *= 1.0f + a.w;
      }
    }
    cur_g = g;
  };
  auto set_sample = [&](uint64_t g) {
    request_sample(g);
    build_sample(g);
  };
  {
    const uint32_t r0 = rbase + slot;
    request_sample(MOD ? (uint64_t)(r0 < last ? r0 : last) / rows_per_sample : 0);
  }
  Raw<DT> ringA = load_raw<DT>(row_ptr(rbase + slot));
  Raw<DT> ringB = load_raw<DT>(row_ptr(rbase + R + slot));
  // the constants are built while the first rows are in flight (4608 x 3072: 14.7 ->
  // 14.5 us with the pair loads moved after the stores)
  __builtin_amdgcn_sched_barrier(0);
  {
    const uint32_t r0 = rbase + slot;
    build_sample(MOD ? (uint64_t)(r0 < last ? r0 : last) / rows_per_sample : 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  int buf = 0;
  // row sums of both rows: each half wave's, then the row's half waves in a fixed
  // order through LDS
  auto row_sum2 = [&](float& ta, float& tb) {
    ta = half_sum(active ? ta : 0.0f);
    tb = half_sum(active ? tb : 0.0f);
    if (H > 1) {
      if ((threadIdx.x & 31u) == 0) {
        part[buf][half] = ta;
        part[buf][kMaxNormHalves + half] = tb;
      }
      __syncthreads();
      const uint32_t h0 = slot * H;
      ta = part[buf][h0];
      tb = part[buf][kMaxNormHalves + h0];
      for (uint32_t i = h0 + 1; i < h0 + H; ++i) {
        ta += part[buf][i];
        tb += part[buf][kMaxNormHalves + i];
      }
      buf ^= 1;
    }
  };
  // the transform, rstd and the modulation constant, then the encoder
  auto finish = [&](float (&v)[kBlk], float rstd, uint32_t r, bool store) {
#pragma unroll
    for (int i = 0; i < kBlk; ++i) v[i] *= k.d[i];
    shears<false>(v, k);
    if (MOD) {
#pragma unroll
      for (int i = 0; i < kBlk; ++i) v[i] = __builtin_fmaf(rstd, v[i], cvec[i]);
    } else {
#pragma unroll
      for (int i = 0; i < kBlk; ++i) v[i] *= rstd;
    }
    if (store) {
      if (WRITE_Y)
        store_y(reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(y) + (uint64_t)r * ldy) + b * kBlk, v);
      encode_store(v, q + (uint64_t)r * ldq + b * (kBlk / 2), s + (uint64_t)r * lds + b);
    }
  };

  for (;;) {
    const uint32_t ra = rbase + slot, rb = rbase + R + slot;
    const uint32_t raa = ra < last ? ra : last, rbb = rb < last ? rb : last;
    const bool storeA = active && ra <= last, storeB = active && rb <= last;
    const uint64_t ga = MOD ? raa / rows_per_sample : 0, gb = MOD ? rbb / rows_per_sample : 0;
    float va[kBlk], vb[kBlk];
    unpack(ringA, va);
    unpack(ringB, vb);
    const uint32_t rnext = rbase + rstep;
    // statistics of both rows first (no per-sample constants involved), then each
    // row's transform with its sample's constants
    float sa = block_sum(va), sb = block_sum(vb);
    row_sum2(sa, sb);
    const float ma = sa * inv_d, mb = sb * inv_d;
    float m2a = 0.0f, m2b = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      va[i] -= ma;
      m2a = __builtin_fmaf(va[i], va[i], m2a);
      vb[i] -= mb;
      m2b = __builtin_fmaf(vb[i], vb[i], m2b);
    }
    row_sum2(m2a, m2b);
    const float rsa = __builtin_amdgcn_rsqf(m2a * inv_d + eps);
    const float rsb = __builtin_amdgcn_rsqf(m2b * inv_d + eps);
    if (ga != cur_g) set_sample(ga);
    finish(va, rsa, ra, storeA);
    if (gb != cur_g) set_sample(gb);
    finish(vb, rsb, rb, storeB);
    if (rnext > last) return;  // uniform over the workgroup
    rbase = rnext;
    ringA = load_raw<DT>(row_ptr(rbase + slot));
    ringB = load_raw<DT>(row_ptr(rbase + R + slot));
  }
}

// Half wave per row (bf16 rows of at most 32 KB blocks, KB <= 4: d <= 4096).  Each
// half wave of 32 lanes takes one row, lane l the blocks l, l + 32, ... (KB of them,
// past nb idle), so both reductions of a row are 5 lane exchanges and a read of one
// lane, with no LDS and no barrier; a workgroup of 4 waves holds 8 rows.  The
// per-block constants (the diagonal times 1 + scale, the shear coefficients and
// c = T_b shift) are built once per workgroup and sample into LDS, at the top of
// the sample's first pass, and every lane reads its blocks' from there: 42 + 32
// constants per block cost no registers between rows.  At d = 3072 the kernel needs
// 165 VGPRs, three waves per SIMD (4608 x 3072: 14.6 -> 13.8 us against the LDS
// meeting of half waves).  Building the constants while the rows are in flight
// keeps more registers live than three waves per SIMD allow (185-215 VGPRs,
// 14.6-17.1 us, in every order tried), and widening the rows again in each pass to
// reach four waves per SIMD (124 VGPRs) costs more VALU than it hides (15.3 us).
constexpr int kHwRows = 8;                 // rows per workgroup pass (one per half wave)
constexpr int kHwMaxBlocks = 128;          // d <= 4096
constexpr int kHwStride = 76;              // floats per block in LDS: e[32] su[5] ll[5] . . c[32] . .

template <bool MOD, bool WRITE_Y, int KB>
__global__ __launch_bounds__(256) void norm_hw_kernel(
    const uint8_t* __restrict__ x, uint32_t rows, uint32_t nb, uint32_t ldx,
    const float* __restrict__ shift, const float* __restrict__ scale, uint32_t rows_per_sample,
    float eps, float inv_d, const float* __restrict__ params, uint8_t* __restrict__ q,
    uint32_t ldq, uint8_t* __restrict__ s, uint32_t lds, float* __restrict__ y, uint32_t ldy) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) float cs[kHwMaxBlocks * kHwStride];
  const uint32_t hw = threadIdx.x >> 5, l = threadIdx.x & 31u;
  const uint64_t d = (uint64_t)nb * kBlk;
  // the sample whose constants are in LDS (none yet)
  uint64_t cur_g = ~0ull;
  // the constants of sample g for every block, by the workgroup's lanes
  auto build = [&](uint64_t g) {
    for (uint32_t b = threadIdx.x; b < nb; b += blockDim.x) {
      BlockParams bp = load_params(params, b);
      BlockConsts k;
      make_consts<false>(bp, k);
      float* dst = cs + b * kHwStride;
      if (MOD) {
        float cv[kBlk];
        const f32x4* o4 = reinterpret_cast<const f32x4*>(shift + g * d + (uint64_t)b * kBlk);
#pragma unroll
        for (int j = 0; j < kBlk / 4; ++j) {
          const f32x4 o = o4[j];
          cv[4 * j] = o.x;
          cv[4 * j + 1] = o.y;
          cv[4 * j + 2] = o.z;
          cv[4 * j + 3] = o.w;
        }
        transform<false>(cv, k);  // c = T_b shift, with the unmodulated diagonal
        const f32x4* a4 = reinterpret_cast<const f32x4*>(scale + g * d + (uint64_t)b * kBlk);
#pragma unroll
        for (int j = 0; j < kBlk / 4; ++j) {
          const f32x4 a = a4[j];
          k.d[4 * j] *= 1.0f + a.x;
          k.d[4 * j + 1] *= 1.0f + a.y;
          k.d[4 * j + 2] *= 1.0f + a.z;
          k.d[4 * j + 3] *= 1.0f + a.w;
        }
#pragma unroll
        for (int i = 0; i < kBlk; ++i) dst[44 + i] = cv[i];
      }
#pragma unroll
      for (int i = 0; i < kBlk; ++i) dst[i] = k.d[i];
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        dst[kBlk + j] = k.su[j];
        dst[kBlk + 5 + j] = k.ll[j];
      }
    }
    cur_g = g;
  };

  // Passes of up to 8 rows of one sample: pass i is chunk i % chunks of sample
  // i / chunks (chunks = ceil(rows_per_sample / 8); without modulation, one sample
  // of all rows), so a sample's constants are built once per workgroup and
  // sample, at the top of its first pass.
  const uint32_t rps = MOD && rows_per_sample < rows ? rows_per_sample : rows;
  const uint32_t chunks = (rps + kHwRows - 1) / kHwRows;
  const uint32_t samples = (rows + rps - 1) / rps;
  const uint64_t passes = (uint64_t)samples * chunks;
  for (uint64_t pi = blockIdx.x; pi < passes; pi += gridDim.x) {
    const uint64_t g = pi / chunks;
    const uint32_t row0 = (uint32_t)(g * rps + (pi % chunks) * kHwRows);
    const uint64_t send = (g + 1) * rps;
    const uint32_t rend = send < rows ? (uint32_t)send : rows;  // the pass's rows: [row0, rend)
    if (g != cur_g) {
      __syncthreads();  // every wave past its reads of the previous sample's constants
      build(g);
      __syncthreads();
    }
    // this half wave's row (past the pass: its first row again, not stored) and its
    // blocks' raw bytes, all requested first
    const uint32_t r = row0 + hw;
    const bool row_ok = r < rend;
    const uint32_t rr = row_ok ? r : row0;
    Raw<DT_BF16> raw[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const uint32_t j = l + 32u * k, jj = j < nb ? j : nb - 1u;
      raw[k] = load_raw<DT_BF16>(x + (uint64_t)rr * ldx + (uint64_t)jj * (kBlk * 2));
    }
    // the mean: each lane's blocks by pairwise sums, in block order, then the half
    // wave's 32 lanes
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      float v[kBlk];
      unpack(raw[k], v);
      const float bs = block_sum(v);
      sum += l + 32u * k < nb ? bs : 0.0f;
    }
    const float mu = half_sum(sum) * inv_d;
    // the variance: squared deviations from the mean, the same way
    float m2 = 0.0f;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      float v[kBlk];
      unpack(raw[k], v);
      float bm = 0.0f;
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        const float dv = v[i] - mu;
        bm = __builtin_fmaf(dv, dv, bm);
      }
      m2 += l + 32u * k < nb ? bm : 0.0f;
    }
    const float rstd = __builtin_amdgcn_rsqf(half_sum(m2) * inv_d + eps);
    if (!row_ok) continue;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const uint32_t j = l + 32u * k;
      if (j >= nb) continue;
      float v[kBlk];
      unpack(raw[k], v);
      const f32x4* c4 = reinterpret_cast<const f32x4*>(cs + j * kHwStride);
#pragma unroll
      for (int i = 0; i < kBlk / 4; ++i) {
        const f32x4 e = c4[i];
        v[4 * i] = (v[4 * i] - mu) * e.x;
        v[4 * i + 1] = (v[4 * i + 1] - mu) * e.y;
        v[4 * i + 2] = (v[4 * i + 2] - mu) * e.z;
        v[4 * i + 3] = (v[4 * i + 3] - mu) * e.w;
      }
      BlockConsts k2;
      const f32x4 sa = c4[8], sbq = c4[9], sc2 = c4[10];
      const float sh[12] = {sa.x, sa.y, sa.z, sa.w, sbq.x, sbq.y, sbq.z, sbq.w, sc2.x, sc2.y, sc2.z, sc2.w};
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        k2.su[i] = sh[i];
        k2.ll[i] = sh[5 + i];
      }
      shears<false>(v, k2);
      if (MOD) {
#pragma unroll
        for (int i = 0; i < kBlk / 4; ++i) {
          const f32x4 c = c4[11 + i];
          v[4 * i] = __builtin_fmaf(rstd, v[4 * i], c.x);
          v[4 * i + 1] = __builtin_fmaf(rstd, v[4 * i + 1], c.y);
          v[4 * i + 2] = __builtin_fmaf(rstd, v[4 * i + 2], c.z);
          v[4 * i + 3] = __builtin_fmaf(rstd, v[4 * i + 3], c.w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kBlk; ++i) v[i] *= rstd;
      }
      if (WRITE_Y)
        store_y(reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(y) + (uint64_t)r * ldy) + j * kBlk, v);
      encode_store(v, q + (uint64_t)r * ldq + j * (kBlk / 2), s + (uint64_t)r * lds + j);
    }
  }
}

template <bool MOD, bool WRITE_Y, int KB>
hipError_t launch_hw_t(const NormArgs& n) {
  const LaunchArgs& a = n.a;
  const int64_t rps = MOD && n.rows_per_sample < a.rows ? n.rows_per_sample : a.rows;
  const int64_t groups = (a.rows + rps - 1) / rps * ((rps + kHwRows - 1) / kHwRows);  // passes
  int64_t grid = (int64_t)a.cus * 3;  // 3 waves per SIMD at d <= 3072 (165 VGPRs; LDS 39 KB)
  if (grid > groups) grid = groups;
  hipLaunchKernelGGL((norm_hw_kernel<MOD, WRITE_Y, KB>), dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)a.stream, (const uint8_t*)a.x, (uint32_t)a.rows, (uint32_t)a.nb,
                     (uint32_t)(a.ldx * 2), n.shift, n.scale, (uint32_t)n.rows_per_sample, n.eps,
                     (float)(1.0 / (double)a.d), (const float*)a.t, a.q, (uint32_t)a.ldq, a.s,
                     (uint32_t)a.lds, a.y, (uint32_t)(a.ldy * 4));
  return hipGetLastError();
}

template <bool MOD, bool WRITE_Y>
hipError_t launch_hw(const NormArgs& n) {
  const int64_t kb = (n.a.nb + 31) / 32;
  if (kb <= 1) return launch_hw_t<MOD, WRITE_Y, 1>(n);
  if (kb == 2) return launch_hw_t<MOD, WRITE_Y, 2>(n);
  if (kb == 3) return launch_hw_t<MOD, WRITE_Y, 3>(n);
  return launch_hw_t<MOD, WRITE_Y, 4>(n);
}

template <int DT, bool MOD, bool WRITE_Y>
hipError_t launch_t(const NormArgs& n) {
  const LaunchArgs& a = n.a;
  const int64_t H = (a.nb + 31) / 32;
  int64_t R = 256 / (32 * H);
  if (R < 1) R = 1;
  const int64_t threads = (32 * H * R + 63) / 64 * 64;
  // the resident waves per compute unit the register budget allows (2 per SIMD)
  int64_t per_cu = 8 / (threads / 64);
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)a.cus * per_cu;
  const int64_t groups = (a.rows + 2 * R - 1) / (2 * R);  // 2R rows per workgroup pass
  if (grid > groups) grid = groups;
  const int64_t esz = DT == DT_BF16 ? 2 : 4;
  hipLaunchKernelGGL((norm_kernel<DT, MOD, WRITE_Y>), dim3((unsigned)grid), dim3((unsigned)threads),
                     0, (hipStream_t)a.stream, (const uint8_t*)a.x, (uint32_t)a.rows,
                     (uint32_t)a.nb, (uint32_t)(a.ldx * esz), n.shift, n.scale,
                     (uint32_t)n.rows_per_sample, n.eps, (float)(1.0 / (double)a.d),
                     (const float*)a.t, a.q, (uint32_t)a.ldq, a.s, (uint32_t)a.lds, a.y,
                     (uint32_t)(a.ldy * 4), (uint32_t)H, (uint32_t)R);
  return hipGetLastError();
}

template <bool MOD>
hipError_t launch_mod(const NormArgs& n) {
  // bf16 rows of up to 4096 channels: a half wave per row; wider or fp32 rows: the
  // half waves of a row meet through LDS
  if (n.a.dtype == DT_BF16 && n.a.nb <= kHwMaxBlocks)
    return n.a.y ? launch_hw<MOD, true>(n) : launch_hw<MOD, false>(n);
  if (n.a.dtype == DT_BF16)
    return n.a.y ? launch_t<DT_BF16, MOD, true>(n) : launch_t<DT_BF16, MOD, false>(n);
  return n.a.y ? launch_t<DT_FP32, MOD, true>(n) : launch_t<DT_FP32, MOD, false>(n);
}

}  // namespace

hipError_t launch_norm(const NormArgs& n) {
  return n.shift ? launch_mod<true>(n) : launch_mod<false>(n);
}

}  // namespace kq
