// kq_device.hpp — device helpers shared by the gfx950 quantizer kernels:
// block loads, the MXFP4 encoder (OCP MX v1.0: E8M0 scale from the block amax,
// E2M1 elements rounded to nearest even with saturation) and the packed stores.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef KQ_NT_LOAD
#define KQ_NT_LOAD 0
#endif

namespace kq {

constexpr int kBlk = 32;  // channels per transform block and per MX block

enum : int { DT_BF16 = 0, DT_FP32 = 1 };

// Raw bytes of one 32-channel block: 64 B of bf16 or 128 B of fp32.
template <int DT> struct Raw;
template <> struct Raw<DT_BF16> { uint4 w[4]; };
template <> struct Raw<DT_FP32> { uint4 w[8]; };

template <int DT>
__device__ __forceinline__ Raw<DT> load_raw(const void* x, int64_t elem_off) {
  Raw<DT> r;
  const uint4* p = reinterpret_cast<const uint4*>(
      static_cast<const char*>(x) + elem_off * (DT == DT_BF16 ? 2 : 4));
#pragma unroll
  for (int k = 0; k < (int)(sizeof(r.w) / sizeof(uint4)); ++k) {
#if KQ_NT_LOAD
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + k));
    r.w[k] = make_uint4(v.x, v.y, v.z, v.w);
#else
    r.w[k] = p[k];
#endif
  }
  return r;
}

// Walk rows t, t + tstep, ... < rows of one lane's block column `col` (element
// offset), calling f(raw, row) for each.  Two-stage software pipeline: the next
// row's load is issued before the current row is processed.  The prefetch is
// unconditional (its row is clamped to the last row, an in-bounds re-read) so
// the compiler can keep exact counts of the loads in flight.
template <int DT, class F>
__device__ __forceinline__ void for_each_row(const void* __restrict__ x, int64_t rows, int64_t ldx,
                                             int64_t col, int64_t t, int64_t tstep, F&& f) {
  const int64_t last = rows - 1;
  Raw<DT> ra = load_raw<DT>(x, t * ldx + col);
  for (;;) {
    int64_t tn = t + tstep;
    Raw<DT> rb = load_raw<DT>(x, (tn < last ? tn : last) * ldx + col);
    f(ra, t);
    if (tn > last) return;
    t = tn;
    tn = t + tstep;
    ra = load_raw<DT>(x, (tn < last ? tn : last) * ldx + col);
    f(rb, t);
    if (tn > last) return;
    t = tn;
  }
}

#ifndef KQ_LDS_STAGE
#define KQ_LDS_STAGE 0
#endif

// LDS-staged walker for bf16 input (one wave = 64 consecutive units).  The wave
// loads its 4 KB with fully coalesced 16-byte lanes (lane l fetches chunk l%4 of
// unit 16k + l/4), parks the chunks in LDS (80-byte unit pitch: conflict-free
// reads) and each lane then reads back its own unit.  g is the lane's flat unit
// index; G (the grid's lane count) is a multiple of nb.  Every lane of the wave
// stays in the loop while the wave's first unit is in range.
template <class F>
__device__ __forceinline__ void for_each_row_lds(const void* __restrict__ x, int64_t rows,
                                                 int64_t ldx, int64_t nb, int64_t g, int64_t G,
                                                 uint4 (*__restrict__ wlds)[5], F&& f) {
  const int lane = threadIdx.x & 63;
  const int64_t u0 = g - lane;
  const int64_t tstep = G / nb;
  const int64_t last = rows - 1;
  int64_t rk[4], ck[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t uk = u0 + 16 * k + (lane >> 2);
    rk[k] = uk / nb;
    ck[k] = (uk % nb) * kBlk + (lane & 3) * 8;
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  int64_t t = g / nb;
  int64_t t0 = u0 / nb;
  for (; t0 <= last; t0 += tstep, t += tstep) {
    uint4 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = rk[k] < last ? rk[k] : last;
      c[k] = *reinterpret_cast<const uint4*>(xb + r * ldx + ck[k]);
      rk[k] += tstep;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) wlds[16 * k + (lane >> 2)][lane & 3] = c[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    Raw<DT_BF16> mine;
#pragma unroll
    for (int k = 0; k < 4; ++k) mine.w[k] = wlds[lane][k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t <= last) f(mine, t);
  }
}

// Widen to fp32.  bf16 is the top half of an fp32, so the widening is exact.
__device__ __forceinline__ void unpack(const Raw<DT_BF16>& r, float (&v)[kBlk]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w[4] = {r.w[k].x, r.w[k].y, r.w[k].z, r.w[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * k + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * k + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}
__device__ __forceinline__ void unpack(const Raw<DT_FP32>& r, float (&v)[kBlk]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[4 * k + 0] = __uint_as_float(r.w[k].x);
    v[4 * k + 1] = __uint_as_float(r.w[k].y);
    v[4 * k + 2] = __uint_as_float(r.w[k].z);
    v[4 * k + 3] = __uint_as_float(r.w[k].w);
  }
}

// NaN-propagating max of |a|, |b|, |c| (v_maximum3_f32 with abs modifiers).
__device__ __forceinline__ float amax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, __builtin_fabsf(b)),
                                       __builtin_fabsf(c));
}

// E8M0 byte of a block from its amax m >= 0:  e = floor(log2 m) - 2 clamped to
// [-127, 127], byte e + 127.  For a finite m with exponent field E this is
// max(E - 2, 0) (E <= 2 covers zero, subnormal and clamped amax); E == 255
// (NaN or Inf in the block) gives 0xFF.
__device__ __forceinline__ uint32_t e8m0_of_amax(float m) {
  const uint32_t E = __float_as_uint(m) >> 23;  // m >= 0 (or NaN): sign bit clear
  return E >= 255u ? 255u : (E > 2u ? E - 2u : 0u);
}

// Encode 32 fp32 values as MXFP4 and store 16 code bytes + 1 scale byte.
// The hardware scaled convert divides by 2^(exponent field of its scale
// operand), rounds to nearest even, saturates at 6 and keeps the sign of zero.
// Blocks whose scale is tiny (byte < 25) are pre-multiplied by 2^64 (exact:
// their amax is below 2^-100) so that the convert never sees a subnormal
// scale or subnormal inputs.
__device__ __forceinline__ void encode_store(float (&y)[kBlk], uint8_t* __restrict__ qp,
                                             uint8_t* __restrict__ sp) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlk; i += 2) m = amax3(m, y[i], y[i + 1]);
  const uint32_t S = e8m0_of_amax(m);
  uint32_t Sc = S;
  if (__builtin_expect(S < 25u, 0)) {
#pragma unroll
    for (int i = 0; i < kBlk; ++i) y[i] *= 0x1p64f;
    Sc = S + 64u;
  }
  const float sc = __uint_as_float(Sc << 23);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t a = 0;
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 0], y[8 * k + 1], sc, 0);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 2], y[8 * k + 3], sc, 1);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 4], y[8 * k + 5], sc, 2);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 6], y[8 * k + 7], sc, 3);
    w[k] = S == 255u ? 0u : a;
  }
  *reinterpret_cast<uint4*>(qp) = make_uint4(w[0], w[1], w[2], w[3]);
  *sp = (uint8_t)S;
}

__device__ __forceinline__ void store_y(float* __restrict__ yp, const float (&y)[kBlk]) {
#pragma unroll
  for (int i = 0; i < kBlk; ++i) yp[i] = y[i];
}

}  // namespace kq
