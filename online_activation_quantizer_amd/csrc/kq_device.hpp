// kq_device.hpp — device helpers shared by the gfx950 quantizer kernels:
// block loads, the MXFP4 encoder (OCP MX v1.0: E8M0 scale from the block amax,
// E2M1 elements rounded to nearest even with saturation) and the packed stores.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

constexpr int kBlk = 32;  // channels per transform block and per MX block

enum : int { DT_BF16 = 0, DT_FP32 = 1 };

// Raw bytes of one 32-channel block: 64 B of bf16 or 128 B of fp32.
template <int DT> struct Raw;
template <> struct Raw<DT_BF16> { uint4 w[4]; };
template <> struct Raw<DT_FP32> { uint4 w[8]; };

template <int DT>
__device__ __forceinline__ Raw<DT> load_raw(const uint8_t* p) {
  Raw<DT> r;
  const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int k = 0; k < (int)(sizeof(r.w) / sizeof(uint4)); ++k) r.w[k] = v[k];
  return r;
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

// Row walker.  Lane-to-unit mapping is row-major: the grid's lanes cover
// consecutive (row, block) units, and since the lane count is a multiple of nb
// each lane keeps one block column and walks rows t, t + tstep, ... < rows,
// calling f(v, row) with the row's 32 values widened to fp32.  `xcol` points at
// the lane's block column in row 0 and `ldx` is the row pitch in bytes; row
// arithmetic is 32-bit, so every address is one multiply-add.
//  - `request` issues the loads of the lane's constants and runs first; `setup`
//    (their arithmetic) runs after the first row has been requested.  Vector loads
//    complete in the order they were issued, so constants requested after the row
//    could only be used once the row had arrived; requested before it, they are
//    built while the row is in flight.  Every lane runs both, also one whose first
//    row is past the end (its load is clamped in bounds), so a set-up may hold a
//    workgroup barrier.
//  - Each row is loaded, transformed and stored before the next row is requested:
//    a lane has 2-3 rows at the sizes of interest and the grid keeps 12 waves per
//    compute unit in flight, which covers the memory latency; a one-row prefetch
//    ring measured slower (its extra registers, and a re-read of the last row by
//    every lane whose rows ran out) on 4608 x 3072.
template <int DT, class R, class S, class F>
__device__ __forceinline__ void for_each_row(const uint8_t* __restrict__ xcol, uint32_t rows,
                                             uint32_t ldx, uint32_t t, uint32_t tstep, R&& request,
                                             S&& setup, F&& f) {
  const uint32_t last = rows - 1;
  request();
  Raw<DT> raw = load_raw<DT>(xcol + (uint64_t)(t < last ? t : last) * ldx);
  // keep the row's load ahead of the constants' arithmetic (which waits for their loads)
  __builtin_amdgcn_sched_barrier(0);
  setup();
  __builtin_amdgcn_sched_barrier(0);
  // lanes with no row (past the last unit) ran the set-up with the others, since it
  // may hold a workgroup barrier, and stop here
  if (t > last) return;
  for (;;) {
    float v[kBlk];
    unpack(raw, v);
    f(v, t);
    t += tstep;  // rows < 2^31 and tstep < 2^24: no wrap
    if (t > last) return;
    raw = load_raw<DT>(xcol + (uint64_t)t * ldx);
  }
}

// A wave-uniform value kept in a scalar register.
__device__ __forceinline__ float uniform(float v) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
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

// Encode 32 fp32 values as MXFP4: 16 code bytes into w (low nibble first) and
// the E8M0 scale byte as the result.  The hardware scaled convert divides by
// 2^(exponent field of its scale operand), rounds to nearest even, saturates at 6
// and keeps the sign of zero.  Blocks whose scale is tiny (byte < 25) are
// pre-multiplied by 2^64 (exact: their amax is below 2^-100) so that the convert
// never sees a subnormal scale or subnormal inputs.
__device__ __forceinline__ uint32_t encode(float (&y)[kBlk], uint32_t (&w)[4]) {
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
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t a = 0;
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 0], y[8 * k + 1], sc, 0);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 2], y[8 * k + 3], sc, 1);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 4], y[8 * k + 5], sc, 2);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, y[8 * k + 6], y[8 * k + 7], sc, 3);
    w[k] = S == 255u ? 0u : a;
  }
  return S;
}

// encode, then store the 16 code bytes at qp and the scale byte at sp.
__device__ __forceinline__ void encode_store(float (&y)[kBlk], uint8_t* __restrict__ qp,
                                             uint8_t* __restrict__ sp) {
  uint32_t w[4];
  const uint32_t S = encode(y, w);
  // streaming stores: the codes are consumed by a later kernel, not re-read here
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 wv = {w[0], w[1], w[2], w[3]};
  __builtin_nontemporal_store(wv, reinterpret_cast<u32x4*>(qp));
  __builtin_nontemporal_store((uint8_t)S, sp);
}

__device__ __forceinline__ void store_y(float* __restrict__ yp, const float (&y)[kBlk]) {
#pragma unroll
  for (int i = 0; i < kBlk; ++i) yp[i] = y[i];
}

}  // namespace kq
