// kq_factors.hpp — the factored block transform in registers (KroQuant
// researchpod summary, method paragraph: T_b is the Kronecker product of five
// 2x2 unit-determinant LU factors F = L U).  Each F = L S D with the shear
// S = [[1, u v],[0, 1]] and D = diag(u, 1/u); by the mixed-product rule T_b is the
// product of three Kronecker products of one-bit operators, applied as a
// per-channel diagonal, five upper shears and five lower shears.  The inverse
// transposed (weight side) and the fixed block-Hadamard comparison transform use
// the same index pairs.  Included by the kernels that need them.
#pragma once
#include "kq_device.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

struct BlockConsts {
  float d[kBlk];
  float su[5];  // u_k * v_k   (negated for the weight side)
  float ll[5];  // l_k         (negated for the weight side)
};

// The 15 factor parameters (l, u, v) x 5 of block b.
struct BlockParams {
  float p[15];
};

__device__ __forceinline__ BlockParams load_params(const float* __restrict__ params, uint32_t b) {
  BlockParams r;
  const float* src = params + (size_t)b * 15;
#pragma unroll
  for (int i = 0; i < 15; ++i) r.p[i] = src[i];
  return r;
}

// The 42 constants of a block from its parameters.  INV builds those of T_b^-T:
// the diagonal swaps u and 1/u, and both shear coefficients change sign.
template <bool INV>
__device__ __forceinline__ void make_consts(const BlockParams& bp, BlockConsts& c) {
  float d0[5], d1[5];  // the factor's diagonal entry for index bit 0 and bit 1
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const float l = bp.p[3 * k + 0], uk = bp.p[3 * k + 1], v = bp.p[3 * k + 2];
    const float iu = __builtin_amdgcn_rcpf(uk);  // within 1 ulp; exact for powers of two
    d0[k] = INV ? iu : uk;
    d1[k] = INV ? uk : iu;
    c.su[k] = INV ? -(uk * v) : uk * v;
    c.ll[k] = INV ? -l : l;
  }
  // d = [d0_1, d1_1] (x) [d0_2, d1_2] (x) ... (x) [d0_5, d1_5], built from the right.
  c.d[0] = d0[4];
  c.d[1] = d1[4];
#pragma unroll
  for (int k = 3, n = 2; k >= 0; --k, n *= 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < n) {
        c.d[n + i] = d1[k] * c.d[i];
        c.d[i] = d0[k] * c.d[i];
      }
    }
  }
}

// x_p += coef_k x_q over the pairs p < q that differ in index bit 4-k.
__device__ __forceinline__ void upper_shears(float (&v)[kBlk], const float (&coef)[5]) {
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int st = 16 >> k;
#pragma unroll
    for (int i = 0; i < kBlk; ++i)
      if (!(i & st)) v[i] = __builtin_fmaf(coef[k], v[i + st], v[i]);
  }
}

// x_q += coef_k x_p over the same pairs.
__device__ __forceinline__ void lower_shears(float (&v)[kBlk], const float (&coef)[5]) {
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int st = 16 >> k;
#pragma unroll
    for (int i = 0; i < kBlk; ++i)
      if (!(i & st)) v[i + st] = __builtin_fmaf(coef[k], v[i], v[i + st]);
  }
}

enum : int { kForward = 0, kWeights = 1, kHadamard = 2 };

// (a, b) -> (a + b, a - b) over the pairs of every index bit, then 1/sqrt(32).
__device__ __forceinline__ void hadamard(float (&v)[kBlk]) {
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int st = 16 >> k;
#pragma unroll
    for (int i = 0; i < kBlk; ++i)
      if (!(i & st)) {
        const float a = v[i], b = v[i + st];
        v[i] = a + b;
        v[i + st] = a - b;
      }
  }
#pragma unroll
  for (int i = 0; i < kBlk; ++i) v[i] *= 0.17677669529663687f;  // fp32(1/sqrt(32))
}

// T_b x (upper shears by u v, then lower by l) or, for INV, T_b^-T x (lower shears
// by -u v, then upper by -l), after the diagonal.
// The shear part alone (what follows the diagonal).
template <bool INV>
__device__ __forceinline__ void shears(float (&v)[kBlk], const BlockConsts& c) {
  if (INV) {
    lower_shears(v, c.su);
    upper_shears(v, c.ll);
  } else {
    upper_shears(v, c.su);
    lower_shears(v, c.ll);
  }
}

template <bool INV>
__device__ __forceinline__ void transform(float (&v)[kBlk], const BlockConsts& c) {
#pragma unroll
  for (int i = 0; i < kBlk; ++i) v[i] *= c.d[i];
  shears<INV>(v, c);
}

}  // namespace
}  // namespace kq
