// kq_mfma.hip — matrix-core variant: the block transform as small GEMMs
// (KroQuant abstract: the block-local structure runs as small tensor-core GEMMs).
//
// For a 32-channel block b and 32 token rows, Y_b^T (32 channels x 32 tokens) =
// T_b (32x32) * X_b^T (32 x 32 tokens) on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  T_b is given as three bf16 parts hi + mid + lo that sum exactly
// to its fp32 entries (kq_expand_factors, KQ_T_DENSE_BF16X3); bf16 x bf16 products
// are exact in fp32, so the three-pass product carries fp32 accuracy in T.  The
// input must be bf16 (its values are exact MFMA operands).
//
// Operand layout of the 32x32x16 bf16 MFMA (wave64): lane l supplies 8 consecutive
// K values k = 8*(l/32) .. +7 of row (A) / column (B) l%32; the 16 fp32 results of
// lane l are column l%32, rows 8*g + 4*(l/32) + r (g, r = 0..3).  With A = T_b rows
// and B = token columns, each lane therefore holds 16 channels of one token, the
// other 16 sit in lane l^32: the block amax and the packed code bytes are completed
// with one cross-half exchange each.
//
// Each wave owns a pair of adjacent blocks (128 contiguous input bytes per token
// row) and keeps their 12 A operands in VGPRs while it walks 32-row tiles.
#include "kq_device.hpp"
#include "kq_launch.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaBlocksPerCU = 2;

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <bool WRITE_Y>
__device__ __forceinline__ void encode_tile(floatx16 acc, int h, bool store, uint8_t* qrow,
                                            uint8_t* srow, float* yrow) {
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) m = amax3(m, acc[r], acc[r + 1]);
  m = __builtin_elementwise_maximum(m, __shfl_xor(m, 32));
  if (WRITE_Y && store) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(yrow + 8 * g + 4 * h) =
          make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
  }
  const uint32_t S = e8m0_of_amax(m);
  uint32_t Sc = S;
  if (__builtin_expect(S < 25u, 0)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] *= 0x1p64f;
    Sc = S + 64u;
  }
  const float sc = __uint_as_float(Sc << 23);
  // lane half h holds channels 8g + 4h + (0..3): code bytes 4g + 2h and 4g + 2h + 1
  uint32_t w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[0], acc[1], sc, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[2], acc[3], sc, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[4], acc[5], sc, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[6], acc[7], sc, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[8], acc[9], sc, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[10], acc[11], sc, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[12], acc[13], sc, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[14], acc[15], sc, 3);
  if (S == 255u) w0 = w1 = 0u;
  // h = 0 holds bytes {0,1,4,5 | 8,9,12,13}, h = 1 holds {2,3,6,7 | 10,11,14,15}:
  // swap one word across halves so lane h stores bytes 8h .. 8h+7 contiguously.
  const uint32_t recv = (uint32_t)__shfl_xor((int)(h ? w0 : w1), 32);
  const uint32_t lo = h ? recv : w0, hi = h ? w1 : recv;
  const uint32_t o0 = (lo & 0xFFFFu) | (hi << 16);
  const uint32_t o1 = (lo >> 16) | (hi & 0xFFFF0000u);
  if (store) {
    *reinterpret_cast<uint2*>(qrow + 8 * h) = make_uint2(o0, o1);
    if (h == 0) *srow = (uint8_t)S;
  }
}

template <bool WRITE_Y>
__global__ __launch_bounds__(kThreads) void mfma_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t nb, int64_t ldx,
    const uint16_t* __restrict__ T3, uint8_t* __restrict__ q, int64_t ldq,
    uint8_t* __restrict__ s, int64_t lds, float* __restrict__ y, int64_t ldy, uint32_t tstep) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  // the wave count gridDim.x * 4 is a multiple of npair (tstep tiles per pass)
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t npair = (uint32_t)((nb + 1) / 2);
  const uint32_t pair = wave % npair;
  const int64_t ntiles = (rows + 31) / 32;
  int64_t tile = wave / npair;
  if (tile >= ntiles) return;

  const int64_t b0 = 2 * (int64_t)pair;
  const bool has2 = b0 + 1 < nb;
  int64_t bb[2] = {b0, has2 ? b0 + 1 : b0};

  // A operands: [block][split hi/mid/lo][K half]
  bf16x8 A[2][3][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        A[j][sp][kh] = load8(T3 + (sp * nb + bb[j]) * 1024 + n * 32 + 16 * kh + 8 * h);

  for (; tile < ntiles; tile += tstep) {
    const int64_t t = tile * 32 + n;
    const bool valid = t < rows;
    const int64_t tl = valid ? t : rows - 1;  // tail lanes re-read a valid row, store nothing
    bf16x8 B[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) B[j][kh] = load8(x + tl * ldx + 32 * bb[j] + 16 * kh + 8 * h);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      floatx16 acc = {};
      // smallest parts first
#pragma unroll
      for (int sp = 2; sp >= 0; --sp)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j][sp][kh], B[j][kh], acc, 0, 0, 0);
      const bool store = valid && (j == 0 || has2);
      encode_tile<WRITE_Y>(acc, h, store, q + t * ldq + 16 * bb[j], s + t * lds + bb[j],
                           WRITE_Y ? y + t * ldy + 32 * bb[j] : nullptr);
    }
  }
}

template <bool WRITE_Y>
hipError_t launch_t(const LaunchArgs& a) {
  const int64_t npair = (a.nb + 1) / 2;
  const int64_t waves_per_wg = kThreads / 64;
  const int64_t m = npair / gcd64(npair, waves_per_wg);  // grid granule
  const int64_t ntiles = (a.rows + 31) / 32;
  const int64_t need = (npair * ntiles + waves_per_wg - 1) / waves_per_wg;
  int64_t target = (int64_t)a.cus * kMfmaBlocksPerCU;
  if (target > need) target = need;
  int64_t k = (target + m - 1) / m;
  if (k < 1) k = 1;
  const uint32_t tstep = (uint32_t)(k * m * waves_per_wg / npair);
  hipLaunchKernelGGL((mfma_kernel<WRITE_Y>), dim3((unsigned)(k * m)), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.x, a.rows, a.nb, a.ldx,
                     (const uint16_t*)a.t, a.q, a.ldq, a.s, a.lds, a.y, a.ldy, tstep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const LaunchArgs& a) {
  return a.y ? launch_t<true>(a) : launch_t<false>(a);
}

}  // namespace kq
