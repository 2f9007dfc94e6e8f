// kq_butterfly.hip — in-register factored transform + MXFP4 encode (gfx950).
//
// One lane owns one (row, block) unit: the 32 channels of one block of one row.
// The block transform T_b = F1 (x) ... (x) F5 (KroQuant researchpod summary,
// method paragraph: Kronecker product of five 2x2 unit-determinant LU factors)
// is applied without ever forming the 32x32 matrix.  Each factor
//     F = L*U = [[1,0],[l,1]] * [[u,v],[0,1/u]]
// splits further into  F = L * S * D  with  S = [[1, u*v],[0,1]]  (a shear) and
// D = diag(u, 1/u).  By the mixed-product rule of the Kronecker product,
//     T_b = (L1 (x) .. (x) L5) (S1 (x) .. (x) S5) (D1 (x) .. (x) D5),
// and each of the three Kronecker products is a product of commuting one-bit
// operators.  So the kernel
//   1. multiplies channel i by d_i = prod_k (bit(4-k) of i ? 1/u_k : u_k)   (1 mul)
//   2. applies the five upper shears  x_p += (u_k v_k) x_q                 (5 x 16 fma)
//   3. applies the five lower shears  x_q += l_k x_p                       (5 x 16 fma)
// where p < q are the index pairs that differ in bit 4-k.  That is 6 fp32
// operations per element instead of 10 for the 2x2 butterfly and 64 for the
// dense product, and everything stays in VGPRs.
//
// The same kernel folds the inverse into a weight matrix W[N][d] (KroQuant
// abstract: the inverse transform goes to the weights).  Row r of W' = W T^-1 is
// w'_b = T_b^-T w_b, and with F^-T = L^-T U^-T = S'(-l) L'(-u v) diag(1/u, u),
// where S'(c) = [[1,c],[0,1]] and L'(c) = [[1,0],[c,1]], the same three Kronecker
// products give: multiply by 1/d_i, lower shears x_q += (-u_k v_k) x_p, then upper
// shears x_p += (-l_k) x_q.  Weight rows are quantized along d like activation rows.
//
// A third mode runs the fixed block-Hadamard comparison transform (KroQuant
// abstract: fixed Hadamard rotations are the accurate but costly alternative):
// five add/subtract stages (a, b) -> (a + b, a - b) over the same index pairs, then
// a multiply by fp32(1/sqrt(32)).  H/sqrt(32) is symmetric and orthogonal, so
// weights take the same transform.
//
// Lanes cover consecutive (row, block) units in memory order (a wave reads 4 KB
// contiguous per row step) and advance through the rows with a stride that is a
// multiple of nb, so every lane keeps one block for its whole life and computes
// its 42 constants (32 d_i, 5 upper and 5 lower shear coefficients) once: the
// block's 15 parameters are requested before the lane's first row and the
// constants are built while that row is in flight.
#include "kq_device.hpp"
#include "kq_factors.hpp"
#include "kq_launch.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

template <int DT, bool WRITE_Y, int MODE>
__global__ __launch_bounds__(kThreads) void butterfly_kernel(
    const uint8_t* __restrict__ x, uint32_t rows, uint32_t nb, uint32_t ldx, uint32_t tstep,
    const float* __restrict__ params, uint8_t* __restrict__ q, uint32_t ldq,
    uint8_t* __restrict__ s, uint32_t lds, float* __restrict__ y, uint32_t ldy) {
  // the lane count gridDim.x * kThreads is a multiple of nb (tstep rows per pass);
  // pitches are in bytes
  const uint32_t gtid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t b = gtid % nb;
  const uint32_t t = gtid / nb;
  if (t >= rows) return;
  BlockParams bp;
  BlockConsts c;
  uint8_t* const qcol = q + b * (kBlk / 2);
  uint8_t* const scol = s + b;
  uint8_t* const ycol = reinterpret_cast<uint8_t*>(y) + b * kBlk * 4;
  for_each_row<DT>(
      x + (size_t)b * kBlk * (DT == DT_BF16 ? 2 : 4), rows, ldx, t, tstep,
      [&] {
        if (MODE != kHadamard) bp = load_params(params, b);
      },
      [&] {
        // built while the first row is in flight (4608 x 3072: 8.24 -> 8.05 us against
        // parameters requested after the row)
        if (MODE != kHadamard) make_consts<MODE == kWeights>(bp, c);
      },
      [&](float (&v)[kBlk], uint32_t r) {
        if (MODE == kHadamard) hadamard(v);
        else transform<MODE == kWeights>(v, c);
        if (WRITE_Y) store_y(reinterpret_cast<float*>(ycol + (uint64_t)r * ldy), v);
        encode_store(v, qcol + (uint64_t)r * ldq, scol + (uint64_t)r * lds);
      });
}

template <int DT, bool WRITE_Y, int MODE>
hipError_t launch_t(const LaunchArgs& a) {
  uint32_t tstep = 0;
  const int64_t grid = grid_for_units(a.rows, a.nb, a.cus, kBlocksPerCU, &tstep);
  const int64_t esz = DT == DT_BF16 ? 2 : 4;
  hipLaunchKernelGGL((butterfly_kernel<DT, WRITE_Y, MODE>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint8_t*)a.x, (uint32_t)a.rows,
                     (uint32_t)a.nb, (uint32_t)(a.ldx * esz), tstep, (const float*)a.t, a.q,
                     (uint32_t)a.ldq, a.s, (uint32_t)a.lds, a.y, (uint32_t)(a.ldy * 4));
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const LaunchArgs& a) {
  if (a.dtype == DT_BF16)
    return a.y ? launch_t<DT_BF16, true, MODE>(a) : launch_t<DT_BF16, false, MODE>(a);
  return a.y ? launch_t<DT_FP32, true, MODE>(a) : launch_t<DT_FP32, false, MODE>(a);
}

}  // namespace

hipError_t launch_butterfly(const LaunchArgs& a) { return launch_mode<kForward>(a); }

hipError_t launch_weights(const LaunchArgs& a) { return launch_mode<kWeights>(a); }

hipError_t launch_hadamard(const LaunchArgs& a) { return launch_mode<kHadamard>(a); }

}  // namespace kq
