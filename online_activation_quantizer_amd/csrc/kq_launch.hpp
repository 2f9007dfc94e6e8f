// kq_launch.hpp — host-side launch plumbing shared by the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

constexpr int kThreads = 256;             // threads per workgroup (4 wave64)
// Resident-grid target of the unit-per-lane kernels (3 workgroups = 12 waves per
// CU measured best on MI355X for 4608 x 3072 and 4608 x 12288), and how many rows
// ahead each lane's loads run (deeper rings measured no faster).
#ifndef KQ_BPCU
#define KQ_BPCU 3
#endif
constexpr int kBlocksPerCU = KQ_BPCU;
#ifndef KQ_DEPTH
#define KQ_DEPTH 1
#endif
constexpr int kRowDepth = KQ_DEPTH;

struct LaunchArgs {
  const void* x;
  int dtype;
  int64_t rows, d, nb, ldx;
  const void* t;  // params / expanded transform / SmoothQuant multipliers
  uint8_t* q;
  int64_t ldq;
  uint8_t* s;
  int64_t lds;
  float* y;  // optional fp32 pre-quantization output (validation entry points)
  int64_t ldy;
  void* stream;
  int cus;  // compute units of the current device
};

// Normalization-fused quantizer: the quantize arguments plus the modulation.
struct NormArgs {
  LaunchArgs a;
  const float* shift;  // [samples][d] or NULL (then scale is NULL too)
  const float* scale;
  int64_t rows_per_sample;
  float eps;
};
// Resident-grid target of the row-per-wave normalization kernel.
constexpr int kNormBlocksPerCU = 4;

// W4A4 product of two MXFP4 operands (codes + E8M0 scales, K along rows).
struct GemmArgs {
  const uint8_t* qa;
  int64_t lda;   // bytes
  const uint8_t* sa;
  int64_t ldsa;  // bytes
  const uint8_t* qb;
  int64_t ldb;
  const uint8_t* sb;
  int64_t ldsb;
  int64_t M, N, K;
  void* out;     // [M][ldo] float32 or bf16
  int64_t ldo;   // elements
  bool out_bf16;
  void* stream;
  int cus;       // compute units of the device (persistent grid size)
};

inline int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t r = a % b;
    a = b;
    b = r;
  }
  return a;
}

// Grid for the unit-per-lane kernels: the lane count (grid * kThreads) must be a
// multiple of nb so each lane keeps one block; aim for blocks_per_cu workgroups
// per compute unit but never more lanes than (row, block) units (rounded up to
// the next legal size).  *tstep receives the row stride of every lane.
inline int64_t grid_for_units(int64_t rows, int64_t nb, int cus, int blocks_per_cu,
                              uint32_t* tstep) {
  const int64_t m = nb / gcd64(nb, kThreads);  // grid granule
  const int64_t need = (rows * nb + kThreads - 1) / kThreads;
  int64_t target = (int64_t)cus * blocks_per_cu;
  if (target > need) target = need;
  int64_t k = (target + m - 1) / m;
  if (k < 1) k = 1;
  *tstep = (uint32_t)(k * m * kThreads / nb);
  return k * m;
}

hipError_t launch_butterfly(const LaunchArgs& a);
hipError_t launch_weights(const LaunchArgs& a);   // W T^-1 along each row, then MXFP4
hipError_t launch_hadamard(const LaunchArgs& a);  // fixed block-Hadamard, then MXFP4
hipError_t launch_norm(const NormArgs& n);        // LayerNorm + modulation, T_b, MXFP4
hipError_t launch_mx_gemm(const GemmArgs& g);    // Y = deq(A) deq(B)^T on scaled MFMA
hipError_t launch_sq(const LaunchArgs& a);
hipError_t launch_mfma(const LaunchArgs& a);
hipError_t launch_expand(const float* params, int64_t nb, int tfmt, void* out, void* stream);

}  // namespace kq
