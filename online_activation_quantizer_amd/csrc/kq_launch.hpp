// kq_launch.hpp — host-side launch plumbing shared by the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

constexpr int kThreads = 256;             // threads per workgroup (4 wave64)
// Resident-grid target of the unit-per-lane kernels (3 workgroups = 12 waves per
// CU measured best on MI355X for 4608 x 3072: 2, 4 and 6 were slower).
#ifndef KQ_BPCU
#define KQ_BPCU 3
#endif
constexpr int kBlocksPerCU = KQ_BPCU;

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
  // device workspace for tiles split in K parts (flags first, zero between calls),
  // or NULL for whole tiles only; tiles are split only as far as it holds their
  // parts (all of mx_gemm_workspace_bytes() when it holds that much)
  void* workspace = nullptr;
  int64_t workspace_bytes = 0;
};

// Workspace of the W4A4 product's split tiles: kSplitFlagBytes of flags (one
// 32-bit word per split tile, zero between calls), then one 256 x 256 fp32 tile of
// partial sums (a slot) per K part of every split tile.
constexpr int64_t kSplitFlagBytes = 4096;
constexpr int64_t kSplitMaxTiles = kSplitFlagBytes / 4;
constexpr int64_t kSplitTileBytes = 256 * 256 * 4;

// The library's own split workspace for callers that cannot allocate: a static
// device array of kStaticScratchBytes on every device the library runs on (flags,
// then kStaticSplitTiles slots of partial sums: on a device of 256 compute units,
// every split schedule of two parts fits, and more parts as far as they fit).
constexpr int64_t kStaticSplitTiles = 128;
constexpr int64_t kStaticScratchBytes = kSplitFlagBytes + kStaticSplitTiles * kSplitTileBytes;
// Device address of the current device's static workspace (set up on its first
// use: looked up once, flags cleared by a kernel on `stream`).
hipError_t static_scratch(void** ptr, void* stream);

// The W4A4 product with the quantizer in its prologue: X bf16 [M][ldx] and its
// factor parameters [K/32][15] in place of the activations' MXFP4 operand.
struct FusedGemmArgs {
  const void* x;
  int64_t ldx;  // elements
  const float* params;
  const uint8_t* qb;
  int64_t ldb;  // bytes
  const uint8_t* sb;
  int64_t ldsb;
  int64_t M, N, K;
  void* out;    // [M][ldo] float32 or bf16
  int64_t ldo;  // elements
  bool out_bf16;
  void* stream;
  int cus;
  // device workspace for tiles split in K parts (flags first, zero between calls),
  // or NULL for whole tiles only; tiles are split only as far as it holds their
  // parts (all of mx_gemm_fused_workspace_bytes() when it holds that much)
  void* workspace = nullptr;
  int64_t workspace_bytes = 0;
};
// Every block's transform constants sit in the fused product's LDS: K <= 32 x this.
constexpr int64_t kFusedMaxBlocks = 512;
// One slot of a split 128 x 256 output tile's fp32 partial sums.
constexpr int64_t kFusedSplitTileBytes = 128 * 256 * 4;

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
hipError_t launch_mx_gemm_fused(const FusedGemmArgs& g);  // Y = deq(Q(T X)) deq(B)^T
// Workspace bytes of the fused product's split schedule (0 if its tiles are not split).
int64_t mx_gemm_fused_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus);
// Workspace bytes of the split schedule of an M x N x K product on `cus` compute
// units whose workspace holds at most max_slots partial-sum slots (0 if its tiles
// are not split).
int64_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus,
                                int64_t max_slots = INT64_MAX);
hipError_t launch_sq(const LaunchArgs& a);
hipError_t launch_mfma(const LaunchArgs& a);
hipError_t launch_expand(const float* params, int64_t nb, int tfmt, void* out, void* stream);

}  // namespace kq
