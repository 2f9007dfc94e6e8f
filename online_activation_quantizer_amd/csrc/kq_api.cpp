// kq_api.cpp — the C ABI declared in include/kq.h: host-side argument checks,
// variant dispatch and launches.  Every check runs before the first HIP call.
#include "../../include/kq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>

#include "kq_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not queried yet

int fail_hip(hipError_t e) {
  g_last_hip_error = (int)e;
  return KQ_ERR_HIP;
}

// Compute units of the current device (cached per device).
int current_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return KQ_OK;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail_hip(e);
  if (c < 1) c = 1;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return KQ_OK;
}

// Kernels index lanes, rows and row pitches with 32-bit arithmetic: at most 2^22
// blocks (d <= 2^27), rows < 2^31 and row pitches below 4 GiB.
constexpr int64_t kMaxBlocks = int64_t(1) << 22;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxPitch = (int64_t(1) << 32) - 1;
constexpr int64_t kMaxGemmCodePitch = int64_t(1) << 24;
// The normalization-fused kernel holds one row per workgroup: at most 512 blocks.
constexpr int64_t kMaxNormWidth = 16384;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int elem_size(int dtype) { return dtype == KQ_BF16 ? 2 : 4; }

// Checks shared by the quantize entry points.
int check_common(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                 const void* t, const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds) {
  if (dtype != KQ_BF16 && dtype != KQ_FP32) return KQ_ERR_DTYPE;
  if (rows < 0 || d <= 0 || d % 32 != 0 || ldx < d || ldq < d / 2 || lds < d / 32)
    return KQ_ERR_SHAPE;
  if (d / 32 > kMaxBlocks || rows > kMaxRows || ldx * elem_size(dtype) > kMaxPitch ||
      ldq > kMaxPitch || lds > kMaxPitch)
    return KQ_ERR_SHAPE;
  if (rows == 0) return KQ_OK;
  if (!x || !t || !q || !s) return KQ_ERR_NULL;
  if (!aligned(x, 16) || (ldx * elem_size(dtype)) % 16 != 0 || !aligned(q, 16) || ldq % 16 != 0)
    return KQ_ERR_ALIGN;
  return KQ_OK;
}

int resolve_variant(int variant, int tfmt, int* out) {
  if (tfmt != KQ_T_PARAMS && tfmt != KQ_T_DENSE_F32 && tfmt != KQ_T_DENSE_BF16X3)
    return KQ_ERR_FORMAT;
  switch (variant) {
    case KQ_AUTO:
      if (tfmt == KQ_T_PARAMS) *out = KQ_BUTTERFLY;
      else if (tfmt == KQ_T_DENSE_BF16X3) *out = KQ_MFMA;
      else return KQ_ERR_FORMAT;
      return KQ_OK;
    case KQ_BUTTERFLY:
      if (tfmt != KQ_T_PARAMS) return KQ_ERR_FORMAT;
      *out = KQ_BUTTERFLY;
      return KQ_OK;
    case KQ_MFMA:
      if (tfmt != KQ_T_DENSE_BF16X3) return KQ_ERR_FORMAT;
      *out = KQ_MFMA;
      return KQ_OK;
    default:
      return KQ_ERR_VARIANT;
  }
}

int quantize_impl(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, const void* t,
                  int tfmt, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, int variant,
                  float* y, int64_t ldy, bool debug, void* stream) {
  int rc = check_common(x, dtype, rows, d, ldx, t, q, ldq, s, lds);
  if (rc != KQ_OK) return rc;
  int v = 0;
  rc = resolve_variant(variant, tfmt, &v);
  if (rc != KQ_OK) return rc;
  if (debug) {
    if (ldy < d || ldy * 4 > kMaxPitch) return KQ_ERR_SHAPE;
    if (rows > 0 && !y) return KQ_ERR_NULL;
    if (rows > 0 && !aligned(y, 4)) return KQ_ERR_ALIGN;
  }
  if (rows == 0) return KQ_OK;
  if (!aligned(t, v == KQ_MFMA ? 16 : 4)) return KQ_ERR_ALIGN;
  if (v == KQ_MFMA && dtype != KQ_BF16) return KQ_ERR_DTYPE;
  kq::LaunchArgs a{x, dtype, rows, d, d / 32, ldx, t, q, ldq, s, lds, debug ? y : nullptr,
                   ldy, stream, 0};
  rc = current_cus(&a.cus);
  if (rc != KQ_OK) return rc;
  const hipError_t e = v == KQ_MFMA ? kq::launch_mfma(a) : kq::launch_butterfly(a);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int sq_impl(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, const float* mult,
            uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y, int64_t ldy, bool debug,
            void* stream) {
  int rc = check_common(x, dtype, rows, d, ldx, mult, q, ldq, s, lds);
  if (rc != KQ_OK) return rc;
  if (debug) {
    if (ldy < d || ldy * 4 > kMaxPitch) return KQ_ERR_SHAPE;
    if (rows > 0 && !y) return KQ_ERR_NULL;
    if (rows > 0 && !aligned(y, 4)) return KQ_ERR_ALIGN;
  }
  if (rows == 0) return KQ_OK;
  if (!aligned(mult, 16)) return KQ_ERR_ALIGN;
  kq::LaunchArgs a{x, dtype, rows, d, d / 32, ldx, mult, q, ldq, s, lds, debug ? y : nullptr,
                   ldy, stream, 0};
  rc = current_cus(&a.cus);
  if (rc != KQ_OK) return rc;
  const hipError_t e = kq::launch_sq(a);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int weights_impl(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                 const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y,
                 int64_t ldy, bool debug, void* stream) {
  int rc = check_common(w, dtype, rows, d, ldw, params, q, ldq, s, lds);
  if (rc != KQ_OK) return rc;
  if (debug) {
    if (ldy < d || ldy * 4 > kMaxPitch) return KQ_ERR_SHAPE;
    if (rows > 0 && !y) return KQ_ERR_NULL;
    if (rows > 0 && !aligned(y, 4)) return KQ_ERR_ALIGN;
  }
  if (rows == 0) return KQ_OK;
  if (!aligned(params, 4)) return KQ_ERR_ALIGN;
  kq::LaunchArgs a{w, dtype, rows, d, d / 32, ldw, params, q, ldq, s, lds, debug ? y : nullptr,
                   ldy, stream, 0};
  rc = current_cus(&a.cus);
  if (rc != KQ_OK) return rc;
  const hipError_t e = kq::launch_weights(a);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int hadamard_impl(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, uint8_t* q,
                  int64_t ldq, uint8_t* s, int64_t lds, float* y, int64_t ldy, bool debug,
                  void* stream) {
  // the transform takes no operand: any non-null stand-in passes the shared check
  int rc = check_common(x, dtype, rows, d, ldx, q, q, ldq, s, lds);
  if (rc != KQ_OK) return rc;
  if (debug) {
    if (ldy < d || ldy * 4 > kMaxPitch) return KQ_ERR_SHAPE;
    if (rows > 0 && !y) return KQ_ERR_NULL;
    if (rows > 0 && !aligned(y, 4)) return KQ_ERR_ALIGN;
  }
  if (rows == 0) return KQ_OK;
  kq::LaunchArgs a{x, dtype, rows, d, d / 32, ldx, nullptr, q, ldq, s, lds, debug ? y : nullptr,
                   ldy, stream, 0};
  rc = current_cus(&a.cus);
  if (rc != KQ_OK) return rc;
  const hipError_t e = kq::launch_hadamard(a);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int norm_impl(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, const float* shift,
              const float* scale, int64_t rows_per_sample, float eps, const float* params,
              uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y, int64_t ldy, bool debug,
              void* stream) {
  int rc = check_common(x, dtype, rows, d, ldx, params, q, ldq, s, lds);
  if (rc != KQ_OK) return rc;
  if (rows_per_sample < 1 || d > kMaxNormWidth) return KQ_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return KQ_ERR_VALUE;
  if (debug) {
    if (ldy < d || ldy * 4 > kMaxPitch) return KQ_ERR_SHAPE;
    if (rows > 0 && !y) return KQ_ERR_NULL;
    if (rows > 0 && !aligned(y, 4)) return KQ_ERR_ALIGN;
  }
  if (rows == 0) return KQ_OK;
  if ((shift == nullptr) != (scale == nullptr)) return KQ_ERR_NULL;
  if (!aligned(params, 4) || (shift && (!aligned(shift, 16) || !aligned(scale, 16))))
    return KQ_ERR_ALIGN;
  kq::NormArgs n{{x, dtype, rows, d, d / 32, ldx, params, q, ldq, s, lds, debug ? y : nullptr,
                  ldy, stream, 0},
                 shift, scale, rows_per_sample < rows ? rows_per_sample : rows, eps};
  rc = current_cus(&n.a.cus);
  if (rc != KQ_OK) return rc;
  const hipError_t e = kq::launch_norm(n);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

// argument checks shared by the product's entry points (KQ_OK: launch; the empty
// product returns KQ_OK with *empty set)
int check_mx_gemm(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
                  const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                  int64_t N, int64_t K, const void* out, int64_t ldo, int out_dtype, bool* empty) {
  *empty = false;
  if (out_dtype != KQ_FP32 && out_dtype != KQ_BF16) return KQ_ERR_DTYPE;
  // code pitches below 16 MiB: a tile's 256 rows are read through one 32-bit range
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || K / 32 > kMaxBlocks || M > kMaxRows ||
      N > kMaxRows || lda < K / 2 || ldb < K / 2 || ldsa < K / 32 || ldsb < K / 32 || ldo < N ||
      lda >= kMaxGemmCodePitch || ldb >= kMaxGemmCodePitch || ldsa > kMaxPitch ||
      ldsb > kMaxPitch || ldo * (out_dtype == KQ_FP32 ? 4 : 2) > kMaxPitch)
    return KQ_ERR_SHAPE;
  if (M == 0 || N == 0) {
    *empty = true;
    return KQ_OK;
  }
  if (((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX) return KQ_ERR_SHAPE;
  if (!qa || !sa || !qb || !sb || !out) return KQ_ERR_NULL;
  if (!aligned(qa, 16) || !aligned(qb, 16) || lda % 16 != 0 || ldb % 16 != 0 ||
      !aligned(out, out_dtype == KQ_FP32 ? 4 : 2))
    return KQ_ERR_ALIGN;
  return KQ_OK;
}

int mx_gemm_impl(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
                 const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                 int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* workspace,
                 int64_t workspace_bytes, void* stream) {
  bool empty = false;
  int rc = check_mx_gemm(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo, out_dtype, &empty);
  if (rc != KQ_OK || empty) return rc;
  if (!workspace && workspace_bytes != 0) return KQ_ERR_NULL;
  if (workspace && !aligned(workspace, 256)) return KQ_ERR_ALIGN;
  int cus = 0;
  rc = current_cus(&cus);
  if (rc != KQ_OK) return rc;
  if (workspace && workspace_bytes < kq::mx_gemm_workspace_bytes(M, N, K, cus)) return KQ_ERR_VALUE;
  kq::GemmArgs g{qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo,
                 out_dtype == KQ_BF16, stream, cus};
  g.workspace = workspace;
  g.workspace_bytes = workspace_bytes;
  const hipError_t e = kq::launch_mx_gemm(g);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int mx_gemm_fused_impl(const void* x, int dtype, int64_t ldx, const float* params, const uint8_t* qb,
                       int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M, int64_t N, int64_t K,
                       void* out, int64_t ldo, int out_dtype, void* workspace, int64_t workspace_bytes,
                       void* stream) {
  if (dtype != KQ_BF16) return KQ_ERR_DTYPE;  // the prologue reads bf16 activations only
  if (out_dtype != KQ_FP32 && out_dtype != KQ_BF16) return KQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || K / 32 > kq::kFusedMaxBlocks || M > kMaxRows ||
      N > kMaxRows || ldx < K || ldb < K / 2 || ldsb < K / 32 || ldo < N || ldx * 2 > kMaxPitch ||
      ldb > kMaxPitch || ldsb > kMaxPitch || ldo * (out_dtype == KQ_FP32 ? 4 : 2) > kMaxPitch)
    return KQ_ERR_SHAPE;
  if (M == 0 || N == 0) return KQ_OK;
  if (!x || !params || !qb || !sb || !out) return KQ_ERR_NULL;
  if (!aligned(x, 16) || (ldx * 2) % 16 != 0 || !aligned(qb, 16) || ldb % 16 != 0 ||
      !aligned(out, out_dtype == KQ_FP32 ? 4 : 2))
    return KQ_ERR_ALIGN;
  if (!workspace && workspace_bytes != 0) return KQ_ERR_NULL;
  if (workspace && !aligned(workspace, 256)) return KQ_ERR_ALIGN;
  int cus = 0;
  const int rc = current_cus(&cus);
  if (rc != KQ_OK) return rc;
  if (workspace && workspace_bytes < kq::mx_gemm_fused_workspace_bytes(M, N, K, cus)) return KQ_ERR_VALUE;
  kq::FusedGemmArgs g{x, ldx, params, qb, ldb, sb, ldsb, M, N, K, out, ldo,
                      out_dtype == KQ_BF16, stream, cus};
  g.workspace = workspace;
  g.workspace_bytes = workspace_bytes;
  const hipError_t e = kq::launch_mx_gemm_fused(g);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

}  // namespace

extern "C" {

int kq_expand_factors(const float* params, int64_t nb, int tfmt, void* t_out, void* stream) {
  if (tfmt != KQ_T_DENSE_F32 && tfmt != KQ_T_DENSE_BF16X3 && tfmt != KQ_T_FACTORS_2X2_F32)
    return KQ_ERR_FORMAT;
  if (nb < 0 || nb > INT32_MAX) return KQ_ERR_SHAPE;
  if (nb == 0) return KQ_OK;
  if (!params || !t_out) return KQ_ERR_NULL;
  if (!aligned(params, 4) || !aligned(t_out, tfmt == KQ_T_FACTORS_2X2_F32 ? 16 : 4))
    return KQ_ERR_ALIGN;
  const hipError_t e = kq::launch_expand(params, nb, tfmt, t_out, stream);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int kq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, const void* t,
                int tfmt, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, int variant,
                void* stream) {
  return quantize_impl(x, dtype, rows, d, ldx, t, tfmt, q, ldq, s, lds, variant, nullptr, 0,
                       false, stream);
}

int sq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                const float* mult, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                void* stream) {
  return sq_impl(x, dtype, rows, d, ldx, mult, q, ldq, s, lds, nullptr, 0, false, stream);
}

int kq_transform_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       const void* t, int tfmt, uint8_t* q, int64_t ldq, uint8_t* s,
                       int64_t lds, int variant, float* y, int64_t ldy, void* stream) {
  return quantize_impl(x, dtype, rows, d, ldx, t, tfmt, q, ldq, s, lds, variant, y, ldy, true,
                       stream);
}

int sq_transform_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       const float* mult, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                       float* y, int64_t ldy, void* stream) {
  return sq_impl(x, dtype, rows, d, ldx, mult, q, ldq, s, lds, y, ldy, true, stream);
}

int kq_quantize_weights(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                        const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                        void* stream) {
  return weights_impl(w, dtype, rows, d, ldw, params, q, ldq, s, lds, nullptr, 0, false, stream);
}

int kq_weights_debug(const void* w, int dtype, int64_t rows, int64_t d, int64_t ldw,
                     const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                     float* y, int64_t ldy, void* stream) {
  return weights_impl(w, dtype, rows, d, ldw, params, q, ldq, s, lds, y, ldy, true, stream);
}

int hq_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, uint8_t* q,
                int64_t ldq, uint8_t* s, int64_t lds, void* stream) {
  return hadamard_impl(x, dtype, rows, d, ldx, q, ldq, s, lds, nullptr, 0, false, stream);
}

int hq_transform_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                       uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y, int64_t ldy,
                       void* stream) {
  return hadamard_impl(x, dtype, rows, d, ldx, q, ldq, s, lds, y, ldy, true, stream);
}

int kq_norm_quantize(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                     const float* shift, const float* scale, int64_t rows_per_sample, float eps,
                     const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                     void* stream) {
  return norm_impl(x, dtype, rows, d, ldx, shift, scale, rows_per_sample, eps, params, q, ldq, s,
                   lds, nullptr, 0, false, stream);
}

int kq_norm_debug(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx,
                  const float* shift, const float* scale, int64_t rows_per_sample, float eps,
                  const float* params, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, float* y,
                  int64_t ldy, void* stream) {
  return norm_impl(x, dtype, rows, d, ldx, shift, scale, rows_per_sample, eps, params, q, ldq, s,
                   lds, y, ldy, true, stream);
}

int kq_mx_gemm(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
               const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
               int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* stream) {
  return mx_gemm_impl(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo, out_dtype, nullptr,
                      0, stream);
}

int kq_mx_gemm_fused(const void* x, int dtype, int64_t ldx, const float* params,
                     const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                     int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* stream) {
  return mx_gemm_fused_impl(x, dtype, ldx, params, qb, ldb, sb, ldsb, M, N, K, out, ldo, out_dtype, nullptr, 0,
                            stream);
}

int kq_mx_gemm_fused_ws(const void* x, int dtype, int64_t ldx, const float* params,
                        const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                        int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  return mx_gemm_fused_impl(x, dtype, ldx, params, qb, ldb, sb, ldsb, M, N, K, out, ldo, out_dtype, workspace,
                            workspace_bytes, stream);
}

int kq_mx_gemm_fused_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes) return KQ_ERR_NULL;
  *bytes = 0;
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || K / 32 > kq::kFusedMaxBlocks || M > kMaxRows ||
      N > kMaxRows)
    return KQ_ERR_SHAPE;
  if (M == 0 || N == 0) return KQ_OK;
  int cus = 0;
  const int rc = current_cus(&cus);
  if (rc != KQ_OK) return rc;
  *bytes = kq::mx_gemm_fused_workspace_bytes(M, N, K, cus);
  return KQ_OK;
}

int kq_mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes) return KQ_ERR_NULL;
  *bytes = 0;
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || K / 32 > kMaxBlocks || M > kMaxRows || N > kMaxRows)
    return KQ_ERR_SHAPE;
  if (M == 0 || N == 0) return KQ_OK;
  if (((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX) return KQ_ERR_SHAPE;
  int cus = 0;
  const int rc = current_cus(&cus);
  if (rc != KQ_OK) return rc;
  *bytes = kq::mx_gemm_workspace_bytes(M, N, K, cus);
  return KQ_OK;
}

int kq_mx_gemm_static(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
                      const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                      int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* stream) {
  bool empty = false;
  int rc = check_mx_gemm(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo, out_dtype, &empty);
  if (rc != KQ_OK || empty) return rc;
  int cus = 0;
  rc = current_cus(&cus);
  if (rc != KQ_OK) return rc;
  // the split schedule whose part slots the static array holds
  const int64_t need = kq::mx_gemm_workspace_bytes(M, N, K, cus, kq::kStaticSplitTiles);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = kq::static_scratch(&ws, stream);
    if (e != hipSuccess) return fail_hip(e);
  }
  kq::GemmArgs g{qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo,
                 out_dtype == KQ_BF16, stream, cus};
  g.workspace = ws;
  g.workspace_bytes = ws ? kq::kStaticScratchBytes : 0;
  const hipError_t e = kq::launch_mx_gemm(g);
  return e == hipSuccess ? KQ_OK : fail_hip(e);
}

int kq_mx_gemm_ws(const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t ldsa,
                  const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t M,
                  int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype, void* workspace,
                  int64_t workspace_bytes, void* stream) {
  return mx_gemm_impl(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo, out_dtype, workspace,
                      workspace_bytes, stream);
}

const char* kq_status_string(int status) {
  switch (status) {
    case KQ_OK: return "ok";
    case KQ_ERR_NULL: return "null pointer";
    case KQ_ERR_SHAPE: return "bad shape or pitch";
    case KQ_ERR_ALIGN: return "misaligned pointer or pitch";
    case KQ_ERR_DTYPE: return "unsupported dtype";
    case KQ_ERR_FORMAT: return "unsupported transform format";
    case KQ_ERR_VARIANT: return "unknown variant";
    case KQ_ERR_HIP: return "HIP error";
    case KQ_ERR_VALUE: return "scalar argument out of range";
    default: return "unknown status";
  }
}

int kq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
