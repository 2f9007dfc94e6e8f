// Host-side argument checks of the C ABI (include/kq.h), built with the address
// and undefined-behaviour sanitizers and linked against stand-ins for the kernel
// launches (never reached: every case here is rejected, or is a no-op, before any
// HIP call).  Exits non-zero on the first status that differs from the expected one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "kq.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// Fake, suitably aligned device addresses: validation never dereferences them.
uint8_t* const X = reinterpret_cast<uint8_t*>(0x10000);
uint8_t* const T = reinterpret_cast<uint8_t*>(0x20000);
uint8_t* const Q = reinterpret_cast<uint8_t*>(0x30000);
uint8_t* const S = reinterpret_cast<uint8_t*>(0x40000);
float* const Y = reinterpret_cast<float*>(0x50000);
const float* const P = reinterpret_cast<const float*>(0x20000);

int quant(const void* x, int dtype, int64_t rows, int64_t d, int64_t ldx, const void* t, int tfmt,
          uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, int variant) {
  return kq_quantize(x, dtype, rows, d, ldx, t, tfmt, q, ldq, s, lds, variant, nullptr);
}

}  // namespace

int main() {
  // kq_quantize
  EXPECT(quant(X, 7, 4, 64, 64, T, 0, Q, 32, S, 2, 0), KQ_ERR_DTYPE);
  EXPECT(quant(X, 0, 4, 48, 48, T, 0, Q, 24, S, 2, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 0, 4, 0, 0, T, 0, Q, 0, S, 0, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 0, -1, 64, 64, T, 0, Q, 32, S, 2, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 0, int64_t(1) << 31, 64, 64, T, 0, Q, 32, S, 2, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 0, 4, int64_t(1) << 28, int64_t(1) << 28, T, 0, Q, int64_t(1) << 27, S,
               int64_t(1) << 23, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 1, 4, 64, int64_t(1) << 30, T, 0, Q, 32, S, 2, 0), KQ_ERR_SHAPE);  // pitch >= 4 GiB
  EXPECT(quant(X, 0, 4, 64, 32, T, 0, Q, 32, S, 2, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q, 16, S, 2, 0), KQ_ERR_SHAPE);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q, 32, S, 1, 0), KQ_ERR_SHAPE);
  EXPECT(quant(nullptr, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0), KQ_ERR_NULL);
  EXPECT(quant(X, 0, 4, 64, 64, nullptr, 0, Q, 32, S, 2, 0), KQ_ERR_NULL);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, nullptr, 32, S, 2, 0), KQ_ERR_NULL);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q, 32, nullptr, 2, 0), KQ_ERR_NULL);
  EXPECT(quant(X + 8, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0), KQ_ERR_ALIGN);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q + 4, 32, S, 2, 0), KQ_ERR_ALIGN);
  EXPECT(quant(X, 0, 4, 64, 68, T, 0, Q, 32, S, 2, 0), KQ_ERR_ALIGN);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q, 40, S, 2, 0), KQ_ERR_ALIGN);
  EXPECT(quant(X, 0, 4, 64, 64, T + 2, 0, Q, 32, S, 2, 0), KQ_ERR_ALIGN);
  EXPECT(quant(X, 0, 4, 64, 64, T, 9, Q, 32, S, 2, 0), KQ_ERR_FORMAT);
  EXPECT(quant(X, 0, 4, 64, 64, T, 1, Q, 32, S, 2, 0), KQ_ERR_FORMAT);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 2), KQ_ERR_FORMAT);
  EXPECT(quant(X, 0, 4, 64, 64, T, 2, Q, 32, S, 2, 1), KQ_ERR_FORMAT);
  EXPECT(quant(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 5), KQ_ERR_VARIANT);
  EXPECT(quant(X, 1, 4, 64, 64, T, 2, Q, 32, S, 2, 2), KQ_ERR_DTYPE);
  EXPECT(quant(nullptr, 0, 0, 64, 64, nullptr, 0, nullptr, 32, nullptr, 2, 0), KQ_OK);
  EXPECT(kq_transform_debug(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0, nullptr, 64, nullptr), KQ_ERR_NULL);
  EXPECT(kq_transform_debug(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0, Y, 32, nullptr), KQ_ERR_SHAPE);

  // sq_quantize
  EXPECT(sq_quantize(X, 0, 4, 64, 64, nullptr, Q, 32, S, 2, nullptr), KQ_ERR_NULL);
  EXPECT(sq_quantize(X, 0, 4, 64, 64, P + 1, Q, 32, S, 2, nullptr), KQ_ERR_ALIGN);
  EXPECT(sq_quantize(X, 3, 4, 64, 64, P, Q, 32, S, 2, nullptr), KQ_ERR_DTYPE);
  EXPECT(sq_transform_debug(X, 0, 4, 64, 64, P, Q, 32, S, 2, nullptr, 64, nullptr), KQ_ERR_NULL);

  // weights, Hadamard
  EXPECT(kq_quantize_weights(X, 0, 4, 64, 64, nullptr, Q, 32, S, 2, nullptr), KQ_ERR_NULL);
  EXPECT(kq_quantize_weights(X, 0, 4, 48, 48, P, Q, 24, S, 2, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_weights_debug(X, 0, 4, 64, 64, P, Q, 32, S, 2, Y, 32, nullptr), KQ_ERR_SHAPE);
  EXPECT(hq_quantize(nullptr, 0, 4, 64, 64, Q, 32, S, 2, nullptr), KQ_ERR_NULL);
  EXPECT(hq_quantize(X + 4, 0, 4, 64, 64, Q, 32, S, 2, nullptr), KQ_ERR_ALIGN);
  EXPECT(hq_transform_debug(X, 0, 4, 64, 64, Q, 32, S, 2, Y, 63, nullptr), KQ_ERR_SHAPE);

  // fused normalization
  const float* sh = reinterpret_cast<const float*>(0x60000);
  const float* sc = reinterpret_cast<const float*>(0x70000);
  EXPECT(kq_norm_quantize(X, 0, 4, 64, 64, sh, sc, 0, 1e-6f, P, Q, 32, S, 2, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_norm_quantize(X, 0, 4, 64, 64, sh, sc, 4, -1.0f, P, Q, 32, S, 2, nullptr), KQ_ERR_VALUE);
  EXPECT(kq_norm_quantize(X, 0, 4, 64, 64, sh, sc, 4, std::nanf(""), P, Q, 32, S, 2, nullptr),
         KQ_ERR_VALUE);
  EXPECT(kq_norm_quantize(X, 0, 4, 64, 64, sh, sc, 4, INFINITY, P, Q, 32, S, 2, nullptr), KQ_ERR_VALUE);
  EXPECT(kq_norm_quantize(X, 0, 4, 64, 64, nullptr, sc, 4, 1e-6f, P, Q, 32, S, 2, nullptr), KQ_ERR_NULL);
  EXPECT(kq_norm_quantize(X, 0, 4, 64, 64, sh + 1, sc, 4, 1e-6f, P, Q, 32, S, 2, nullptr), KQ_ERR_ALIGN);
  EXPECT(kq_norm_quantize(X, 0, 4, 16416, 16416, sh, sc, 4, 1e-6f, P, Q, 8208, S, 513, nullptr),
         KQ_ERR_SHAPE);
  EXPECT(kq_norm_debug(X, 0, 4, 64, 64, nullptr, nullptr, 4, 1e-6f, P, Q, 32, S, 2, nullptr, 64, nullptr),
         KQ_ERR_NULL);

  // W4A4 product
  EXPECT(kq_mx_gemm(Q, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 5, nullptr), KQ_ERR_DTYPE);
  EXPECT(kq_mx_gemm(Q, 32, S, 4, T, 32, S, 4, 8, 8, 48, X, 8, 1, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm(Q, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 7, 1, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm(Q, 64, S, 4, T, 64, S, 4, -1, 8, 128, X, 8, 1, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm(nullptr, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1, nullptr), KQ_ERR_NULL);
  EXPECT(kq_mx_gemm(Q + 8, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1, nullptr), KQ_ERR_ALIGN);
  EXPECT(kq_mx_gemm(Q, 64, S, 4, T, 64, S, 4, 8, 8, 128, X + 2, 8, 1, nullptr), KQ_ERR_ALIGN);
  EXPECT(kq_mx_gemm(nullptr, 64, nullptr, 4, nullptr, 64, nullptr, 4, 0, 8, 128, nullptr, 8, 1, nullptr),
         KQ_OK);
  // code pitches of 16 MiB and more
  EXPECT(kq_mx_gemm(Q, 1 << 24, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm(Q, 64, S, 4, T, 1 << 24, S, 4, 8, 8, 128, X, 8, 1, nullptr), KQ_ERR_SHAPE);
  // with a workspace: the same checks first, then the workspace's own
  void* const W = reinterpret_cast<void*>(0x60000);
  EXPECT(kq_mx_gemm_ws(Q, 64, S, 4, T, 64, S, 4, 8, 8, 48, X, 8, 1, W, 1 << 20, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_ws(Q, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1, nullptr, 4096, nullptr), KQ_ERR_NULL);
  EXPECT(kq_mx_gemm_ws(Q, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1,
                       reinterpret_cast<uint8_t*>(W) + 128, 1 << 20, nullptr),
         KQ_ERR_ALIGN);
  EXPECT(kq_mx_gemm_ws(nullptr, 64, nullptr, 4, nullptr, 64, nullptr, 4, 8, 0, 128, nullptr, 8, 1, W, 0,
                       nullptr),
         KQ_OK);
  // the static-workspace variant: the product's checks, before any HIP call
  EXPECT(kq_mx_gemm_static(Q, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 5, nullptr), KQ_ERR_DTYPE);
  EXPECT(kq_mx_gemm_static(Q, 64, S, 4, T, 64, S, 4, 8, 8, 48, X, 8, 1, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_static(nullptr, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1, nullptr), KQ_ERR_NULL);
  EXPECT(kq_mx_gemm_static(Q + 8, 64, S, 4, T, 64, S, 4, 8, 8, 128, X, 8, 1, nullptr), KQ_ERR_ALIGN);
  EXPECT(kq_mx_gemm_static(nullptr, 64, nullptr, 4, nullptr, 64, nullptr, 4, 0, 8, 128, nullptr, 8, 1,
                           nullptr),
         KQ_OK);
  // the prologue-fused product: bf16 activations, K <= 16384
  EXPECT(kq_mx_gemm_fused(X, 1, 128, P, Q, 64, S, 4, 8, 8, 128, Y, 8, 1, nullptr), KQ_ERR_DTYPE);
  EXPECT(kq_mx_gemm_fused(X, 0, 16416, P, Q, 8208, S, 513, 8, 8, 16416, Y, 8, 1, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_fused(X, 0, 128, nullptr, Q, 64, S, 4, 8, 8, 128, Y, 8, 1, nullptr), KQ_ERR_NULL);
  EXPECT(kq_mx_gemm_fused(X + 8, 0, 128, P, Q, 64, S, 4, 8, 8, 128, Y, 8, 1, nullptr), KQ_ERR_ALIGN);
  EXPECT(kq_mx_gemm_fused(nullptr, 0, 128, nullptr, nullptr, 64, nullptr, 4, 0, 8, 128, nullptr, 8, 1,
                          nullptr),
         KQ_OK);
  // the prologue-fused product with a workspace: the product's checks, then the
  // workspace's own, all before any HIP call
  EXPECT(kq_mx_gemm_fused_ws(X, 1, 128, P, Q, 64, S, 4, 8, 8, 128, Y, 8, 1, W, 1 << 20, nullptr), KQ_ERR_DTYPE);
  EXPECT(kq_mx_gemm_fused_ws(X, 0, 128, P, Q, 64, S, 4, 8, 8, 48, Y, 8, 1, W, 1 << 20, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_fused_ws(X, 0, 128, P, Q, 64, S, 4, 8, 8, 128, Y, 8, 1, nullptr, 4096, nullptr),
         KQ_ERR_NULL);
  EXPECT(kq_mx_gemm_fused_ws(X, 0, 128, P, Q, 64, S, 4, 8, 8, 128, Y, 8, 1,
                             reinterpret_cast<uint8_t*>(W) + 128, 1 << 20, nullptr),
         KQ_ERR_ALIGN);
  EXPECT(kq_mx_gemm_fused_ws(nullptr, 0, 128, nullptr, nullptr, 64, nullptr, 4, 0, 8, 128, nullptr, 8, 1, W, 0,
                             nullptr),
         KQ_OK);
  int64_t bytes = -1;
  EXPECT(kq_mx_gemm_fused_workspace_size(8, 8, 128, nullptr), KQ_ERR_NULL);
  EXPECT(kq_mx_gemm_fused_workspace_size(8, 8, 48, &bytes), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_fused_workspace_size(8, 8, 16416, &bytes), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_fused_workspace_size(0, 8, 128, &bytes), KQ_OK);
  EXPECT((int)bytes, 0);
  bytes = -1;
  EXPECT(kq_mx_gemm_workspace_size(8, 8, 128, nullptr), KQ_ERR_NULL);
  EXPECT(kq_mx_gemm_workspace_size(8, 8, 48, &bytes), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_workspace_size(-1, 8, 128, &bytes), KQ_ERR_SHAPE);
  EXPECT(kq_mx_gemm_workspace_size(0, 8, 128, &bytes), KQ_OK);
  EXPECT((int)bytes, 0);

  // expansion, status text
  EXPECT(kq_expand_factors(P, 4, 0, Y, nullptr), KQ_ERR_FORMAT);
  EXPECT(kq_expand_factors(P, -1, 1, Y, nullptr), KQ_ERR_SHAPE);
  EXPECT(kq_expand_factors(nullptr, 4, 1, Y, nullptr), KQ_ERR_NULL);
  for (int st = -9; st <= 1; ++st)
    if (!kq_status_string(st)) ++failures;
  EXPECT(kq_last_hip_error(), 0);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi checks: all passed\n");
  return 0;
}
