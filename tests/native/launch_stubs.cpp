// Stand-ins for the kernel launches of the HIP library, so that the C ABI's host
// code (kq_api.cpp) links into a CPU-only program built with the sanitizers.  The
// argument-check tests never reach them: each returns an error if one ever does.
#include <hip/hip_runtime_api.h>

#include "../../online_activation_quantizer_amd/csrc/kq_launch.hpp"

namespace kq {

hipError_t launch_butterfly(const LaunchArgs&) { return hipErrorNotSupported; }
hipError_t launch_weights(const LaunchArgs&) { return hipErrorNotSupported; }
hipError_t launch_hadamard(const LaunchArgs&) { return hipErrorNotSupported; }
hipError_t launch_norm(const NormArgs&) { return hipErrorNotSupported; }
hipError_t launch_mx_gemm(const GemmArgs&) { return hipErrorNotSupported; }
hipError_t launch_mx_gemm_fused(const FusedGemmArgs&) { return hipErrorNotSupported; }
int64_t mx_gemm_fused_workspace_bytes(int64_t, int64_t, int64_t, int) {
  return kSplitFlagBytes + kFusedSplitTileBytes;
}
int64_t mx_gemm_workspace_bytes(int64_t, int64_t, int64_t, int, int64_t) { return kSplitFlagBytes + kSplitTileBytes; }
hipError_t static_scratch(void**, void*) { return hipErrorNotSupported; }
hipError_t launch_sq(const LaunchArgs&) { return hipErrorNotSupported; }
hipError_t launch_mfma(const LaunchArgs&) { return hipErrorNotSupported; }
hipError_t launch_expand(const float*, int64_t, int, void*, void*) { return hipErrorNotSupported; }

}  // namespace kq
