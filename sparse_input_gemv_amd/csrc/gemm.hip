// MFMA matmuls: dense GEMM baseline and batched N:M activation-sparse GEMM.
#include "common.hpp"
#include "launch.hpp"

namespace sa {

hipError_t launch_dense_gemm(const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t,
                             uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_nm_spmm(const uint16_t*, const uint32_t*, int64_t, int64_t, int, int,
                          const uint16_t*, int64_t, uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sa
