// Read-stream calibration kernel: the achievable HBM read rate of this GPU,
// reported beside the 8 TB/s nominal peak so that the GEMV kernels' roofline
// fractions can be read against both.  Every byte of the buffer is read once
// with 16-byte non-temporal loads (the hint the GEMV's weight stream uses;
// measured faster than plain loads, and than unrolled grid-stride loads),
// grid-stride; each wave folds what it read into one word (xor) so the loads
// cannot be dropped.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

__global__ __launch_bounds__(kReadStreamThreads) void k_read_stream(const u32x4* __restrict__ src,
                                                                    int64_t n16,
                                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kReadStreamThreads;
  for (int64_t i = (int64_t)blockIdx.x * kReadStreamThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
  if (lane_id() == 0)
    sink[blockIdx.x * (kReadStreamThreads / kWave) + threadIdx.x / kWave] = acc;
}

}  // namespace

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_read_stream, dim3(blocks), dim3(kReadStreamThreads), 0, s,
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace sa
