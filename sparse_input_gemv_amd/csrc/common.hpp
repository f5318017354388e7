// Device helpers shared by the kernels: wave64 ballot / lane-prefix
// primitives, a workgroup exclusive scan and fp16 bit conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef _Float16 half_t;
typedef half_t half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Number of set bits of `m` in the lanes below this one (wave64 prefix).
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(half_t, b);
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (half_t)f);
}
// |x| as a 15-bit key; the order of keys is the order of fp16 magnitudes
// (for non-NaN values), and -0 and +0 share key 0.
__device__ __forceinline__ int mag_key(uint16_t b) { return (int)(b & 0x7fffu); }

// Exclusive scan of one int per thread across a workgroup of NT threads.
// `scratch` holds NT/64 ints of LDS.  Returns the exclusive prefix and sets
// `total`.  Contains two barriers; every thread must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = lane_id();
  const int w = (int)threadIdx.x / kWave;
  int s = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(s, o, kWave);
    if (lane >= o) s += t;
  }
  if (lane == kWave - 1) scratch[w] = s;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    int c = scratch[i];
    base += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + s - v;
}

}  // namespace sa
