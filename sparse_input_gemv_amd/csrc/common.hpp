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

// Loads E consecutive fp16 bit patterns starting at element k0 of a row
// (entries past d read as 0).  The vector path needs a 16-byte aligned row
// and k0 a multiple of 8.
template <int E>
__device__ __forceinline__ void load_run(const uint16_t* __restrict__ xr, int64_t k0, int64_t d,
                                         bool vec, uint16_t (&v)[E]) {
  if (vec && k0 + E <= d) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xr + k0);
#pragma unroll
    for (int q = 0; q < E / 8; ++q) {
      u32x4 r = p[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[q * 8 + 2 * i] = (uint16_t)(r[i] & 0xffffu);
        v[q * 8 + 2 * i + 1] = (uint16_t)(r[i] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = (k0 + e < d) ? xr[k0 + e] : (uint16_t)0;
  }
}

// Inclusive prefix sum within each row of 16 lanes: DPP row shifts (a VALU
// operand modifier: lane i reads lane i - n of its row, 0 where that lane is
// outside the row).  No LDS traffic.
__device__ __forceinline__ int row16_inclusive_scan(int v) {
  int s = v;
  s += __builtin_amdgcn_update_dpp(0, s, 0x111, 0xf, 0xf, true);  // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, s, 0x112, 0xf, 0xf, true);  // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xf, 0xf, true);  // row_shr:4
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xf, 0xf, true);  // row_shr:8
  return s;
}

// Inclusive prefix sum of one int per lane across a wave64: the rows are
// scanned, then the running totals of rows 0..2 are read out as scalars and
// added to the rows above them.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int s = row16_inclusive_scan(v);
  const int r0 = __builtin_amdgcn_readlane(s, 15);
  const int r1 = r0 + __builtin_amdgcn_readlane(s, 31);
  const int r2 = r1 + __builtin_amdgcn_readlane(s, 47);
  const int row = lane_id() >> 4;
  return s + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r1 : r2);
}

// Exclusive scan of one int per thread across a workgroup of NT <= 1024
// threads, with one barrier.  `scratch` holds NT/64 ints of LDS and must not
// be written again before every thread has passed a later barrier (give
// each scan of a kernel its own, or use block_exclusive_scan).  The waves'
// totals are combined by every wave's first row from LDS, and each wave
// takes its offset as a scalar.  Returns the exclusive prefix and sets
// `total`; every thread must call it.
template <int NT>
__device__ __forceinline__ int block_scan_once(int v, int* scratch, int& total) {
  static_assert(NT % kWave == 0 && NT / kWave <= 16, "wave totals fit one row");
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int s = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[w] = s;
  __syncthreads();
  const int t = row16_inclusive_scan(lane < NW ? scratch[lane] : 0);
  const int base = w == 0 ? 0 : __builtin_amdgcn_readlane(t, w == 0 ? 0 : w - 1);
  total = __builtin_amdgcn_readlane(t, NW - 1);
  return base + s - v;
}

// block_scan_once followed by a barrier, so `scratch` may be reused at once.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int r = block_scan_once<NT>(v, scratch, total);
  __syncthreads();
  return r;
}

}  // namespace sa
