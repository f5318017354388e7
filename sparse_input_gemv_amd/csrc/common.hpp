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
// and k0 a multiple of 8; runs of other lengths always load entry by entry.
template <int E>
__device__ __forceinline__ void load_run(const uint16_t* __restrict__ xr, int64_t k0, int64_t d,
                                         bool vec, uint16_t (&v)[E]) {
  if (E % 8 == 0 && vec && k0 + E <= d) {
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

// The Top-K cutoff of one row, found by one workgroup: the pair (tau, i*)
// with tau the k-th largest 15-bit magnitude key and i* the index of the
// last surviving entry equal to it (ties to the lower index), for a row of
// at most NT x E entries (thread t holds the run of E entries from k0 = t E
// in v, loaded by the caller with load_run).
// Two radix passes over 4 KB of LDS, small enough to sit beside a GEMV's
// own LDS (the one-launch Top-K GEMV runs it in every workgroup):
//  1. key >> 5 into 1024 LDS bins; a workgroup scan of the threads' bin
//     sums (thread t owns 1024 / NT consecutive bins) finds the bin b1 that
//     holds the k-th largest key, and r1 = k - #(keys in higher bins);
//  2. the low 5 bits of the keys in bin b1 into 32 bins; one wave scans them
//     from the top: tau = 32 b1 + that bin, and r = r1 - #(keys of b1 above
//     tau) entries equal to tau survive;
//  3. i* = the index of the r-th entry equal to tau, found by a scan of the
//     threads' counts (thread order is index order).
// k = 0 gives tau = 2^15, i* = -1 (nothing survives).  Requires k <= d.
// Every thread of the workgroup must call it.
constexpr int kSelBins = 1024, kSelSub = 32;
struct SelLds {
  int h1[kSelBins];
  int h2[kSelSub];
  int scan[2][16];
  int sel[3];
};

template <int NT, int E>
__device__ void wg_topk_cutoff(const uint16_t (&v)[E], int64_t d, int64_t k, SelLds& s,
                               int& tau_out, int& istar_out) {
  constexpr int BPT = kSelBins / NT;
  static_assert(kSelBins % NT == 0 && BPT >= 1, "bins split over the threads");
  const int tid = (int)threadIdx.x;
  if (k <= 0) {
    tau_out = 1 << 15;
    istar_out = -1;
    return;
  }
  const int64_t k0 = (int64_t)tid * E;
  for (int i = tid; i < kSelBins; i += NT) s.h1[i] = 0;
  if (tid < kSelSub) s.h2[tid] = 0;
  int key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (k0 + e < d) ? mag_key(v[e]) : -1;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] >= 0) atomicAdd(&s.h1[key[e] >> 5], 1);
  __syncthreads();
  const int kk = (int)k;
  int c[BPT], mine = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = s.h1[tid * BPT + j];
    mine += c[j];
  }
  int total;
  const int below = block_scan_once<NT>(mine, s.scan[0], total);
  const int above = total - below - mine;  // keys in higher threads' bins
  if (above < kk && kk <= above + mine) {  // exactly one thread
    int acc = above;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (acc < kk && kk <= acc + c[j]) {
        s.sel[0] = tid * BPT + j;
        s.sel[1] = kk - acc;
      }
      acc += c[j];
    }
  }
  __syncthreads();
  const int b1 = s.sel[0], r1 = s.sel[1];
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] >= 0 && (key[e] >> 5) == b1) atomicAdd(&s.h2[key[e] & 31], 1);
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    const int cb = lane < kSelSub ? s.h2[kSelSub - 1 - lane] : 0;
    const int sc = wave_inclusive_scan(cb);  // keys of b1 at or above bin 31 - lane
    const uint64_t hit = __ballot(lane < kSelSub && sc >= r1);
    const int l = __builtin_ctzll(hit);
    if (lane == l) {
      s.sel[0] = b1 * kSelSub + (kSelSub - 1 - l);
      s.sel[1] = r1 - (sc - cb);
    }
  }
  __syncthreads();
  const int tau = s.sel[0], r = s.sel[1];  // r >= 1
  int ties = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) ties += key[e] == tau ? 1 : 0;
  int tie_total;
  const int tr = block_scan_once<NT>(ties, s.scan[1], tie_total);
  if (tr < r && r <= tr + ties) {  // exactly one thread holds the r-th tie
    int n = tr, at = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (key[e] == tau) {
        ++n;
        if (n == r) at = (int)(k0 + e);
      }
    }
    s.sel[2] = at;
  }
  __syncthreads();
  tau_out = tau;
  istar_out = s.sel[2];
  __syncthreads();  // the next row's select may overwrite sel
}

}  // namespace sa
