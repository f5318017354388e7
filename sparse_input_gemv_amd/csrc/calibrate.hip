// Threshold calibration for a target sparsity (TEAL README, Inference Usage
// and Accuracy Usage step 1: per-layer activation histograms map a sparsity
// to a threshold).
//
// The histogram has one bin per fp16 magnitude (15-bit key), so the two
// order statistics around the quantile position are found exactly: a
// two-level radix select (256 bins of the high 8 key bits, then 128 bins of
// the low 7) over the samples, in one workgroup, gives rank lo and, from the
// same second pass, rank lo + 1 unless that one lies in a later high bin
// (then a second select).  The linear interpolation
// is done in fp64, operation by operation, and rounded once to fp32.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kCalThreads = 1024;

// Samples held in registers: up to kCalThreads x kCalRun of them, thread t
// holding the run from t kCalRun (loaded once for all four passes); larger
// sample sets are read from memory in every pass.
constexpr int kCalRun = 16;
struct RegKeys {
  int key[kCalRun];  // -1 past the end
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int e = 0; e < kCalRun; ++e)
      if (key[e] >= 0) f(key[e]);
  }
};
struct MemKeys {
  const uint16_t* smp;
  int64_t n;
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
    for (int64_t i = threadIdx.x; i < n; i += kCalThreads) f(mag_key(smp[i]));
  }
};

// Key of the r-th smallest magnitude (0-based), and in *next the key of
// rank r + 1 when the second pass already holds it (rank r + 1 in the same
// 128-key bin), else -1.  All threads call it.
template <typename Keys>
__device__ int select_rank(const Keys& keys, int64_t r, int* hist, int* sel, int* next) {
  const int tid = (int)threadIdx.x;
  for (int i = tid; i < 256; i += kCalThreads) hist[i] = 0;
  __syncthreads();
  keys.each([&](int key) { atomicAdd(&hist[key >> 7], 1); });
  __syncthreads();
  if (tid < kWave) {
    // lane l holds bins 4l..4l+3; C(b) = count in bins <= b.  The bins with
    // C(b) <= r form a prefix; the selected bin is the first one after it.
    int c[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = hist[tid * 4 + j];
      s += c[j];
    }
    int pre = s;  // inclusive prefix over lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(pre, o, kWave);
      if (tid >= o) pre += t;
    }
    const int cbel = pre - s;  // C(4l - 1)
    int C = cbel, nb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      C += c[j];
      nb += (C <= r) ? 1 : 0;
    }
    int b1 = nb;
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) b1 += __shfl_xor(b1, o, kWave);
    // b1 = first bin with C(b) > r; its owner lane computes C(b1 - 1)
    int mine = cbel;
#pragma unroll
    for (int j = 0; j < 3; ++j) mine += (j < (b1 & 3)) ? c[j] : 0;
    const int below = __shfl(mine, (b1 >> 2) & (kWave - 1), kWave);
    if (tid == 0) {
      sel[0] = b1;
      sel[1] = below;
    }
  }
  __syncthreads();
  const int b1 = sel[0];
  const int below = sel[1];
  __syncthreads();
  for (int i = tid; i < 128; i += kCalThreads) hist[i] = 0;
  __syncthreads();
  keys.each([&](int key) {
    if ((key >> 7) == b1) atomicAdd(&hist[key & 127], 1);
  });
  __syncthreads();
  if (tid < kWave) {
    const int c0 = hist[tid * 2], c1 = hist[tid * 2 + 1];
    int pre = c0 + c1;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(pre, o, kWave);
      if (tid >= o) pre += t;
    }
    const int C0 = below + pre - c1;  // count <= bin 2l
    const int C1 = below + pre;       // count <= bin 2l+1
    int nb = (C0 <= r ? 1 : 0) + (C1 <= r ? 1 : 0);
    int nb1 = (C0 <= r + 1 ? 1 : 0) + (C1 <= r + 1 ? 1 : 0);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      nb += __shfl_xor(nb, o, kWave);
      nb1 += __shfl_xor(nb1, o, kWave);
    }
    if (tid == 0) {
      sel[2] = (b1 << 7) | nb;
      sel[3] = nb1 < 128 ? ((b1 << 7) | nb1) : -1;
    }
  }
  __syncthreads();
  const int key = sel[2];
  *next = sel[3];
  __syncthreads();
  return key;
}

__device__ float interpolate(int64_t n, double s, int key_lo, int key_hi) {
#pragma clang fp contract(off)
  const double h = (double)(n - 1) * s;
  double lo = floor(h);
  if (lo < 0.0) lo = 0.0;
  if (lo > (double)(n - 1)) lo = (double)(n - 1);
  const double frac = h - lo;
  const double vlo = (double)h2f((uint16_t)key_lo);
  const double vhi = (double)h2f((uint16_t)key_hi);
  const double diff = vhi - vlo;
  const double q = vlo + frac * diff;
  return (float)q;
}

__global__ __launch_bounds__(kCalThreads) void k_calibrate(const uint16_t* __restrict__ smp,
                                                            int64_t n, double s,
                                                            float* __restrict__ t_out) {
  __shared__ int hist[256];
  __shared__ int sel[4];
  double h = (double)(n - 1) * s;
  int64_t lo = (int64_t)floor(h);
  if (lo < 0) lo = 0;
  if (lo > n - 1) lo = n - 1;
  const int64_t hi = (lo + 1 < n) ? lo + 1 : n - 1;
  int key_lo, key_hi, next;
  if (n <= (int64_t)kCalThreads * kCalRun) {
    RegKeys keys;
    const int64_t k0 = (int64_t)threadIdx.x * kCalRun;
    uint16_t v[kCalRun];
    load_run<kCalRun>(smp, k0, n, (reinterpret_cast<uintptr_t>(smp) & 15u) == 0, v);
#pragma unroll
    for (int e = 0; e < kCalRun; ++e) keys.key[e] = k0 + e < n ? mag_key(v[e]) : -1;
    key_lo = select_rank(keys, lo, hist, sel, &next);
    key_hi = (hi == lo) ? key_lo : next >= 0 ? next : select_rank(keys, hi, hist, sel, &next);
  } else {
    const MemKeys keys{smp, n};
    key_lo = select_rank(keys, lo, hist, sel, &next);
    key_hi = (hi == lo) ? key_lo : next >= 0 ? next : select_rank(keys, hi, hist, sel, &next);
  }
  if (threadIdx.x == 0) t_out[0] = interpolate(n, s, key_lo, key_hi);
}

}  // namespace

hipError_t launch_calibrate(const uint16_t* samples, int64_t n, double s, float* t_out,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_calibrate, dim3(1), dim3(kCalThreads), 0, st, samples, n, s, t_out);
  return hipGetLastError();
}

}  // namespace sa
