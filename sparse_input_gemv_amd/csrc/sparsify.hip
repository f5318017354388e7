// Activation sparsifiers for gfx950: magnitude threshold, per-token Top-K and
// N:M.  One pass over the activation; kept entries are compacted in ascending
// order with wave64 ballots, lane prefix counts (mbcnt) and an LDS scan of
// the per-wave totals.
//
// Pages: TEAL (README, Abstract) -- magnitude threshold of hidden states;
// Q-Sparse (author replies) -- per-token Top-K (answer comparing with MoE)
// and N:M over consecutive entries (answer on batched inference); the
// flexible N:M activation-sparsity summary, section 2 (methodology) -- N of
// every M kept, scored by |activation|.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int kSparsifyThreads = 1024;

// Writes the kept entries of one run per thread (bit e of `bits` <-> element
// k0+e) at their ascending positions, and the bitmask words of the run.
// Threads cover consecutive runs, so thread order is index order.
template <int NT, int E>
__device__ __forceinline__ void compact_run(uint64_t bits, const uint16_t (&v)[E], int64_t k0,
                                            int64_t d, int& base, int* scan,
                                            int32_t* __restrict__ ir, uint16_t* __restrict__ vr,
                                            uint32_t* __restrict__ mr) {
  int total;
  int pos = base + block_exclusive_scan<NT>(__popcll(bits), scan, total);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((bits >> e) & 1ull) {
      ir[pos] = (int32_t)(k0 + e);
      vr[pos] = v[e];
      ++pos;
    }
  }
  if (mr != nullptr) {
    if constexpr (E == 16) {
      // two neighbouring threads hold the two halves of one 32-bit word
      uint32_t other = (uint32_t)__shfl_xor((int)bits, 1, kWave);
      if ((threadIdx.x & 1) == 0 && k0 < d) mr[k0 >> 5] = (uint32_t)bits | (other << 16);
    } else {
#pragma unroll
      for (int q = 0; q < E / 32; ++q)
        if (k0 + 32 * q < d) mr[(k0 >> 5) + q] = (uint32_t)(bits >> (32 * q));
    }
  }
  base += total;
}

// A whole row in one pass (d <= NT * E): the mask words as compact_run
// writes them, the kept entries to LDS at their list positions, then out
// with coalesced stores (each thread's own scattered stores had cost ~1.7
// us at d = 11008).  Returns the kept count.  Every thread must call it.
template <int NT, int E>
__device__ __forceinline__ int compact_row_lds(uint64_t bits, const uint16_t (&v)[E], int64_t k0,
                                               int64_t d, int* scan, int32_t* sidx,
                                               uint16_t* sval, int32_t* __restrict__ ir,
                                               uint16_t* __restrict__ vr,
                                               uint32_t* __restrict__ mr) {
  const int tid = (int)threadIdx.x;
  if (mr != nullptr) {
    if constexpr (E < 32) {
      // 32 / E neighbouring threads hold the parts of one 32-bit word
      static_assert(32 % E == 0, "runs tile the mask words");
      constexpr int G = 32 / E;
      uint32_t w = (uint32_t)bits;
#pragma unroll
      for (int j = 1; j < G; ++j) w |= (uint32_t)__shfl_down((int)bits, j, kWave) << (E * j);
      if (tid % G == 0 && k0 < d) mr[k0 >> 5] = w;
    } else {
#pragma unroll
      for (int q = 0; q < E / 32; ++q)
        if (k0 + 32 * q < d) mr[(k0 >> 5) + q] = (uint32_t)(bits >> (32 * q));
    }
  }
  int kept;
  int pos = block_scan_once<NT>(__popcll(bits), scan, kept);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((bits >> e) & 1ull) {
      sidx[pos] = (int32_t)(k0 + e);
      sval[pos] = v[e];
      ++pos;
    }
  }
  __syncthreads();
  for (int i = tid; i < kept; i += NT) {
    ir[i] = sidx[i];
    vr[i] = sval[i];
  }
  return kept;
}

// keep_i = (|x_i| >= t) && (x_i != 0), compared in fp32 (fp16 widening is
// exact, so this is the exact comparison).  One workgroup per row.  A row
// that fits one pass (d <= NT * E) stages its list in LDS and writes it out
// with coalesced stores; longer rows compact pass by pass.
template <int NT, int E>
__global__ __launch_bounds__(NT) void k_sparsify_threshold(
    const uint16_t* __restrict__ x, int64_t d, float t, uint32_t* __restrict__ mask,
    int32_t* __restrict__ idx, uint16_t* __restrict__ val, int32_t* __restrict__ nnz,
    int64_t cap, int vec) {
  __shared__ int scan[NT / kWave];
  __shared__ __align__(16) int32_t sidx[NT * E];
  __shared__ __align__(16) uint16_t sval[NT * E];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  int32_t* ir = idx + row * cap;
  uint16_t* vr = val + row * cap;
  uint32_t* mr = mask ? mask + row * ((d + 31) >> 5) : nullptr;
  if (d <= (int64_t)NT * E) {
    const int64_t k0 = (int64_t)threadIdx.x * E;
    uint16_t v[E];
    load_run<E>(xr, k0, d, vec != 0, v);
    uint64_t bits = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint16_t b = v[e];
      const bool keep = (k0 + e < d) && (mag_key(b) != 0) && (fabsf(h2f(b)) >= t);
      bits |= (uint64_t)keep << e;
    }
    const int kept = compact_row_lds<NT, E>(bits, v, k0, d, scan, sidx, sval, ir, vr, mr);
    if (threadIdx.x == 0) nnz[row] = kept;
    return;
  }
  int base = 0;
  for (int64_t c0 = 0; c0 < d; c0 += (int64_t)NT * E) {
    const int64_t k0 = c0 + (int64_t)threadIdx.x * E;
    uint16_t v[E];
    load_run<E>(xr, k0, d, vec != 0, v);
    uint64_t bits = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint16_t b = v[e];
      const bool keep = (k0 + e < d) && (mag_key(b) != 0) && (fabsf(h2f(b)) >= t);
      bits |= (uint64_t)keep << e;
    }
    compact_run<NT, E>(bits, v, k0, d, base, scan, ir, vr, mr);
  }
  if (threadIdx.x == 0) nnz[row] = base;
}

// Two-pass form of the threshold kind for long rows (kScoredThrMinD <= d
// <= kScoredThrMaxD): the scores need x, mu and the fp64 weight norms (12
// bytes per entry), which one workgroup per row reads through one CU.  The
// first pass (k_scored_thr_bits) spreads the decisions over chunks of
// kScoredThrChunk entries, one workgroup each: it writes the mask and
// stages the keep bits (as half-words at the head of the row's val buffer)
// and the chunk's fp64 sums of x'^2 and kept x'^2 (as int32 pairs at the
// head of the row's idx buffer; the row holds cap >= d entries of each).
// The second pass, k_sparsify_scored<.., true>, reads them back and writes
// the list from x and mu alone.
constexpr int kScoredThrChunk = 1024;
constexpr int64_t kScoredThrMinD = 4096;
constexpr int64_t kScoredThrMaxD = 65536;

__global__ __launch_bounds__(256) void k_scored_thr_bits(
    const uint16_t* __restrict__ x, int64_t d, const uint16_t* __restrict__ mu,
    const double* __restrict__ cn, double t, uint32_t* __restrict__ mask,
    int32_t* __restrict__ idx, uint16_t* __restrict__ val, int64_t cap) {
  constexpr int E = kScoredThrChunk / 256;  // 4 entries per thread
  __shared__ double ws[2][256 / kWave];
  const int64_t row = blockIdx.x, c = blockIdx.y;
  const int tid = (int)threadIdx.x;
  const int64_t k0 = c * kScoredThrChunk + (int64_t)tid * E;
  const uint16_t* xr = x + row * d;
  uint32_t bits = 0;
  double s_all = 0.0, s_kept = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t k = k0 + e;
    if (k < d) {
      uint16_t v = xr[k];
      if (mu != nullptr) v = f2h(h2f(v) - h2f(mu[k]));
      const double a = fabs((double)h2f(v));
      const bool keep = (cn != nullptr ? a * cn[k] : a) >= t && h2f(v) != 0.f;
      const double q = (double)h2f(v) * (double)h2f(v);
      s_all += q;
      s_kept += keep ? q : 0.0;
      bits |= (uint32_t)keep << e;
    }
  }
  // 8 neighbouring threads hold one 32-bit word
  uint32_t w = bits << (E * (tid % 8));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) w |= (uint32_t)__shfl_xor((int)w, o, kWave);
  const int64_t wi = (c * kScoredThrChunk + (int64_t)tid * E) >> 5;
  if (tid % 8 == 0 && wi * 32 < d) {
    if (mask != nullptr) mask[row * ((d + 31) >> 5) + wi] = w;
    uint16_t* vr = val + row * cap;
    vr[2 * wi] = (uint16_t)(w & 0xffffu);
    if (wi * 32 + 16 < d) vr[2 * wi + 1] = (uint16_t)(w >> 16);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    s_all += __shfl_xor(s_all, o, kWave);
    s_kept += __shfl_xor(s_kept, o, kWave);
  }
  if (lane_id() == 0) {
    ws[0][tid / kWave] = s_all;
    ws[1][tid / kWave] = s_kept;
  }
  __syncthreads();
  if (tid == 0) {
    double a = 0.0, k = 0.0;
    for (int i = 0; i < 256 / kWave; ++i) {
      a += ws[0][i];
      k += ws[1][i];
    }
    int32_t* ir = idx + row * cap + 4 * c;
    const uint64_t ab = __builtin_bit_cast(uint64_t, a), kb = __builtin_bit_cast(uint64_t, k);
    ir[0] = (int32_t)(uint32_t)ab;
    ir[1] = (int32_t)(uint32_t)(ab >> 32);
    ir[2] = (int32_t)(uint32_t)kb;
    ir[3] = (int32_t)(uint32_t)(kb >> 32);
  }
}

// Weight-aware selection with a static shift (the flexible N:M
// activation-sparsity summary, section 2: WT and Amber-Pruner score entries
// by the weight they multiply; S-PTS shifts activations towards zero; VAR
// restores the output scale).  Per row, per entry:
//   x' = fp16(fp32(x) - fp32(mu))   (mu null: x' = x)
//   score = |x'| * c in fp64         (c null: |x'|; the fp64 product is
//                                     correctly rounded, one operation)
//   threshold kind: keep iff score >= t and x' != 0
//   N:M kinds (k_sparsify_scored_nm below): keep the n largest scores of
//           every M consecutive entries, ties to the lower index
// This kernel takes the threshold kind, one workgroup per row: the kept x'
// are compacted as the threshold sparsifier does.  alpha[row] =
// sqrt(sum x'^2 / sum_kept x'^2) (1 when nothing is kept), in fp64.
//
// PRE (the second pass of the two-pass form below): the keep bits and the
// per-chunk sums come from k_scored_thr_bits, staged in this row's own val
// and idx buffers; they are read into LDS first, then the list overwrites
// them.  The mask was written by the first pass.
template <int NT, int E, bool PRE = false>
__global__ __launch_bounds__(NT) void k_sparsify_scored(
    const uint16_t* __restrict__ x, int64_t d, const uint16_t* __restrict__ mu,
    const double* __restrict__ cn, double t, uint32_t* __restrict__ mask,
    int32_t* __restrict__ idx, uint16_t* __restrict__ val, int32_t* __restrict__ nnz,
    float* __restrict__ alpha, int64_t cap, int vec, int vec_mu) {
  __shared__ int scan[NT / kWave];
  __shared__ double sums[2][NT / kWave];
  __shared__ __align__(16) int32_t sidx[NT * E];
  __shared__ __align__(16) uint16_t sval[NT * E];
  __shared__ uint16_t pbits[PRE ? kScoredThrMaxD / 16 : 1];
  const bool one_pass = d <= (int64_t)NT * E;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  int32_t* ir = idx + row * cap;
  uint16_t* vr = val + row * cap;
  uint32_t* mr = (mask && !PRE) ? mask + row * ((d + 31) >> 5) : nullptr;
  int base = 0;
  double s_all = 0.0, s_kept = 0.0;
  if constexpr (PRE) {
    // every staged value is read before the first list write
    const int64_t nh = (d + 15) / 16;
    for (int64_t i = threadIdx.x; i < nh; i += NT) pbits[i] = vr[i];
    if (threadIdx.x == 0 && alpha != nullptr) {
      const int64_t nc = (d + kScoredThrChunk - 1) / kScoredThrChunk;
      double a = 0.0, k = 0.0;
      for (int64_t c = 0; c < nc; ++c) {  // chunk order: a fixed sum
        a += __builtin_bit_cast(double, (uint64_t)(uint32_t)ir[4 * c] |
                                            ((uint64_t)(uint32_t)ir[4 * c + 1] << 32));
        k += __builtin_bit_cast(double, (uint64_t)(uint32_t)ir[4 * c + 2] |
                                            ((uint64_t)(uint32_t)ir[4 * c + 3] << 32));
      }
      sums[0][0] = a;
      sums[1][0] = k;
    }
    __syncthreads();
  }
  for (int64_t c0 = 0; c0 < d; c0 += (int64_t)NT * E) {
    const int64_t k0 = c0 + (int64_t)threadIdx.x * E;
    uint16_t v[E];
    load_run<E>(xr, k0, d, vec != 0, v);
    if (mu != nullptr) {
      uint16_t m[E];
      load_run<E>(mu, k0, d, vec_mu != 0, m);
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = (k0 + e < d) ? f2h(h2f(v[e]) - h2f(m[e])) : (uint16_t)0;
    }
    uint64_t bits = 0;
    if constexpr (PRE) {
      static_assert(E == 16, "a thread's run is one staged half-word of bits");
      bits = k0 < d ? (uint64_t)pbits[k0 / 16] : 0ull;
    } else {
      double sc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double a = fabs((double)h2f(v[e]));
        sc[e] = (k0 + e < d) ? (cn != nullptr ? a * cn[k0 + e] : a) : 0.0;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool keep = (k0 + e < d) && sc[e] >= t && h2f(v[e]) != 0.f;
        bits |= (uint64_t)keep << e;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double q = (double)h2f(v[e]) * (double)h2f(v[e]);
        s_all += (k0 + e < d) ? q : 0.0;
        s_kept += ((bits >> e) & 1ull) ? q : 0.0;
      }
    }
    if (one_pass)
      base = compact_row_lds<NT, E>(bits, v, k0, d, scan, sidx, sval, ir, vr, mr);
    else
      compact_run<NT, E>(bits, v, k0, d, base, scan, ir, vr, mr);
  }
  if (PRE && alpha != nullptr && threadIdx.x == 0)
    alpha[row] = sums[1][0] > 0.0 ? (float)sqrt(sums[0][0] / sums[1][0]) : 1.f;
  if (!PRE && alpha != nullptr) {
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      s_all += __shfl_xor(s_all, o, kWave);
      s_kept += __shfl_xor(s_kept, o, kWave);
    }
    const int w = (int)threadIdx.x / kWave;
    if (lane_id() == 0) {
      sums[0][w] = s_all;
      sums[1][w] = s_kept;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double a = 0.0, k = 0.0;
      for (int i = 0; i < NT / kWave; ++i) {
        a += sums[0][i];
        k += sums[1][i];
      }
      alpha[row] = k > 0.0 ? (float)sqrt(a / k) : 1.f;
    }
  }
  if (threadIdx.x == 0) nnz[row] = base;
}

// The N:M kinds of k_sparsify_scored spread over many workgroups: every
// group keeps exactly n entries, so group g's survivors go to slots
// [g n, g n + n) of the row's list whatever the other groups keep, and no
// compaction across groups is needed.  One thread per group of M, one wave
// per workgroup (64 groups).  The selection is k_sparsify_scored's (n rounds
// of taking the group's largest score not yet taken, the first of equal
// scores), so the masks and lists are the same bit for bit.  The variance
// correction needs the whole row: k_scored_alpha, launched after, sums x'^2
// over the row and over its kept values.
constexpr int kScoredNmGroups = 64;

template <int M>
__global__ __launch_bounds__(kScoredNmGroups) void k_sparsify_scored_nm(
    const uint16_t* __restrict__ x, int64_t d, const uint16_t* __restrict__ mu,
    const double* __restrict__ cn, int n, uint32_t* __restrict__ mask,
    int32_t* __restrict__ idx, uint16_t* __restrict__ val, int32_t* __restrict__ nnz,
    int64_t cap, int vec, int vec_mu) {
  static_assert(M == 4 || M == 8 || M == 16 || M == 32, "group sizes");
  const int64_t row = blockIdx.x;  // rows in x (up to 2^31 - 1), a row's chunks in y
  const int lane = (int)threadIdx.x;
  const int64_t ng = d / M;
  const int64_t g = (int64_t)blockIdx.y * kScoredNmGroups + lane;
  const bool ok = g < ng;
  const int64_t k0 = (ok ? g : 0) * M;
  const uint16_t* xr = x + row * d;
  uint16_t v[M];
  load_run<M>(xr, k0, d, vec != 0, v);
  if (mu != nullptr) {
    uint16_t m[M];
    load_run<M>(mu, k0, d, vec_mu != 0, m);
#pragma unroll
    for (int e = 0; e < M; ++e) v[e] = f2h(h2f(v[e]) - h2f(m[e]));
  }
  double sc[M];
#pragma unroll
  for (int e = 0; e < M; ++e) {
    const double a = fabs((double)h2f(v[e]));
    sc[e] = cn != nullptr ? a * cn[k0 + e] : a;
  }
  uint32_t bits = 0;
  for (int it = 0; it < n; ++it) {
    int best = 0;
    double bs = -1.0;  // scores are >= 0
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const bool take = ((bits >> j) & 1u) == 0 && sc[j] > bs;
      bs = take ? sc[j] : bs;
      best = take ? j : best;
    }
    bits |= 1u << best;
  }
  if (!ok) bits = 0;
  if (ok) {
    int32_t* ir = idx + row * cap + g * n;
    uint16_t* vr = val + row * cap + g * n;
    int j = 0;
#pragma unroll
    for (int e = 0; e < M; ++e) {
      if ((bits >> e) & 1u) {
        ir[j] = (int32_t)(k0 + e);
        vr[j] = v[e];
        ++j;
      }
    }
  }
  if (mask != nullptr) {
    // a mask word holds 32 / M consecutive groups, i.e. lanes: OR their bits
    constexpr int GPW = 32 / M;
    uint32_t w = bits << (M * (lane % GPW));
#pragma unroll
    for (int o = 1; o < GPW; o <<= 1) w |= (uint32_t)__shfl_xor((int)w, o, kWave);
    const int64_t words = (d + 31) >> 5;
    const int64_t wi = (g * M) >> 5;
    if (lane % GPW == 0 && wi < words) mask[row * words + wi] = w;
  }
  if (blockIdx.y == 0 && lane == 0) nnz[row] = (int32_t)(ng * n);
}

// alpha[row] = sqrt(sum x'^2 / sum_kept x'^2), 1 when the kept sum is 0: both
// sums in fp64 over the row (x' recomputed from x and mu) and over its
// nk kept values, in a fixed order (thread-strided, then a wave and a
// workgroup tree).
__global__ __launch_bounds__(1024) void k_scored_alpha(const uint16_t* __restrict__ x, int64_t d,
                                                        const uint16_t* __restrict__ mu,
                                                        const uint16_t* __restrict__ val,
                                                        int64_t cap, int64_t nk,
                                                        float* __restrict__ alpha, int vec,
                                                        int vec_mu, int vec_val) {
  __shared__ double sums[2][1024 / kWave];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  const uint16_t* vr = val + row * cap;
  // Runs of 8 per thread (16-byte loads where aligned), two runs in flight
  // per pass, so a pass costs one memory round trip.
  double a = 0.0, k = 0.0;
  const bool vx = vec != 0, vv = vec_val != 0;
  for (int64_t i0 = (int64_t)threadIdx.x * 8; i0 < d; i0 += 2 * 1024 * 8) {
    uint16_t xa[8], xb[8], ma[8], mb[8];
    const int64_t i1 = i0 + 1024 * 8;
    load_run<8>(xr, i0, d, vx, xa);
    load_run<8>(xr, i1, d, vx, xb);
    if (mu != nullptr) {
      load_run<8>(mu, i0, d, vec_mu != 0, ma);
      load_run<8>(mu, i1, d, vec_mu != 0, mb);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t p = mu != nullptr ? f2h(h2f(xa[e]) - h2f(ma[e])) : xa[e];
      const uint16_t q = mu != nullptr ? f2h(h2f(xb[e]) - h2f(mb[e])) : xb[e];
      const double dp = (i0 + e < d) ? (double)h2f(p) : 0.0;
      const double dq = (i1 + e < d) ? (double)h2f(q) : 0.0;
      a += dp * dp;
      a += dq * dq;
    }
  }
  for (int64_t i0 = (int64_t)threadIdx.x * 8; i0 < nk; i0 += 1024 * 8) {
    uint16_t va[8];
    load_run<8>(vr, i0, nk, vv, va);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double q = (double)h2f(va[e]);  // entries past nk read as 0
      k += q * q;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o, kWave);
    k += __shfl_xor(k, o, kWave);
  }
  const int w = (int)threadIdx.x / kWave;
  if (lane_id() == 0) {
    sums[0][w] = a;
    sums[1][w] = k;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ta = 0.0, tk = 0.0;
    for (int i = 0; i < 1024 / kWave; ++i) {
      ta += sums[0][i];
      tk += sums[1][i];
    }
    alpha[row] = tk > 0.0 ? (float)sqrt(ta / tk) : 1.f;
  }
}

// Exactly k survivors per row: the k largest magnitudes, ties to the lower
// index (fp16 magnitudes compared exactly as 15-bit keys; -0 == +0); rows
// longer than 4096 entries (shorter ones take the radix select below).
//  1. One LDS bin per key value (2^15 bins, 128 KB); a single pass of LDS
//     atomics counts every key.
//  2. Each thread owns 32 consecutive keys' bins.  A workgroup scan of the
//     threads' sums, read from the top, finds the thread, and its wave the
//     bin, where the count of larger keys reaches k: that bin is tau, the
//     k-th largest key, and r = k - #(keys > tau) of its entries survive.
//     A thread's bins are stored as int4 runs a workgroup-width apart (bin
//     address below), so a wave reads 64 consecutive int4 at a time, free
//     of LDS bank conflicts (contiguous runs would put the 128-byte stride
//     between threads, and so a whole wave, on the same four banks).
//  3. i* is the index of the r-th entry equal to tau in index order, found
//     by a scan of the threads' counts of such entries.
// Entry i survives iff key_i > tau, or key_i == tau and i <= i* (k = 0:
// tau = 2^15, i* = -1, nothing survives).  Outputs: the pair (tau, i*) per
// row in `cut` (may be NULL), the bitmask, and the compacted list (staged in
// LDS for d <= NT * 16, so it leaves in coalesced stores).  One workgroup
// per row; each thread keeps E keys.
constexpr int kTopkBins = 1 << 15;

// LDS word of key `key`'s bin: thread t = key / BPT owns the int4 runs
// q * NT + t, q < BPT / 4, holding its keys in order.
template <int NT, int BPT>
__device__ __forceinline__ int topk_bin(int key) {
  return ((((key % BPT) >> 2) * NT + key / BPT) << 2) | (key & 3);
}

template <int NT, int E>
__global__ __launch_bounds__(NT) void k_topk(const uint16_t* __restrict__ x, int64_t d, int64_t k,
                                             int32_t* __restrict__ cut,
                                             uint32_t* __restrict__ mask,
                                             int32_t* __restrict__ idx,
                                             uint16_t* __restrict__ val,
                                             int32_t* __restrict__ nnz, int64_t cap, int vec) {
  __shared__ __align__(16) int hist[kTopkBins];  // the counts; then the output staging
  __shared__ int scan[3][NT / kWave];             // one per block scan
  __shared__ int sel[3];                          // tau, ties to keep, i*
  constexpr int BPT = kTopkBins / NT;  // bins per thread
  static_assert(BPT % 4 == 0 && kTopkBins % NT == 0 && BPT <= kWave, "bins split into int4 runs");
  const int tid = (int)threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  const int64_t k0 = (int64_t)tid * E;
  int4* h4 = reinterpret_cast<int4*>(hist);
  uint16_t v[E];
  load_run<E>(xr, k0, d, vec != 0, v);
  // clear the bins while the row's loads are in flight
  if (k > 0)
    for (int i = tid; i < kTopkBins / 4; i += NT) h4[i] = int4{0, 0, 0, 0};
  __builtin_amdgcn_sched_barrier(0);
  int key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (k0 + e < d) ? mag_key(v[e]) : -1;

  int tau = kTopkBins, istar = -1;  // k == 0: no key reaches tau
  if (k > 0) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] >= 0) atomicAdd(&hist[topk_bin<NT, BPT>(key[e])], 1);
    __syncthreads();
    int c[BPT];
#pragma unroll
    for (int q = 0; q < BPT / 4; ++q) {
      const int4 t4 = h4[q * NT + tid];
      c[4 * q] = t4.x;
      c[4 * q + 1] = t4.y;
      c[4 * q + 2] = t4.z;
      c[4 * q + 3] = t4.w;
    }
    int mine = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) mine += c[j];
    int total;  // == the number of entries, so k and every count fit an int
    const int below = block_scan_once<NT>(mine, scan[0], total);
    const int above = total - below - mine;  // keys in higher threads' bins
    const int kk = (int)k;
    // Exactly one thread t* has above < k <= above + mine.  Its wave finds
    // the bin: lane l < BPT reads bin BPT*t* + (BPT-1-l) (top first) from
    // LDS, an inclusive scan over those lanes gives the count of keys at or
    // above each bin, and the first lane where above + count reaches k
    // names tau; the keys above tau number gt, and r = k - gt of tau's own
    // entries survive.
    const uint64_t cross = __ballot(above < kk && kk <= above + mine);
    if (cross != 0) {  // uniform: the wave holding t*
      const int src = __builtin_ctzll(cross);
      const int ts = __builtin_amdgcn_readfirstlane((int)threadIdx.x - lane_id() + src);
      const int ab = __builtin_amdgcn_readlane(above, src);
      const int lane = lane_id();
      const int jb = BPT - 1 - (lane & (BPT - 1));
      const int cb = lane < BPT ? hist[topk_bin<NT, BPT>(ts * BPT + jb)] : 0;
      const int sc = BPT <= 16 ? row16_inclusive_scan(cb) : wave_inclusive_scan(cb);
      const uint64_t hit = __ballot(lane < BPT && ab + sc >= kk);
      const int l = __builtin_ctzll(hit);
      if (lane == l) {
        sel[0] = ts * BPT + jb;
        sel[1] = kk - (ab + sc - cb);
      }
    }
    __syncthreads();
    tau = __builtin_amdgcn_readfirstlane(sel[0]);
    const int r = __builtin_amdgcn_readfirstlane(sel[1]);  // >= 1
    int ties = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) ties += (key[e] == tau) ? 1 : 0;
    int tie_total;
    const int tr = block_scan_once<NT>(ties, scan[1], tie_total);
    if (tr < r && r <= tr + ties) {  // exactly one thread holds the r-th tie
      int n = tr, at = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (key[e] == tau) {
          ++n;
          if (n == r) at = (int)(k0 + e);
        }
      }
      sel[2] = at;
    }
    __syncthreads();
    istar = sel[2];
  }
  if (cut != nullptr && tid == 0) {
    cut[2 * row] = tau;
    cut[2 * row + 1] = istar;
  }
  if (idx == nullptr && mask == nullptr) {
    if (nnz != nullptr && tid == 0) nnz[row] = (int32_t)k;
    return;
  }

  uint64_t bits = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool keep = key[e] > tau || (key[e] == tau && k0 + e <= (int64_t)istar);
    bits |= (uint64_t)keep << e;
  }
  int32_t* ir = idx + row * cap;
  uint16_t* vr = val + row * cap;
  uint32_t* mr = mask ? mask + row * ((d + 31) >> 5) : nullptr;
  if constexpr ((int64_t)NT * E * 6 <= (int64_t)kTopkBins * 4) {
    // stage the list in LDS (the counts are no longer read), then copy it out
    if (mr != nullptr) {
      if constexpr (E == 16) {
        const uint32_t other = (uint32_t)__shfl_xor((int)bits, 1, kWave);
        if ((tid & 1) == 0 && k0 < d) mr[k0 >> 5] = (uint32_t)bits | (other << 16);
      } else {
#pragma unroll
        for (int q = 0; q < E / 32; ++q)
          if (k0 + 32 * q < d) mr[(k0 >> 5) + q] = (uint32_t)(bits >> (32 * q));
      }
    }
    int kept;
    int pos = block_scan_once<NT>(__popcll(bits), scan[2], kept);
    int32_t* sidx = hist;
    uint16_t* sval = reinterpret_cast<uint16_t*>(hist + NT * E);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((bits >> e) & 1ull) {
        sidx[pos] = (int32_t)(k0 + e);
        sval[pos] = v[e];
        ++pos;
      }
    }
    __syncthreads();
    for (int i = tid; i < kept; i += NT) {
      ir[i] = sidx[i];
      vr[i] = sval[i];
    }
  } else {
    int base = 0;
    compact_run<NT, E>(bits, v, k0, d, base, scan[2], ir, vr, mr);
  }
  if (tid == 0) nnz[row] = (int32_t)k;
}

// Rows of up to 4096 entries: the two-pass radix select of wg_topk_cutoff,
// one workgroup of 512 threads per row -- k_topk_cut for the cutoff pairs
// alone (act_topk_cutoff and the two-launch Top-K GEMV), k_topk_radix for
// the lists.  Measured (d = 4096, batch 1): 3.0 us for the pairs and 4.7 us
// with the lists, against 4.5 and 6.6 us for k_topk, whose 128 KB of bins
// take longer to clear and scan.  Longer rows stay on k_topk: at d = 11008
// the radix select took 5.0 us with 1024 threads of 16 entries (5.0-5.2 us
// whether the first pass bins the keys' top 10, 11 or 12 bits, so LDS atomic
// contention is not the cause), 5.7 with 512 of 32, 8.0 with 256 of 48, and
// 6.3 with 1024 threads each holding every 1024th entry, against 4.6 for
// k_topk.
constexpr int kCutThreads = 512, kCutE = 8;
template <int NT, int E>
__global__ __launch_bounds__(NT) void k_topk_cut(const uint16_t* __restrict__ x, int64_t d,
                                                 int64_t k, int32_t* __restrict__ cut,
                                                 int32_t* __restrict__ nnz) {
  __shared__ SelLds lds;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  uint16_t v[E];
  load_run<E>(xr, (int64_t)threadIdx.x * E, d, (reinterpret_cast<uintptr_t>(xr) & 15u) == 0, v);
  int tau, istar;
  wg_topk_cutoff<NT, E>(v, d, k, lds, tau, istar);
  if (threadIdx.x == 0) {
    cut[2 * row] = tau;
    cut[2 * row + 1] = istar;
    if (nnz != nullptr) nnz[row] = (int32_t)k;
  }
}

// The lists of act_sparsify_topk (and its cutoff pairs where asked) for rows
// of up to 4096 entries: the same select, then the kept entries -- key >
// tau, or key == tau and index <= i* -- compacted through LDS.
template <int NT, int E>
__global__ __launch_bounds__(NT) void k_topk_radix(const uint16_t* __restrict__ x, int64_t d,
                                                   int64_t k, int32_t* __restrict__ cut,
                                                   uint32_t* __restrict__ mask,
                                                   int32_t* __restrict__ idx,
                                                   uint16_t* __restrict__ val,
                                                   int32_t* __restrict__ nnz, int64_t cap) {
  __shared__ SelLds lds;
  __shared__ int scan[NT / kWave];
  __shared__ __align__(16) int32_t sidx[NT * E];
  __shared__ __align__(16) uint16_t sval[NT * E];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  const int64_t k0 = (int64_t)threadIdx.x * E;
  uint16_t v[E];
  load_run<E>(xr, k0, d, (reinterpret_cast<uintptr_t>(xr) & 15u) == 0, v);
  int tau, istar;
  wg_topk_cutoff<NT, E>(v, d, k, lds, tau, istar);
  uint64_t bits = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int key = mag_key(v[e]);
    const bool keep = k0 + e < d && (key > tau || (key == tau && k0 + e <= (int64_t)istar));
    bits |= (uint64_t)keep << e;
  }
  compact_row_lds<NT, E>(bits, v, k0, d, scan, sidx, sval, idx + row * cap, val + row * cap,
                         mask ? mask + row * ((d + 31) >> 5) : nullptr);
  if (threadIdx.x == 0) {
    if (cut != nullptr) {
      cut[2 * row] = tau;
      cut[2 * row + 1] = istar;
    }
    nnz[row] = (int32_t)k;
  }
}

// N:M, M <= 8: each thread owns 8 consecutive entries (one 16-byte load),
// so its groups are its own.  An entry is kept iff fewer than n entries of
// its group rank before it, where j ranks before i iff |x_j| > |x_i|, or
// they are equal and j < i; the ranks are counted pairwise.  The flattened
// array is a sequence of groups because d % M == 0 and d % 32 == 0.
// Every group yields exactly n values, so a workgroup's 2048 entries give a
// fixed, contiguous run of 2048*n/M outputs: the kept values are placed in
// LDS at their slots and the run is written out with 16-byte stores.
constexpr int kNmThreads = 256;
constexpr int kNmPerBlock = kNmThreads * 8;

// Exchanges within an aligned quad of lanes by DPP quad permutes (a VALU
// operand modifier, no LDS round trip).  quad_perm control: lane i of the
// quad reads lane ((ctrl >> 2i) & 3).
template <int CTRL>
__device__ __forceinline__ int quad_perm(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
constexpr int kQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
constexpr int kQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);
template <int M>
__global__ __launch_bounds__(kNmThreads) void k_sparsify_nm(const uint16_t* __restrict__ x,
                                                            int64_t n8, int n,
                                                            uint32_t* __restrict__ mask,
                                                            uint16_t* __restrict__ val,
                                                            int vec_out) {
  __shared__ __align__(16) uint16_t outs[kNmPerBlock];
  const int tid = (int)threadIdx.x;
  const int64_t g8 = (int64_t)blockIdx.x * kNmThreads + tid;
  const bool active = g8 < n8;
  const int lane = lane_id();
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (active) raw = *reinterpret_cast<const u32x4*>(x + g8 * 8);
  uint16_t v[8];
  int key[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (uint16_t)(raw[i] & 0xffffu);
    v[2 * i + 1] = (uint16_t)(raw[i] >> 16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) key[i] = mag_key(v[i]);

  static_assert(M <= 8, "groups within a thread");
  uint32_t keep = 0;
  constexpr int GPT = 8 / M;
#pragma unroll
  for (int gi = 0; gi < GPT; ++gi) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int p = gi * M + i;
      int rank = 0;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int q = gi * M + j;
        rank += (key[q] > key[p] || (key[q] == key[p] && j < i)) ? 1 : 0;
      }
      if (rank < n) keep |= 1u << p;
    }
    // local group index gi of thread tid -> slots (tid*GPT + gi)*n ...
    if (active) {
      int slot = (tid * GPT + gi) * n;
#pragma unroll
      for (int i = 0; i < M; ++i)
        if ((keep >> (gi * M + i)) & 1u) outs[slot++] = v[gi * M + i];
    }
  }
  // four neighbouring threads (a lane quad) make one 32-bit mask word
  uint32_t w = keep << (8 * (lane & 3));
  w |= (uint32_t)quad_perm<kQuadXor1>((int)w);
  w |= (uint32_t)quad_perm<kQuadXor2>((int)w);
  if (active && (lane & 3) == 0) mask[g8 >> 2] = w;

  __syncthreads();
  // this workgroup's entries and outputs
  const int64_t first = (int64_t)blockIdx.x * kNmThreads;
  const int64_t nthr = (n8 - first) < kNmThreads ? (n8 - first) : kNmThreads;
  const int count = (int)(nthr * 8 / M) * n;
  uint16_t* dst = val + first * 8 / M * n;
  if (vec_out && (count % 8) == 0) {
    for (int i = tid; i < count / 8; i += kNmThreads)
      *reinterpret_cast<u32x4*>(dst + 8 * i) = *reinterpret_cast<const u32x4*>(outs + 8 * i);
  } else {
    for (int i = tid; i < count; i += kNmThreads) dst[i] = outs[i];
  }
}

// N:M, M = 16 / 32 with n != M / 2 (n = M / 2 takes k_sparsify_nm_half
// below): each thread takes two consecutive groups A and B whole
// (2M entries, M/4 16-byte loads) and works on both at once: entry i of A
// and entry i of B share one 32-bit register, A in the low half, so each
// compare-exchange of a sorting network over the M registers is one packed
// 16-bit max and one packed min for the two groups.  Batcher's odd-even
// merge sort puts each group's 15-bit magnitude keys in descending order;
// tau, the n-th largest, is entry n - 1.  The keys >= tau (one packed
// subtraction and its sign bits per register) are exactly the survivors
// unless ties at tau make more than n of them; then the surplus ties with
// the highest positions are dropped (ties go to the lower position).  The
// kept values are placed in LDS at their slots (group g's n outputs start
// at g * n) and leave in 16-byte stores, as above.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr int kNmPkThreads = 256;
constexpr int kNmPkBlocksPerCu = 4;  // workgroups of the grid per compute unit
// LDS region of one thread's outputs (its two groups' survivors, at most
// 2 M - 2 values) plus its spare slot, in fp16 units.  M + 1 dwords is odd,
// so the 64 lanes' regions start on 64 different banks: with regions of
// 2 n values (M / 2 or M dwords, a multiple of 8) the lanes' stores met on
// 4 to 8 banks.
template <int M>
constexpr int kNmPkRegion = 2 * M + 2;

__device__ __forceinline__ uint32_t pk_bits(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 pk_vec(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// Descending sort of N packed pairs, both halves at once (Batcher's
// odd-even merge sort: N = 16 takes 63 compare-exchanges, N = 32 takes 191).
template <int N>
__device__ __forceinline__ void pk_sort_desc(u16x2 (&s)[N]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1) {
#pragma unroll
    for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
      for (int j = k % p; j + k < N; j += 2 * k) {
#pragma unroll
        for (int i = 0; i < k; ++i) {
          const int a = i + j, b = i + j + k;
          if (b < N && a / (2 * p) == b / (2 * p)) {
            const u16x2 x = s[a], y = s[b];
            s[a] = __builtin_elementwise_max(x, y);
            s[b] = __builtin_elementwise_min(x, y);
          }
        }
      }
    }
  }
}

// The survivors of one group (half h of the packed keys) when more than n
// keys reach tau: every key above tau, then the ties in position order.
// Packed keys of entries 2j (sel 0x05040100) or 2j + 1 (sel 0x07060302)
// of A (low half) and B (high half), from the raw fp16 words.
__device__ __forceinline__ uint32_t nm_pk_key(uint32_t wa, uint32_t wb, uint32_t sel) {
  return __builtin_amdgcn_perm(wb, wa, sel) & 0x7fff7fffu;
}

template <int M>
__device__ __forceinline__ uint32_t nm_pk_ties(const uint32_t (&w)[M / 2], uint32_t tau,
                                               uint32_t ge, int n) {
  uint32_t gt = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) gt |= (((w[i / 2] >> (16 * (i & 1))) & 0x7fffu) > tau ? 1u : 0u) << i;
  uint32_t ties = ge & ~gt;
  for (int drop = __popc(ge) - n; drop > 0; --drop) ties &= ~(1u << (31 - __clz(ties)));
  return gt | ties;
}

// One block of 2 * kNmPkThreads groups: thread tid takes groups 2 tid and
// 2 tid + 1 of it, whose raw fp16 words are wa and wb.
template <int M>
__device__ __forceinline__ void nm_pk_block(const uint32_t (&wa)[M / 2], const uint32_t (&wb)[M / 2],
                                            int64_t blk, int64_t ngroups, int n,
                                            uint32_t* __restrict__ mask,
                                            uint16_t* __restrict__ val, int vec_out,
                                            uint16_t* outs) {
  constexpr int W = M / 2;
  constexpr int64_t kGroups = kNmPkThreads * 2;
  const int tid = (int)threadIdx.x;
  const int64_t ga = blk * kGroups + 2 * tid;
  const bool has_a = ga < ngroups, has_b = ga + 1 < ngroups;
  // packed keys: entry i of A (low half) and of B (high half)
  u16x2 sk[M];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    sk[2 * j] = pk_vec(nm_pk_key(wa[j], wb[j], 0x05040100u));
    sk[2 * j + 1] = pk_vec(nm_pk_key(wa[j], wb[j], 0x07060302u));
  }
  pk_sort_desc<M>(sk);
  const int r = n - 1;  // 0 <= r < M (checked on the host); uniform
  u16x2 tv = sk[0];
#pragma unroll
  for (int i = 1; i < M; ++i) tv = r == i ? sk[i] : tv;
  // Key i of A / B below its group's tau: sign bit 15 / 31 of the packed
  // difference.  Shifting it right by 15 - (i % 16) puts A's bit at
  // i % 16 and B's at 16 + i % 16; entries 16..31 gather in a second word.
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const uint32_t kp = nm_pk_key(wa[i / 2], wb[i / 2], (i & 1) ? 0x07060302u : 0x05040100u);
    const uint32_t dd = pk_bits(pk_vec(kp) - tv);  // keys rebuilt: fewer live registers
    const int j = i & 15;
    if (i < 16)
      lo |= (dd >> (15 - j)) & (0x10001u << j);
    else
      hi |= (dd >> (15 - j)) & (0x10001u << j);
  }
  const uint32_t lt_a = M == 16 ? lo & 0xffffu : (lo & 0xffffu) | (hi << 16);
  const uint32_t lt_b = M == 16 ? lo >> 16 : (lo >> 16) | (hi & 0xffff0000u);
  constexpr uint32_t kAll = M == 32 ? 0xffffffffu : 0xffffu;
  uint32_t keep_a = ~lt_a & kAll, keep_b = ~lt_b & kAll;
  const uint32_t tb = pk_bits(tv);
  if (__popc(keep_a) > n) keep_a = nm_pk_ties<M>(wa, tb & 0xffffu, keep_a, n);
  if (__popc(keep_b) > n) keep_b = nm_pk_ties<M>(wb, tb >> 16, keep_b, n);

  if (has_a) {
    // every entry is stored: a kept one at its slot, a dropped one at this
    // thread's spare slot, the last of its region (no branch per entry)
    // (slot - spare masked by 0 or -1, the entry's bit sign-extended)
    const int spare = tid * kNmPkRegion<M> + kNmPkRegion<M> - 1;
    int sa = tid * kNmPkRegion<M> - spare, sb = sa + n;  // next slot of A / B, from spare
    const uint32_t kb = has_b ? keep_b : 0u;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int m = (int)(keep_a << (31 - i)) >> 31;
      outs[spare + (sa & m)] = (uint16_t)(wa[i / 2] >> (16 * (i & 1)));
      sa -= m;
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int m = (int)(kb << (31 - i)) >> 31;
      outs[spare + (sb & m)] = (uint16_t)(wb[i / 2] >> (16 * (i & 1)));
      sb -= m;
    }
    if constexpr (M == 16) {
      mask[ga >> 1] = keep_a | (keep_b << 16);  // the pair's 32 entries
    } else {
      mask[ga] = keep_a;
      if (has_b) mask[ga + 1] = keep_b;
    }
  }
  __syncthreads();
  const int64_t first = blk * kGroups;  // the block's first group
  const int64_t ng = (ngroups - first) < kGroups ? (ngroups - first) : kGroups;
  const int count = (int)ng * n;
  const int per = 2 * n;  // outputs of one thread's region
  uint16_t* dst = val + first * n;
  if (vec_out && (count % 8) == 0 && (per % 8) == 0) {
    // 8 outputs never straddle two regions; a region starts on a dword
    for (int i = tid; i < count / 8; i += kNmPkThreads) {
      const int e = 8 * i;
      const int r = e / per;
      const uint32_t* src =
          reinterpret_cast<const uint32_t*>(outs + r * kNmPkRegion<M> + (e - r * per));
      const u32x4 v = {src[0], src[1], src[2], src[3]};
      *reinterpret_cast<u32x4*>(dst + e) = v;
    }
  } else {
    for (int i = tid; i < count; i += kNmPkThreads) {
      const int r = i / per;
      dst[i] = outs[r * kNmPkRegion<M> + (i - r * per)];
    }
  }
  __syncthreads();  // outs is rewritten by the next block
}

template <int M>
__global__ __launch_bounds__(kNmPkThreads) void k_sparsify_nm_pk(const uint16_t* __restrict__ x,
                                                               int64_t ngroups, int n,
                                                               uint32_t* __restrict__ mask,
                                                               uint16_t* __restrict__ val,
                                                               int vec_out) {
  static_assert(M == 16 || M == 32, "two whole groups per thread");
  constexpr int W = M / 2;                       // 32-bit words of one group
  constexpr int64_t kGroups = kNmPkThreads * 2;  // groups of one block
  __shared__ __align__(16) uint16_t outs[kNmPkThreads * kNmPkRegion<M>];
  const int tid = (int)threadIdx.x;
  const int64_t nblk = (ngroups + kGroups - 1) / kGroups;
  // A workgroup walks blocks blockIdx.x, + gridDim.x, ...; the next block's
  // loads are issued before the current one is worked on, so HBM stays busy
  // while the sorts run.  Two register sets take turns (no copies).
  // Groups past the end read the last group instead (their results are
  // not stored): every load is unconditional.
  auto load = [&](int64_t blk, uint32_t (&ra_)[W], uint32_t (&rb_)[W]) {
    const int64_t ga = blk * kGroups + 2 * tid;
    const u32x4* sa = reinterpret_cast<const u32x4*>(x + (ga < ngroups ? ga : ngroups - 1) * M);
    const u32x4* sb =
        reinterpret_cast<const u32x4*>(x + (ga + 1 < ngroups ? ga + 1 : ngroups - 1) * M);
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const u32x4 ra = sa[q];
      const u32x4 rb = sb[q];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ra_[4 * q + c] = ra[c];
        rb_[4 * q + c] = rb[c];
      }
    }
  };
  const int64_t step = gridDim.x;
  uint32_t a0[W], b0[W], a1[W], b1[W];
  int64_t blk = blockIdx.x;
  if (blk < nblk) load(blk, a0, b0);
  while (blk < nblk) {
    if (blk + step < nblk) load(blk + step, a1, b1);
    nm_pk_block<M>(a0, b0, blk, ngroups, n, mask, val, vec_out, outs);
    blk += step;
    if (blk >= nblk) break;
    if (blk + step < nblk) load(blk + step, a0, b0);
    nm_pk_block<M>(a1, b1, blk, ngroups, n, mask, val, vec_out, outs);
    blk += step;
  }
}

// n = m / 2 for m = 16, 32 with one group per thread: entry i of the group
// (low half) and entry m/2 + i (high half) share packed key register i, so
// one packed sort of m/2 registers sorts both halves of the group at once,
// and the half-cleaner pairs half a's i-th largest with half b's
// (m/2 - 1 - i)-th: tau, the (m/2)-th largest key, is min over i of
// max(a_i, b_(m/2-1-i)).  A thread holds one group's m raw values and m/2
// keys instead of k_sparsify_nm_pk's two groups, so more waves share a SIMD
// and cover each other's loads (16:32 at 2048 x 4096: 8.03 -> 6.86 us).
constexpr int kNmHalfThreads = 256;
constexpr int kNmHalfBlocksPerCu = 8;  // workgroups of the grid per compute unit
// LDS region of one thread's m/2 survivors plus its spare slot, fp16 units:
// m/4 + 1 dwords, odd, so the lanes' regions start on distinct banks
template <int M>
constexpr int kNmHalfRegion = M / 2 + 2;

template <int M>
__global__ __launch_bounds__(kNmHalfThreads) void k_sparsify_nm_half(
    const uint16_t* __restrict__ x, int64_t ngroups, uint32_t* __restrict__ mask,
    uint16_t* __restrict__ val, int vec_out) {
  static_assert(M == 16 || M == 32, "packed halves of one group");
  constexpr int N = M / 2;   // survivors per group; also packed key registers
  constexpr int W = M / 2;   // 32-bit words of raw values
  constexpr int RG = kNmHalfRegion<M>;
  __shared__ __align__(16) uint16_t outs[kNmHalfThreads * RG];
  const int tid = (int)threadIdx.x;
  const int64_t nblk = (ngroups + kNmHalfThreads - 1) / kNmHalfThreads;
  // Groups past the end read the last group instead (their results are not
  // stored): every load is unconditional.
  auto load = [&](int64_t blk, uint32_t (&w)[W]) {
    int64_t g = blk * kNmHalfThreads + tid;
    if (g >= ngroups) g = ngroups - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + g * M);
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const u32x4 r = src[q];
#pragma unroll
      for (int c = 0; c < 4; ++c) w[4 * q + c] = r[c];
    }
  };
  // packed key of entries i (low) and N + i (high)
  auto key2 = [&](const uint32_t (&w)[W], int i) {
    return nm_pk_key(w[i / 2], w[N / 2 + i / 2], (i & 1) ? 0x07060302u : 0x05040100u);
  };
  auto block = [&](const uint32_t (&w)[W], int64_t blk) {
    const int64_t g = blk * kNmHalfThreads + tid;
    u16x2 sk[N];
#pragma unroll
    for (int i = 0; i < N; ++i) sk[i] = pk_vec(key2(w, i));
    pk_sort_desc<N>(sk);
    // r_i = max(a_i, b_(N-1-i)) in the low half, max(b_i, a_(N-1-i)) -- the
    // low half of r_(N-1-i) -- in the high half: r_0 .. r_(N/2-1) hold all N
    auto swapped = [](u16x2 v) {
      return pk_vec(__builtin_amdgcn_alignbit(pk_bits(v), pk_bits(v), 16));
    };
    u16x2 t = __builtin_elementwise_max(sk[0], swapped(sk[N - 1]));
#pragma unroll
    for (int i = 1; i < N / 2; ++i)
      t = __builtin_elementwise_min(t, __builtin_elementwise_max(sk[i], swapped(sk[N - 1 - i])));
    const uint32_t tb = pk_bits(t);
    const uint32_t tau = (tb & 0xffffu) < (tb >> 16) ? (tb & 0xffffu) : (tb >> 16);
    const u16x2 tv = pk_vec(tau | (tau << 16));
    // entry i below tau: sign bit 15 of the packed difference, entry N + i:
    // bit 31; shifted right by 15 - i they land on bits i and 16 + i
    uint32_t lt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t dd = pk_bits(pk_vec(key2(w, i)) - tv);
      lt |= (dd >> (15 - i)) & (0x10001u << i);
    }
    if constexpr (M == 16) lt = (lt & 0xffu) | ((lt >> 8) & 0xff00u);
    constexpr uint32_t kAll = M == 32 ? 0xffffffffu : 0xffffu;
    uint32_t keep = ~lt & kAll;
    if (__popc(keep) > N) {
      // ties at tau: every key above it, then the first ties in position order
      uint32_t gt = 0;
#pragma unroll
      for (int i = 0; i < M; ++i)
        gt |= (((w[i / 2] >> (16 * (i & 1))) & 0x7fffu) > tau ? 1u : 0u) << i;
      uint32_t ties = keep & ~gt;
      for (int drop = __popc(keep) - N; drop > 0; --drop) ties &= ~(1u << (31 - __clz(ties)));
      keep = gt | ties;
    }
    if (g < ngroups) {
      // every entry is stored: a kept one at its slot, a dropped one at the
      // spare slot ending the region (slot - spare masked by 0 or -1)
      const int spare = tid * RG + RG - 1;
      int sl = tid * RG - spare;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int m = (int)(keep << (31 - i)) >> 31;
        outs[spare + (sl & m)] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
        sl -= m;
      }
      if constexpr (M == 32)
        mask[g] = keep;
      else  // two groups per mask word, group g in half g % 2
        reinterpret_cast<uint16_t*>(mask)[g] = (uint16_t)keep;
    }
    __syncthreads();
    const int64_t first = blk * kNmHalfThreads;
    const int64_t ng = (ngroups - first) < kNmHalfThreads ? (ngroups - first) : kNmHalfThreads;
    const int count = (int)ng * N;
    uint16_t* dst = val + first * N;
    if (vec_out) {
      // 8 values of one region per item; a region starts on a dword
      for (int i = tid; i < count / 8; i += kNmHalfThreads) {
        const int r = i / (N / 8);
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(outs + r * RG + 8 * (i % (N / 8)));
        const u32x4 v = {src[0], src[1], src[2], src[3]};
        *reinterpret_cast<u32x4*>(dst + 8 * i) = v;
      }
    } else {
      for (int i = tid; i < count; i += kNmHalfThreads) dst[i] = outs[(i / N) * RG + (i % N)];
    }
    __syncthreads();  // outs is rewritten by the next block
  };
  const int64_t step = gridDim.x;
  if constexpr (M == 32) {
    // one register set: the grid holds every block at once where registers
    // allow (four waves per SIMD), and a second set would cost occupancy
    uint32_t w0[W];
    for (int64_t blk = blockIdx.x; blk < nblk; blk += step) {
      load(blk, w0);
      block(w0, blk);
    }
  } else {
    uint32_t w0[W], w1[W];
    int64_t blk = blockIdx.x;
    if (blk < nblk) load(blk, w0);
    while (blk < nblk) {
      if (blk + step < nblk) load(blk + step, w1);
      block(w0, blk);
      blk += step;
      if (blk >= nblk) break;
      if (blk + step < nblk) load(blk + step, w0);
      block(w1, blk);
      blk += step;
    }
  }
}

}  // namespace

hipError_t launch_sparsify_threshold(const uint16_t* x, int64_t rows, int64_t d, float t,
                                     uint32_t* mask, int32_t* idx, uint16_t* val,
                                     int32_t* nnz, int64_t cap, hipStream_t s) {
  const int vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && (d % 8) == 0) ? 1 : 0;
  // Rows of up to 4096 entries on 512 threads of 8: with 1024 threads of 16
  // most threads held nothing (d = 4096: 3.85 -> 3.03 us; d = 1024: 3.72 ->
  // 2.74 us).  Longer rows keep 1024 threads of 16 (256 of 16: no faster).
  if (d <= (int64_t)kCutThreads * kCutE) {
    hipLaunchKernelGGL((k_sparsify_threshold<kCutThreads, kCutE>), dim3((unsigned)rows),
                       dim3(kCutThreads), 0, s, x, d, t, mask, idx, val, nnz, cap, vec);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_sparsify_threshold<kSparsifyThreads, 16>), dim3((unsigned)rows),
                     dim3(kSparsifyThreads), 0, s, x, d, t, mask, idx, val, nnz, cap, vec);
  return hipGetLastError();
}

hipError_t launch_sparsify_scored(const uint16_t* x, int64_t rows, int64_t d,
                                  const uint16_t* mu, const double* colnorm, int n, int m,
                                  double t, uint32_t* mask, int32_t* idx, uint16_t* val,
                                  int32_t* nnz, float* alpha, int64_t cap, hipStream_t s) {
  const int vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && (d % 8) == 0) ? 1 : 0;
  const int vec_mu = ((reinterpret_cast<uintptr_t>(mu) & 15u) == 0) ? 1 : 0;
  const dim3 grid((unsigned)rows);
  if (m == 0) {
    if (d >= kScoredThrMinD && d <= kScoredThrMaxD && rows <= 0x7fffffffLL) {
      // two passes: decisions over chunks, then the list
      const int64_t nc = (d + kScoredThrChunk - 1) / kScoredThrChunk;
      hipLaunchKernelGGL(k_scored_thr_bits, dim3((unsigned)rows, (unsigned)nc), dim3(256), 0, s,
                         x, d, mu, colnorm, t, mask, idx, val, cap);
      hipLaunchKernelGGL((k_sparsify_scored<kSparsifyThreads, 16, true>), grid,
                         dim3(kSparsifyThreads), 0, s, x, d, mu, colnorm, t, mask, idx, val, nnz,
                         alpha, cap, vec, vec_mu);
      return hipGetLastError();
    }
    // short rows: one workgroup per row
    hipLaunchKernelGGL((k_sparsify_scored<kSparsifyThreads, 16>), grid, dim3(kSparsifyThreads), 0,
                       s, x, d, mu, colnorm, t, mask, idx, val, nnz, alpha, cap, vec, vec_mu);
    return hipGetLastError();
  }
  // N:M: one thread per group over many workgroups, then the row sums of
  // the variance correction
  const int64_t ng = d / m;
  const int64_t gy = (ng + kScoredNmGroups - 1) / kScoredNmGroups;
  if (gy > 65535 || rows > 0x7fffffffLL) return hipErrorNotSupported;  // d <= 4194240 m
  const dim3 g2((unsigned)rows, (unsigned)gy);
#define SA_SCORED_NM(M)                                                                       \
  hipLaunchKernelGGL((k_sparsify_scored_nm<M>), g2, dim3(kScoredNmGroups), 0, s, x, d, mu,   \
                     colnorm, n, mask, idx, val, nnz, cap, vec, vec_mu)
  switch (m) {
    case 4: SA_SCORED_NM(4); break;
    case 8: SA_SCORED_NM(8); break;
    case 16: SA_SCORED_NM(16); break;
    case 32: SA_SCORED_NM(32); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_SCORED_NM
  if (alpha != nullptr)
    hipLaunchKernelGGL(k_scored_alpha, grid, dim3(1024), 0, s, x, d, mu, val, cap, ng * n, alpha,
                       vec, vec_mu,
                       ((reinterpret_cast<uintptr_t>(val) & 15u) == 0 && cap % 8 == 0) ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_sparsify_topk(const uint16_t* x, int64_t rows, int64_t d, int64_t k,
                                uint32_t* mask, int32_t* idx, uint16_t* val, int32_t* nnz,
                                int64_t cap, int32_t* cut, hipStream_t s) {
  const int vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && (d % 8) == 0) ? 1 : 0;
  if (d <= (int64_t)kCutThreads * kCutE) {
    if (mask == nullptr && idx == nullptr)
      hipLaunchKernelGGL((k_topk_cut<kCutThreads, kCutE>), dim3((unsigned)rows),
                         dim3(kCutThreads), 0, s, x, d, k, cut, nnz);
    else
      hipLaunchKernelGGL((k_topk_radix<kCutThreads, kCutE>), dim3((unsigned)rows), dim3(kCutThreads), 0, s, x, d, k, cut,
                         mask, idx, val, nnz, cap);
    return hipGetLastError();
  }
  if (d <= (int64_t)kSparsifyThreads * 16) {
    hipLaunchKernelGGL((k_topk<kSparsifyThreads, 16>), dim3((unsigned)rows),
                       dim3(kSparsifyThreads), 0, s, x, d, k, cut, mask, idx, val, nnz, cap, vec);
  } else {
    hipLaunchKernelGGL((k_topk<kSparsifyThreads, 64>), dim3((unsigned)rows),
                       dim3(kSparsifyThreads), 0, s, x, d, k, cut, mask, idx, val, nnz, cap, vec);
  }
  return hipGetLastError();
}

// ---- tile-shared N:M --------------------------------------------------------
// One N:M pattern for each tile of tt consecutive rows.  A workgroup takes
// one tile and 64 columns: thread (r, c) of its 4 x 64 covers column c in
// rows r, r + 4, r + 8, ... of the tile.  A column's score is the sum of the
// tile's |x| in fp64, which is exact (every fp16 magnitude is an integer
// multiple of 2^-24 below 2^16; at most 256 of them sum below 2^24), so
// neither the split over threads nor the order of the additions can change
// a decision.  The first wave ranks each column within its group of M (kept
// iff fewer than n of the group rank before it: a larger score, or an equal
// one at a lower position) and a ballot gives the two mask words; then every
// thread writes its rows' values at their compressed positions (the group's
// first slot plus the kept bits before).
constexpr int kSharedThreads = 256;
constexpr int kSharedCols = 64;
constexpr int kSharedSlices = kSharedThreads / kSharedCols;

__device__ __forceinline__ double mag_f64(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, (uint16_t)(b & 0x7fffu));
}

template <int M>
__global__ __launch_bounds__(kSharedThreads) void k_sparsify_nm_shared(
    const uint16_t* __restrict__ x, int64_t rows, int64_t d, int n, int tt,
    uint32_t* __restrict__ mask, uint16_t* __restrict__ val) {
  __shared__ double part[kSharedSlices][kSharedCols];
  __shared__ uint32_t words[2];
  const int tid = (int)threadIdx.x;
  const int r = tid / kSharedCols, c = tid % kSharedCols;
  const int64_t t0 = (int64_t)blockIdx.x * tt;
  const int64_t t1 = t0 + tt < rows ? t0 + tt : rows;
  const int64_t k = (int64_t)blockIdx.y * kSharedCols + c;
  const bool active = k < d;  // d % 32 == 0: whole mask words
  constexpr int R = kSharedSlices;
  double sc = 0.0;
  if (active) {
    const uint16_t* xp = x + (t0 + r) * d + k;
    int64_t t = t0 + r;
    for (; t + 3 * R < t1; t += 4 * R, xp += 4 * R * d) {
      uint16_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = xp[u * R * d];
#pragma unroll
      for (int u = 0; u < 4; ++u) sc += mag_f64(v[u]);
    }
    for (; t < t1; t += R, xp += R * d) sc += mag_f64(*xp);
  }
  part[r][c] = sc;
  __syncthreads();
  if (r == 0) {
    double own = 0.0;
#pragma unroll
    for (int q = 0; q < R; ++q) own += part[q][c];
    part[0][c] = own;  // each lane reads and writes only its own column
  }
  __syncthreads();
  if (r == 0) {
    const double own = part[0][c];
    const int g0 = c - c % M;
    int rank = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const double o = part[0][g0 + q];
      rank += (o > own || (o == own && g0 + q < c)) ? 1 : 0;
    }
    const uint64_t ball = __ballot(active && rank < n);
    if (c == 0) {
      words[0] = (uint32_t)ball;
      words[1] = (uint32_t)(ball >> 32);
    }
  }
  __syncthreads();
  if (!active) return;
  const uint32_t word = words[c / 32];
  const int b = c % 32;
  if (r == 0 && b == 0) mask[(int64_t)blockIdx.x * (d / 32) + k / 32] = word;
  if (((word >> b) & 1u) == 0u) return;
  const int gb = b - b % M;
  const int64_t slot = (k / M) * n + __builtin_popcount((word >> gb) & ((1u << (b - gb)) - 1u));
  const int64_t vpr = d / M * n;
  const uint16_t* xp = x + (t0 + r) * d + k;
  uint16_t* vp = val + (t0 + r) * vpr + slot;
  int64_t t = t0 + r;
  for (; t + 3 * R < t1; t += 4 * R, xp += 4 * R * d, vp += 4 * R * vpr) {
    uint16_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = xp[u * R * d];
#pragma unroll
    for (int u = 0; u < 4; ++u) vp[u * R * vpr] = v[u];
  }
  for (; t < t1; t += R, xp += R * d, vp += R * vpr) *vp = *xp;
}

hipError_t launch_sparsify_nm_shared(const uint16_t* x, int64_t rows, int64_t d, int n, int m,
                                     int tt, uint32_t* mask, uint16_t* val, hipStream_t s) {
  const int64_t tiles = (rows + tt - 1) / tt;
  const int64_t chunks = (d + kSharedCols - 1) / kSharedCols;
  if (tiles > 0x7fffffffLL || chunks > 65535) return hipErrorNotSupported;
  const dim3 grid((unsigned)tiles, (unsigned)chunks), block(kSharedThreads);
#define SA_SHARED(MM) \
  hipLaunchKernelGGL(k_sparsify_nm_shared<MM>, grid, block, 0, s, x, rows, d, n, tt, mask, val)
  switch (m) {
    case 4: SA_SHARED(4); break;
    case 8: SA_SHARED(8); break;
    case 16: SA_SHARED(16); break;
    case 32: SA_SHARED(32); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_SHARED
  return hipGetLastError();
}

hipError_t launch_sparsify_nm(const uint16_t* x, int64_t rows, int64_t d, int n, int m,
                              uint32_t* mask, uint16_t* val, hipStream_t s) {
  // whole runs are 16-byte aligned when the output base is (each
  // workgroup's run is a multiple of 8 values at every supported n / m)
  const int vec = (reinterpret_cast<uintptr_t>(val) & 15u) == 0 ? 1 : 0;
  if (m == 16 || m == 32) {
    const int64_t ng = rows * d / m;
    if (2 * n == m) {  // one group per thread, both halves in packed registers
      const int64_t nb = (ng + kNmHalfThreads - 1) / kNmHalfThreads;
      const int64_t cap2 = (int64_t)device_cus() * kNmHalfBlocksPerCu;
      const dim3 g2((unsigned)(nb < cap2 ? nb : cap2));
      if (m == 32)
        hipLaunchKernelGGL(k_sparsify_nm_half<32>, g2, dim3(kNmHalfThreads), 0, s, x, ng, mask,
                           val, vec);
      else
        hipLaunchKernelGGL(k_sparsify_nm_half<16>, g2, dim3(kNmHalfThreads), 0, s, x, ng, mask,
                           val, vec);
      return hipGetLastError();
    }
    // other n: two groups per thread and the full sort
    const int64_t nblk = (ng + 2 * kNmPkThreads - 1) / (2 * kNmPkThreads);
    const int64_t cap = (int64_t)device_cus() * kNmPkBlocksPerCu;
    const dim3 grid((unsigned)(nblk < cap ? nblk : cap));
    if (m == 16)
      hipLaunchKernelGGL(k_sparsify_nm_pk<16>, grid, dim3(kNmPkThreads), 0, s, x, ng, n, mask,
                         val, vec);
    else
      hipLaunchKernelGGL(k_sparsify_nm_pk<32>, grid, dim3(kNmPkThreads), 0, s, x, ng, n, mask,
                         val, vec);
    return hipGetLastError();
  }
  const int64_t n8 = rows * d / 8;
  const dim3 grid((unsigned)((n8 + kNmThreads - 1) / kNmThreads));
  switch (m) {
    case 4:
      hipLaunchKernelGGL(k_sparsify_nm<4>, grid, dim3(kNmThreads), 0, s, x, n8, n, mask, val, vec);
      break;
    case 8:
      hipLaunchKernelGGL(k_sparsify_nm<8>, grid, dim3(kNmThreads), 0, s, x, n8, n, mask, val, vec);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sa
