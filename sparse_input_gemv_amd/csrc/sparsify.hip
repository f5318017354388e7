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

// Loads E consecutive fp16 bit patterns starting at element k0 of a row.
// The vector path needs a 16-byte aligned row and k0 a multiple of 8.
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

// keep_i = (|x_i| >= t) && (x_i != 0), compared in fp32 (fp16 widening is
// exact, so this is the exact comparison).  One workgroup per row.
template <int NT, int E>
__global__ __launch_bounds__(NT) void k_sparsify_threshold(
    const uint16_t* __restrict__ x, int64_t d, float t, uint32_t* __restrict__ mask,
    int32_t* __restrict__ idx, uint16_t* __restrict__ val, int32_t* __restrict__ nnz,
    int64_t cap, int vec) {
  __shared__ int scan[NT / kWave];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  int32_t* ir = idx + row * cap;
  uint16_t* vr = val + row * cap;
  uint32_t* mr = mask ? mask + row * ((d + 31) >> 5) : nullptr;
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

// Weight-aware selection with a static shift (the flexible N:M
// activation-sparsity summary, section 2: WT and Amber-Pruner score entries
// by the weight they multiply; S-PTS shifts activations towards zero; VAR
// restores the output scale).  Per row, per entry:
//   x' = fp16(fp32(x) - fp32(mu))   (mu null: x' = x)
//   score = |x'| * c in fp64         (c null: |x'|; the fp64 product is
//                                     correctly rounded, one operation)
//   M == 0: keep iff score >= t and x' != 0
//   M  > 0: keep the n largest scores of every M consecutive entries, ties to
//           the lower index (n rounds of taking each group's largest score
//           not yet taken; groups lie inside one thread's run, E % M == 0)
// The kept x' are compacted as the threshold sparsifier does.  alpha[row] =
// sqrt(sum x'^2 / sum_kept x'^2) (1 when nothing is kept), in fp64.
template <int NT, int E, int M>
__global__ __launch_bounds__(NT) void k_sparsify_scored(
    const uint16_t* __restrict__ x, int64_t d, const uint16_t* __restrict__ mu,
    const double* __restrict__ cn, double t, int n, uint32_t* __restrict__ mask,
    int32_t* __restrict__ idx, uint16_t* __restrict__ val, int32_t* __restrict__ nnz,
    float* __restrict__ alpha, int64_t cap, int vec, int vec_mu) {
  static_assert(M == 0 || E % M == 0, "groups inside one run");
  __shared__ int scan[NT / kWave];
  __shared__ double sums[2][NT / kWave];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  int32_t* ir = idx + row * cap;
  uint16_t* vr = val + row * cap;
  uint32_t* mr = mask ? mask + row * ((d + 31) >> 5) : nullptr;
  int base = 0;
  double s_all = 0.0, s_kept = 0.0;
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
    double sc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double a = fabs((double)h2f(v[e]));
      sc[e] = (k0 + e < d) ? (cn != nullptr ? a * cn[k0 + e] : a) : 0.0;
    }
    uint64_t bits = 0;
    if constexpr (M == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool keep = (k0 + e < d) && sc[e] >= t && h2f(v[e]) != 0.f;
        bits |= (uint64_t)keep << e;
      }
    } else {
      // n rounds; each takes, in every group, the largest score not yet
      // taken (strict >, scanning upwards: ties go to the lower index)
      for (int it = 0; it < n; ++it) {
#pragma unroll
        for (int g = 0; g < E / M; ++g) {
          int best = g * M;
          double bs = -1.0;  // scores are >= 0
#pragma unroll
          for (int j = 0; j < M; ++j) {
            const int e = g * M + j;
            const bool take = ((bits >> e) & 1ull) == 0 && sc[e] > bs;
            bs = take ? sc[e] : bs;
            best = take ? e : best;
          }
          bits |= 1ull << best;
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (k0 + e >= d) bits &= ~(1ull << e);  // groups past the row end
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double q = (double)h2f(v[e]) * (double)h2f(v[e]);
      s_all += (k0 + e < d) ? q : 0.0;
      s_kept += ((bits >> e) & 1ull) ? q : 0.0;
    }
    compact_run<NT, E>(bits, v, k0, d, base, scan, ir, vr, mr);
  }
  if (alpha != nullptr) {
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

// Exactly k survivors per row: the k largest magnitudes, ties to the lower
// index (fp16 magnitudes compared exactly as 15-bit keys; -0 == +0).  One LDS
// bin per key value (2^15 bins, 128 KB): a single pass of LDS atomics counts
// every key; each thread then owns 32 consecutive keys' bins, and a workgroup
// scan of the threads' sums, read from the top, finds the thread and then the
// bin where the count of larger keys reaches k.  The bins of one thread are
// stored as 8 int4 a workgroup-width apart (bin address below), so that the
// threads of a wave read 64 consecutive int4 at a time, free of LDS bank
// conflicts; stored contiguously, the 128-byte stride between threads put
// every lane of a wave on the same four banks.  That bin is tau, the k-th
// largest key, with r = k - #(keys > tau) of its entries still to keep; a
// scan of the threads' counts of keys equal to tau, in index order, finds
// the r-th of them, at index i*.  Entry i survives iff key_i > tau, or
// key_i == tau and i <= i* (k = 0: tau = 2^15, i* = -1, nothing survives).
// Outputs: the pair (tau, i*) per row in `cut` (may be NULL), the bitmask,
// and the compacted list (staged in LDS for d <= NT * 16, so it leaves in
// coalesced stores).  One workgroup per row; each thread keeps E keys.
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
  static_assert(BPT % 4 == 0 && kTopkBins % NT == 0 && BPT <= 32, "bins split into int4 runs");
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
      int sc = row16_inclusive_scan(cb);
      if constexpr (BPT > 16) sc += (lane >> 4) == 1 ? __builtin_amdgcn_readlane(sc, 15) : 0;
      const uint64_t hit = __ballot(lane < BPT && ab + sc >= kk);
      const int l = __builtin_ctzll(hit);
      if (lane == l) {
        sel[0] = ts * BPT + jb;
        sel[1] = kk - (ab + sc - cb);
      }
    }
    __syncthreads();
    tau = sel[0];
    const int r = sel[1];  // >= 1
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

// N:M: each thread owns 8 consecutive entries (one 16-byte load).  An entry
// is kept iff fewer than n entries of its group rank before it, where j
// ranks before i iff |x_j| > |x_i|, or they are equal and j < i.  For
// M <= 8 the groups are local and ranked pairwise.  For M = 16 / 32 the M/8
// threads of a group find the n-th largest 15-bit magnitude key tau by a
// bitwise binary search (15 steps, each a count of keys >= a candidate,
// summed over the group with cross-lane shuffles), keep every key > tau and
// the first n - #(> tau) keys equal to tau in index order.  The flattened
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
constexpr int kQuadXor3 = 3 | (2 << 2) | (1 << 4) | (0 << 6);

// Selection helpers on a lane's 8 keys (descending order = index order).
// Batcher's odd-even merge sort network for 8 (19 comparators).
__device__ __forceinline__ void nm_cx(int (&k)[8], int i, int j) {
  const int a = k[i], b = k[j];
  k[i] = a > b ? a : b;
  k[j] = a > b ? b : a;
}
__device__ __forceinline__ void nm_sort8(int (&k)[8]) {
  nm_cx(k, 0, 1); nm_cx(k, 2, 3); nm_cx(k, 4, 5); nm_cx(k, 6, 7);
  nm_cx(k, 0, 2); nm_cx(k, 1, 3); nm_cx(k, 4, 6); nm_cx(k, 5, 7);
  nm_cx(k, 1, 2); nm_cx(k, 5, 6);
  nm_cx(k, 0, 4); nm_cx(k, 1, 5); nm_cx(k, 2, 6); nm_cx(k, 3, 7);
  nm_cx(k, 2, 4); nm_cx(k, 3, 5);
  nm_cx(k, 1, 2); nm_cx(k, 3, 4); nm_cx(k, 5, 6);
}
// A bitonic sequence of 8 into descending order (distances 4, 2, 1).
__device__ __forceinline__ void nm_half_clean(int (&k)[8]) {
  nm_cx(k, 0, 4); nm_cx(k, 1, 5); nm_cx(k, 2, 6); nm_cx(k, 3, 7);
  nm_cx(k, 0, 2); nm_cx(k, 1, 3); nm_cx(k, 4, 6); nm_cx(k, 5, 7);
  nm_cx(k, 0, 1); nm_cx(k, 2, 3); nm_cx(k, 4, 5); nm_cx(k, 6, 7);
}
// Compare slot i with slot 7 - i (REV) or slot i of the lane CTRL names;
// the lane holding the earlier part of the sequence keeps the larger key.
template <int CTRL, bool REV>
__device__ __forceinline__ void nm_exchange(int (&k)[8], bool keep_max) {
  int p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = quad_perm<CTRL>(k[REV ? 7 - i : i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int hi = k[i] > p[i] ? k[i] : p[i];
    const int lo = k[i] > p[i] ? p[i] : k[i];
    k[i] = keep_max ? hi : lo;
  }
}

// lane q of each aligned group of G (G = 2 or 4) lanes, to every lane of it
template <int G, int Q>
constexpr int quad_bcast() {
  return G == 4 ? Q * 0x55 : (Q | (Q << 2) | ((2 + Q) << 4) | ((2 + Q) << 6));
}

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

  uint32_t keep = 0;
  if constexpr (M <= 8) {
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
  } else {
    constexpr int G = M / 8;  // threads per group, aligned lane runs
    const int gl = lane & (G - 1);
    static_assert(G == 2 || G == 4, "groups within a lane quad");
    auto group_sum = [&](int c) {
      c += quad_perm<kQuadXor1>(c);
      if constexpr (G == 4) c += quad_perm<kQuadXor2>(c);
      return c;
    };
    // exclusive prefix over the group's lanes of a per-lane count
    auto group_prefix = [&](int x) {
      int e = 0;
      const int x0 = quad_perm<quad_bcast<G, 0>()>(x);
      e += gl > 0 ? x0 : 0;
      if constexpr (G == 4) {
        const int x1 = quad_perm<quad_bcast<G, 1>()>(x);
        const int x2 = quad_perm<quad_bcast<G, 2>()>(x);
        e += gl > 1 ? x1 : 0;
        e += gl > 2 ? x2 : 0;
      }
      return e;
    };
    // tau = the group's n-th largest key.  Each lane sorts its 8 keys, the
    // group's lanes merge them with bitonic steps across lanes (DPP), so the
    // group's M keys lie in descending order along (lane, slot); tau is
    // entry n - 1: slot (n-1) % 8 of lane (n-1) / 8 (n is uniform).  A
    // bisection over the 15 key bits gives the same tau with a dependency
    // chain ~5x longer (measured at 2048 x 4096: 13.1 against 9.1 us at
    // 8:16, 14.0 against 11.5 us at 16:32).
    int sk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sk[i] = key[i];
    nm_sort8(sk);
    nm_exchange<kQuadXor1, true>(sk, (gl & 1) == 0);
    nm_half_clean(sk);
    if constexpr (G == 4) {
      nm_exchange<kQuadXor3, true>(sk, gl < 2);
      nm_exchange<kQuadXor1, false>(sk, (gl & 1) == 0);
      nm_half_clean(sk);
    }
    const int r = n - 1;  // 0 <= r < M (checked on the host)
    int pick = sk[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) pick = (r & 7) == i ? sk[i] : pick;
    int tau;
    if constexpr (G == 2) {
      const int b0 = quad_perm<quad_bcast<2, 0>()>(pick);
      const int b1 = quad_perm<quad_bcast<2, 1>()>(pick);
      tau = (r >> 3) == 0 ? b0 : b1;
    } else {
      const int b0 = quad_perm<quad_bcast<4, 0>()>(pick);
      const int b1 = quad_perm<quad_bcast<4, 1>()>(pick);
      const int b2 = quad_perm<quad_bcast<4, 2>()>(pick);
      const int b3 = quad_perm<quad_bcast<4, 3>()>(pick);
      const int q = r >> 3;
      tau = q == 0 ? b0 : (q == 1 ? b1 : (q == 2 ? b2 : b3));
    }
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gt += key[i] > tau ? 1 : 0;
      eq += key[i] == tau ? 1 : 0;
    }
    const int need = n - group_sum(gt);  // ties at tau still to keep
    int e = group_prefix(eq);             // ties at tau in lower lanes of the group
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (key[i] > tau) {
        keep |= 1u << i;
      } else if (key[i] == tau) {
        if (e < need) keep |= 1u << i;
        ++e;
      }
    }
    // kept entries in lower lanes of the group come first
    const int pre = group_prefix(__popc(keep));
    if (active) {
      int slot = (tid / G) * n + pre;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((keep >> i) & 1u) outs[slot++] = v[i];
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

}  // namespace

hipError_t launch_sparsify_threshold(const uint16_t* x, int64_t rows, int64_t d, float t,
                                     uint32_t* mask, int32_t* idx, uint16_t* val,
                                     int32_t* nnz, int64_t cap, hipStream_t s) {
  const int vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && (d % 8) == 0) ? 1 : 0;
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
  // Groups of 32 need runs of 32 fp64 scores per thread: 256-thread
  // workgroups (one wave per SIMD, up to 512 registers) hold them without
  // spilling; the other kinds fit the 128 registers of 1024 threads.
#define SA_SCORED(NT, E, M)                                                                  \
  hipLaunchKernelGGL((k_sparsify_scored<NT, E, M>), grid, dim3(NT), 0, s, x, d, mu, colnorm, t, \
                     n, mask, idx, val, nnz, alpha, cap, vec, vec_mu)
  switch (m) {
    case 0: SA_SCORED(kSparsifyThreads, 16, 0); break;
    case 4: SA_SCORED(kSparsifyThreads, 16, 4); break;
    case 8: SA_SCORED(kSparsifyThreads, 16, 8); break;
    case 16: SA_SCORED(kSparsifyThreads, 16, 16); break;
    case 32: SA_SCORED(256, 32, 32); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_SCORED
  return hipGetLastError();
}

hipError_t launch_sparsify_topk(const uint16_t* x, int64_t rows, int64_t d, int64_t k,
                                uint32_t* mask, int32_t* idx, uint16_t* val, int32_t* nnz,
                                int64_t cap, int32_t* cut, hipStream_t s) {
  const int vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && (d % 8) == 0) ? 1 : 0;
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
  const int64_t n8 = rows * d / 8;
  const dim3 grid((unsigned)((n8 + kNmThreads - 1) / kNmThreads));
  // whole runs are 16-byte aligned when the output base is (2048*n/M halves
  // per workgroup is a multiple of 64)
  const int vec = (reinterpret_cast<uintptr_t>(val) & 15u) == 0 ? 1 : 0;
  switch (m) {
    case 4:
      hipLaunchKernelGGL(k_sparsify_nm<4>, grid, dim3(kNmThreads), 0, s, x, n8, n, mask, val, vec);
      break;
    case 8:
      hipLaunchKernelGGL(k_sparsify_nm<8>, grid, dim3(kNmThreads), 0, s, x, n8, n, mask, val, vec);
      break;
    case 16:
      hipLaunchKernelGGL(k_sparsify_nm<16>, grid, dim3(kNmThreads), 0, s, x, n8, n, mask, val,
                         vec);
      break;
    case 32:
      hipLaunchKernelGGL(k_sparsify_nm<32>, grid, dim3(kNmThreads), 0, s, x, n8, n, mask, val,
                         vec);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sa
