// Sparse-input GEMV family for gfx950.
//
// y[b] = sum over kept k of WT[k][:] * v[b][k], with WT = W^T stored
// row-major, so each kept activation entry selects one contiguous
// 2*d_out-byte run of weights and every skipped entry skips one.
// (RaNA author replies, Q5.1: the columns of zero activation entries are
// skipped; TEAL README / Q-Sparse replies: decode is a batch-1 GEMV.)
//
// Two kernel designs serve every entry point of the family.
//
// Split-K (large weights).  Launch 1, k_gemv: workgroup i owns output tile
// i % go and input slice i / go.
//   phase 1  it builds the list of kept rows of its slice in LDS: threshold /
//            mask / SwiGLU score decided per element, compacted with wave64
//            ballot + mbcnt and an LDS scan of wave totals (ascending);
//   phase 2  its threads stream the listed rows for the output tile with
//            16-byte loads (8 fp16 per lane; a 128-output tile is one
//            256-byte run per row), U rows in flight per thread, fp32 FMA.
//            The loads carry the non-temporal hint: each weight byte is
//            read once per call, and streaming it through L2 at normal
//            priority would evict x, the partial tiles and the counters
//            (measured: 13.0 -> 12.3 us on the 4096 x 11008 call);
//   phase 3  row lanes are summed in LDS and the fp32 partial tile is
//            stored.
// The partial tiles are then summed over slices, in slice order, into fp16 y
// (deterministic), in one of two ways:
//   two launches  plain partial stores; launch 2, k_reduce, sums them after
//                 the kernel boundary.
//   one launch    partials are written with device-coherent stores, every
//                 wave waits for them to complete, and one thread per
//                 workgroup takes a ticket from its output tile's counter;
//                 the workgroup that draws the last ticket sums the tile
//                 (same grouping and order as k_reduce, so both ways give
//                 identical bits) and resets the counter for the next call.
//                 Each counter sits on its own 128-byte line: same-line
//                 atomics serialise at ~10 ns each on this part, separate
//                 lines proceed in parallel.  When every slice of a tile
//                 runs on one XCD (output tiles a multiple of 8), the
//                 partials stay in that XCD's L2 instead of being written
//                 through, and the ticket verifies the placement
//                 (store_handoff).
//
// Full-K (small weights, batch <= 2).  k_gemv_fk: each workgroup owns
// 8*LPR outputs and walks all of d_in; no partials, one launch.  Chosen
// only where its grid covers every CU or the walk is short; other small
// weights take split-K with one workgroup per CU.
//
// With go a multiple of 8, all slices of one output tile run on one XCD
// (workgroups are dispatched round-robin over the 8 XCDs), and the
// concurrently running workgroups of one slice read the same weight rows.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "validate.hpp"

namespace sa {
namespace {

struct Tiling {
  int tile_o;   // outputs per workgroup
  int threads;  // workgroup size
  int unroll;   // rows in flight per thread
  int full_k;   // 0: split-K (k_gemv + k_reduce), 1: full-K (k_gemv_fk)
};
// Compiled tile shapes (for batch 1; other batches use index 0 / 8).
constexpr Tiling kTilings[] = {
    {128, 256, 8, 0},  {256, 256, 8, 0}, {256, 512, 8, 0}, {128, 512, 8, 0},
    {512, 256, 8, 0},  {128, 256, 16, 0}, {64, 256, 8, 0}, {256, 256, 4, 0},
    {16, 1024, 8, 1},  {16, 512, 16, 1},  {8, 512, 16, 1},
};
constexpr int kNumTilings = (int)(sizeof(kTilings) / sizeof(kTilings[0]));
constexpr bool split_tiles_fit_tickets() {
  for (const Tiling& t : kTilings)
    if (!t.full_k && t.tile_o < kMinSplitTileO) return false;
  return true;
}
static_assert(split_tiles_fit_tickets(), "a split-K tile narrower than the counter region assumes");
constexpr int kDefaultSplitK = 0;     // any batch / mode
constexpr int kDefaultSplitKHot = 0;  // batch 1 of threshold / dense / list (measured best)
constexpr int kDefaultFullK = 8;
// SwiGLU slices start on 64-entry boundaries (each wave writes whole mask
// words); the other modes take any slice length.
constexpr int kSwigluSliceAlign = 64;
// Scored N:M slices start on multiples of 32, so no group of m <= 32 entries
// spans two slices, and a group's entries sit in consecutive lanes.
constexpr int kScoredNMSliceAlign = 32;
constexpr int kMaxGk = 256;     // input slices per output tile
// default split-K grid: about one workgroup per 64 KB a CU streams, 2 to 4
// workgroups per CU (measured)
constexpr double kBytesPerWorkgroup = 65536.0;
constexpr int kMinWgsPerCu = 2;
constexpr int kMaxWgsPerCu = 4;
constexpr int kBatch2OneLaunchMaxGk = 24;  // batch 2: one launch up to this many slices
constexpr int kReduceGroups = 16;  // slice groups of the final sum (both hand-offs)
constexpr size_t kTicketBytes = kGemvTicketBytes;
static_assert((size_t)(kMaxDOut / kMinSplitTileO) * kTicketStride * 4 <= kTicketBytes,
              "one hand-off counter per output tile of the longest output");
constexpr size_t kMaxListLds = 48 * 1024;
// weights up to this size run full-K in one launch (latency-bound anyway)
constexpr int64_t kFullKMaxWeightBytes = 8 << 20;
// Small weights (<= kSmallSplitMaxWeightBytes) on split-K: one workgroup per
// CU and slices of at least kSmallMinSlice rows (shorter ones cost more in
// the hand-off than they gain), 64-wide tiles up to kSmallNarrowDout outputs.
// Full-K serves them only when its grid (one workgroup per 16 outputs)
// covers every CU or a walk is short (d_in <= kFullKShortDin): one
// workgroup streams at a per-CU rate, so a small grid leaves most of the
// chip's bandwidth unused (measured: 1024 x 4096 dense 15.1 us full-K,
// 6.0 us split-K).
constexpr int64_t kSmallSplitMaxWeightBytes = 16 << 20;
constexpr int kSmallMinSlice = 128;
constexpr int64_t kSmallNarrowDout = 1024;
constexpr int kSplitNarrowTiling = 6;
constexpr int64_t kFullKShortDin = 1024;

int g_tiling = -1;     // -1: automatic
int g_target_wgs = 0;  // 0: automatic
int g_handoff = 0;     // 0: automatic, 1: two launches, 2: one launch, 3: one launch, in L2
                        // where every slice of a tile shares an XCD
int g_test_hooks = 0;  // bit 0: slice 0 of each tile reports XCD id ^ 1 (placement check);
                       // bit 1: the Top-K GEMV always takes two launches

struct KParams {
  const uint16_t* wt;
  int64_t d_out, d_in;
  const uint16_t* x;
  const uint32_t* xmask;
  float t;
  const int32_t* idx;
  const uint16_t* val;
  const int32_t* nnz;
  int64_t cap;
  const uint16_t* g;
  const uint16_t* u;
  const double* colnorm;
  double t64;
  int swiglu_mode;
  uint32_t* out_mask;
  int32_t* out_nnz;
  uint16_t* y;
  int batch;
  float* part;
  int32_t* slice_cnt;
  uint32_t* tickets;  // non-null: one-launch hand-off
  int xcd_skew;       // test hook: slice 0 reports XCD id ^ 1 to the placement check
  int go, gk, slice;
  int64_t topk_k;        // kModeTopKSel: entries kept per row
  const float* alpha;    // [batch] output scale per row, or null
  const uint16_t* bias;  // [d_out] fp16 added to every row, or null
  // scored mode (batch 1): shift, weight norms (colnorm), fp64 threshold
  // (t64) and, with the variance correction, per-(slice, tile) sums
  // [gk][go][2] of x'^2 and kept x'^2 (null: no correction)
  const uint16_t* mu;
  double* vsum;
  int var;  // scored mode: apply the variance correction
  int sn, sm;  // scored N:M mode: n kept of every m (m a power of two <= 32)
  const int32_t* cut;  // Top-K mode: [batch][2] (tau, i*) of the select
};

constexpr int kModeListBatched = 5;  // kModeList with batch > 1

// Chunks of x a workgroup loads before deciding (one-pass phase 1); longer
// slices, and batch 8 (whose registers are full), take the chunk loop.
template <int B>
constexpr int kOnePassChunks = B == 1 ? 4 : (B <= 4 ? 2 : 0);

typedef float f4v __attribute__((ext_vector_type(4)));

// Threshold decision on one fp16 activation entry: the magnitude threshold
// (|x| >= t and x != 0), or the rank adapter's masker, x^2 >= t.  The square
// of an fp16 value is exact in fp32, so no rounding takes the decision.
template <int MODE>
__device__ __forceinline__ bool keep_entry(uint16_t xb, float t) {
  const float v = h2f(xb);
  if constexpr (MODE == kModeSquare) return v * v >= t;
  return mag_key(xb) != 0 && fabsf(v) >= t;
}

// Top-K mode: entry i of a row survives the select iff its magnitude key is
// above the row's cutoff tau, or equal to it and i <= i* (the select's pair).
__device__ __forceinline__ bool topk_keep(uint16_t xb, int64_t i, int tau, int istar) {
  const int key = mag_key(xb);
  return key > tau || (key == tau && i <= (int64_t)istar);
}
template <int MODE>
constexpr bool kTopKMode = MODE == kModeTopK || MODE == kModeTopKSel;


// Modes whose output takes the correction alpha * sum + bias (the list GEMV
// and the scored mode); every other mode stores the plain rounding.
template <int MODE>
constexpr bool kScoredMode = MODE == kModeScored || MODE == kModeScoredNM;
template <int MODE>
constexpr bool kCorrected = MODE == kModeList || MODE == kModeListBatched || kScoredMode<MODE>;

// Scored mode, one entry: the shifted value x' = fp16(fp32(x) - fp32(mu))
// (returned in xb), kept iff |x'| * colnorm >= t in fp64 and x' != 0; its
// square joins the variance-correction sums.  m and c are the entry's shift
// and weight norm, loaded with x.
__device__ __forceinline__ bool scored_keep(const KParams& p, uint16_t& xb, uint16_t m, double c,
                                            bool in, double& s_all, double& s_kept) {
  if (p.mu != nullptr) xb = f2h(h2f(xb) - h2f(m));
  const float v = h2f(xb);
  const double a = fabs((double)v);
  const bool kb = in && (p.colnorm != nullptr ? a * c : a) >= p.t64 && v != 0.f;
  const double q = (double)v * (double)v;
  s_all += in ? q : 0.0;
  s_kept += kb ? q : 0.0;
  return kb;
}

// Scored N:M mode, one entry: x' and its score as scored_keep; kept iff
// fewer than n entries of its group of m rank before it (a larger score, or
// an equal score at a lower position), i.e. the n largest scores of the
// group, ties to the lower index -- the rule of the scored sparsifier.  The
// group's m entries sit in m consecutive lanes (slices start on multiples of
// 32 and chunks span whole waves), so the ranks come from m - 1 cross-lane
// reads.  Every lane of the wave calls it; `in` clears lanes past the slice
// (whole groups, as d_in % m == 0).
// Rank of this lane's score in its group of M lanes (unrolled: the M - 1
// cross-lane reads are in flight together).
template <int M>
__device__ __forceinline__ int group_rank(double sc) {
  const int lane = lane_id();
  const int pos = lane & (M - 1), base = lane - pos;
  int rank = 0;
#pragma unroll
  for (int r = 1; r < M; ++r) {
    const int pp = (pos + r) & (M - 1);
    const double so = __shfl(sc, base + pp, kWave);
    rank += (so > sc || (so == sc && pp < pos)) ? 1 : 0;
  }
  return rank;
}

// The same rank from fp32 roundings of the scores, exchanged by DPP row
// rotations (a VALU operand modifier, no LDS round trip).  Rounding to fp32
// is monotone, so a strictly larger fp32 key means a strictly larger fp64
// score; when no two keys of a group are equal the fp32 ranks are the fp64
// ranks.  If any group of the wave has two equal keys (equal scores, zeros,
// or scores closer than fp32 resolves) the whole wave takes group_rank.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {  // every lane reads a lane of its own row
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                             0xf, 0xf, false));
}
// quad_perm controls (lane i of a quad reads lane (ctrl >> 2i) & 3): the
// quad rotated by 1, 2, 3; row_half_mirror: lane i of 8 reads lane 7 - i,
// which sits in the other quad of its 8; row_ror:R rotates a row of 16.
constexpr int kQuadRot1 = 0x39, kQuadRot2 = 0x4e, kQuadRot3 = 0x93, kHalfMirror = 0x141;
constexpr int kRowRor = 0x120;
// Compares f with g rotated by R..15 lanes within the row of 16.
template <int R>
__device__ __forceinline__ void rank_rot(float f, float g, int& rank, bool& tie) {
  if constexpr (R < 16) {
    const float go = dpp_f<kRowRor + R>(g);
    rank += go > f ? 1 : 0;
    tie = tie || go == f;
    rank_rot<R + 1>(f, g, rank, tie);
  }
}
template <int M>
__device__ __forceinline__ int group_rank_fast(double sc, bool in) {
  const float f = (float)sc;
  int rank = 0;
  bool tie = false;
  auto cmp = [&](float g) {
    rank += g > f ? 1 : 0;
    tie = tie || g == f;
  };
  auto quad = [&](float g) {  // the three other lanes of g's quad
    cmp(dpp_f<kQuadRot1>(g));
    cmp(dpp_f<kQuadRot2>(g));
    cmp(dpp_f<kQuadRot3>(g));
  };
  if constexpr (M == 4) {
    quad(f);
  } else if constexpr (M == 8) {
    quad(f);
    const float h = dpp_f<kHalfMirror>(f);  // a lane of the other quad, then its quad
    cmp(h);
    quad(h);
  } else {
    rank_rot<1>(f, f, rank, tie);
    if constexpr (M == 32) {  // the other row of 16 of the group
      const float h = __shfl_xor(f, 16, kWave);
      cmp(h);
      rank_rot<1>(f, h, rank, tie);
    }
  }
  if (__ballot(in && tie) != 0) return group_rank<M>(sc);  // uniform
  return rank;
}

__device__ __forceinline__ bool scored_keep_nm(const KParams& p, uint16_t& xb, uint16_t m,
                                               double c, bool in, double& s_all,
                                               double& s_kept) {
  if (p.mu != nullptr) xb = f2h(h2f(xb) - h2f(m));
  const float v = h2f(xb);
  const double a = fabs((double)v);
  const double sc = p.colnorm != nullptr ? a * c : a;
  int rank;
  switch (p.sm) {  // uniform
    case 4: rank = group_rank_fast<4>(sc, in); break;
    case 8: rank = group_rank_fast<8>(sc, in); break;
    case 16: rank = group_rank_fast<16>(sc, in); break;
    default: rank = group_rank_fast<32>(sc, in); break;
  }
  const bool kb = in && rank < p.sn;
  const double q = (double)v * (double)v;
  s_all += in ? q : 0.0;
  s_kept += kb ? q : 0.0;
  return kb;
}

// The variance correction from the sums: sqrt(all / kept), 1 if none kept.
__device__ __forceinline__ float var_alpha(double all, double kept) {
  return kept > 0.0 ? (float)sqrt(all / kept) : 1.f;
}

// One output value: the fp32 sum, scaled by its row's alpha and shifted by its
// output's bias when the call gives them (the corrected GEMV: variance
// correction and the static shift's product), rounded to fp16.  Without
// either it is the plain rounding, bit for bit.
__device__ __forceinline__ uint16_t finish(float acc, const float* alpha, const uint16_t* bias,
                                           int b, int64_t o) {
  if (alpha == nullptr && bias == nullptr) return f2h(acc);
  const float a = alpha != nullptr ? alpha[b] : 1.f;
  const float c = bias != nullptr ? h2f(bias[o]) : 0.f;
  return f2h(fmaf(acc, a, c));
}

// Slot of this thread in a chunk compaction (ascending thread order) and the
// chunk total.  `wsum` holds NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int chunk_slot(bool keep, int* wsum, int& total, uint64_t& wmask) {
  const uint64_t m = __ballot(keep);
  const int w = (int)threadIdx.x / kWave;
  if (lane_id() == 0) wsum[w] = (int)__popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    const int c = wsum[i];
    off += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  wmask = m;
  return off + lanes_below(m);
}

// s = SiLU(g) = g / (1 + exp(-g)), h = s*u and the masker score, in fp64 and
// in the order written (no contraction), as the pages' masks are defined.
__device__ __forceinline__ bool swiglu_keep(uint16_t gb, uint16_t ub, double cn, int mode,
                                            double t, float& hv) {
#pragma clang fp contract(off)
  const double gg = (double)h2f(gb);
  const double uu = (double)h2f(ub);
  const double s = gg / (1.0 + exp(-gg));
  const double h = s * uu;
  const double score = (mode == 0) ? fabs(s) : fabs(h) * cn;
  hv = (float)h;
  return score >= t;
}

// Device-coherent access for the one-launch hand-off.  Each XCD has its own
// L2, and a device-scope release/acquire fence would write back or
// invalidate a whole L2 per workgroup.  Instead the values handed over are
// written and read with relaxed device-scope atomics, which the hardware
// keeps coherent across XCDs, and each wave waits for its stores to
// complete before its workgroup takes a ticket: a ticket then certifies
// that the workgroup's partials are visible to every XCD.
template <typename T>
__device__ __forceinline__ void store_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The L2-local form.  Workgroups are dispatched to the 8 XCDs round-robin,
// workgroup b on XCD (b + r) mod 8 for one r per launch (measured on every
// grid size tried, also beside a concurrent kernel), so when the number of
// output tiles go is a multiple of 8, every slice of a tile runs on one XCD.
// Its partials then only need that XCD's L2: workgroup-scope atomic stores
// and loads (sc0) skip the L1 but are not written through to memory, which
// saves the write-through's wait before the ticket.  Kernel boundaries write
// back and invalidate L2, so nothing stale outlives a call, and the ticket's
// reset may stay in L2 as well.  The ticket checks the premise: with x its
// XCD, every workgroup adds one arrival, x and x^2 in separate fields, and
// the last one sees one XCD exactly when sum x = gk x_last and
// sum x^2 = gk x_last^2 (zero variance); otherwise it cannot see the other
// XCDs' partials and computes every slice of its tile itself (k_gemv).
template <typename T>
__device__ __forceinline__ void store_handoff(T* p, T v, int local) {
  if (local)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_handoff(const T* p, int local) {
  return local ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
               : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kLocalMaxGk = 64;  // the ticket's fields (k_gemv) hold this many slices
static_assert((kLocalMaxGk - 1) * 15 + 15 < 1024 && kLocalMaxGk * 225 < 65536,
              "the ticket's sum fields must not overflow");
// XCD of the calling workgroup (hardware register XCC_ID, bits 3:0)
__device__ __forceinline__ uint32_t xcd_id() {
  return (uint32_t)__builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 0xfu;
}

__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Variance-correction sums over a row's slices, in one fixed order that both
// hand-offs use: lane l of one wave adds slices l, l + 64, l + 128, ... in
// increasing order (a0/k0 hold slice l's sums, 0 past gk), then the wave's
// lanes are added by an xor tree.  get(kk) returns slice kk's pair.
template <typename Get>
__device__ __forceinline__ void var_wave_sums(double& a, double& k, int gk, Get get) {
  for (int kk = lane_id() + kWave; kk < gk; kk += kWave) {
    const double2 v = get(kk);
    a += v.x;
    k += v.y;
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, kWave);
    k += __shfl_xor(k, off, kWave);
  }
}

// Final sum of one output tile over the gk partial tiles, by the workgroup
// that arrived last.  Thread pairs (g, o) -- slice group g of 16, output o
// -- add slices g, g+16, g+32, ... in increasing order; then the groups are
// added in order 0..15 through LDS.  Per output this is k_reduce's grouping
// and order, so both hand-offs round identically.  A wave's 64 lanes take 64
// consecutive outputs of one slice group, so each load is one wave-uniform
// address plus the lane: whole lines per wave and few address registers.
//
// VAR (scored mode with the variance correction): wave 0 also loads every
// slice's sums of this tile (stored before their tickets), with the partials
// in flight, and sets *alpha_w before the barrier that precedes the outputs.
template <int TILE_O, int NT, int B, bool LOCAL, bool VAR = false>
__device__ __forceinline__ void handoff_reduce(const KParams& p, int64_t o0, unsigned char* smem,
                                               const float* alpha, const uint16_t* bias,
                                               int oblk = 0, float* alpha_w = nullptr) {
  constexpr int G = kReduceGroups;
  constexpr int PAIRS = G * TILE_O;
  constexpr int PP = (PAIRS + NT - 1) / NT;  // pairs per thread
  constexpr int KL = PP >= 16 ? 1 : 16 / PP; // loads per pair per batch
  static_assert(TILE_O % kWave == 0 && NT % kWave == 0, "a wave stays in one slice group");
  float* red = reinterpret_cast<float*>(smem);  // [G][TILE_O]
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int w0 = __builtin_amdgcn_readfirstlane(tid - lane);
  const int64_t stride = (int64_t)B * p.d_out;
  double va = 0.0, vk = 0.0;
  const bool var_wave = VAR && p.var && tid < kWave;
  auto vsum_at = [&](int kk) {
    const double* src = p.vsum + ((int64_t)kk * p.go + oblk) * 2;
    return make_double2(load_handoff(src, (int)LOCAL), load_handoff(src + 1, (int)LOCAL));
  };
  if constexpr (VAR) {
    if (var_wave && lane < p.gk) {
      const double2 v = vsum_at(lane);
      va = v.x;
      vk = v.y;
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    if (b >= p.batch) break;
    float s[PP];
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) s[pp] = 0.f;
    for (int k0 = 0; k0 < p.gk; k0 += G * KL) {
      float tmp[PP][KL];
#pragma unroll
      for (int pp = 0; pp < PP; ++pp) {
        const int e0 = w0 + pp * NT;  // wave-uniform
        const int g = e0 / TILE_O;
        const int col0 = e0 % TILE_O;
        const bool ok_o = e0 < PAIRS && o0 + col0 + lane < p.d_out;
        const float* base = p.part + (int64_t)b * p.d_out + o0 + col0;
#pragma unroll
        for (int q = 0; q < KL; ++q) {
          const int kk = k0 + g + q * G;
          tmp[pp][q] = (ok_o && kk < p.gk)
                           ? load_handoff(base + (int64_t)kk * stride + lane, (int)LOCAL)
                           : 0.f;
        }
      }
#pragma unroll
      for (int pp = 0; pp < PP; ++pp)
#pragma unroll
        for (int q = 0; q < KL; ++q) s[pp] += tmp[pp][q];
    }
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      const int e = tid + pp * NT;
      if (e < PAIRS) red[e] = s[pp];
    }
    if constexpr (VAR) {
      if (var_wave) {
        var_wave_sums(va, vk, p.gk, vsum_at);
        if (tid == 0) *alpha_w = var_alpha(va, vk);
      }
    }
    __syncthreads();
    for (int oo = tid; oo < TILE_O; oo += NT) {
      const int64_t og = o0 + oo;
      if (og < p.d_out) {
        float acc = red[oo];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) acc += red[gg * TILE_O + oo];
        p.y[(int64_t)b * p.d_out + og] = finish(acc, alpha, bias, b, og);
      }
    }
    __syncthreads();
  }
}

// Sampled lower bound in an ascending int32 list: number of entries < key.
// Two rounds of wave loads (64 samples, then one segment) instead of a
// serial binary search.  Whole wave participates; result is wave-uniform.
__device__ __forceinline__ int64_t wave_lower_bound(const int32_t* __restrict__ a, int64_t n,
                                                    int64_t key) {
  if (n <= 0) return 0;
  const int lane = lane_id();
  const int64_t q = ((int64_t)lane * n) / kWave;  // ascending sample positions, q_0 = 0
  const bool below = (int64_t)a[q] < key;
  const int c = (int)__popcll(__ballot(below));  // samples < key form a prefix
  if (c == 0) return 0;
  const int64_t lo = ((int64_t)(c - 1) * n) / kWave;               // a[lo] < key
  const int64_t hi = (c < kWave) ? ((int64_t)c * n) / kWave : n;  // a[hi] >= key (or end)
  int add = 0;
  for (int64_t p0 = lo + 1; p0 < hi; p0 += kWave) {
    const int64_t p = p0 + lane;
    const bool b = p < hi && (int64_t)a[p] < key;
    add += (int)__popcll(__ballot(b));
  }
  return lo + 1 + add;  // a[0..lo] are all < key
}

// ---------------------------------------------------------------------------
// split-K, launch 1
// ---------------------------------------------------------------------------
template <int MODE, int TILE_O, int NT, int U, int B, bool LOCAL = false>
__global__ __launch_bounds__(NT) void k_gemv(KParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int wsum[NT / kWave];
  // The output-correction pointers are read here, with the other arguments:
  // left to the compiler, their scalar load lands where they are first
  // needed, and its wait then holds back the weight stream (measured: +0.25
  // us per call).
  const float* alpha_arg = nullptr;
  const uint16_t* bias_arg = nullptr;
  if constexpr (kCorrected<MODE>) {
    alpha_arg = p.alpha;
    bias_arg = p.bias;
    asm volatile("" : "+s"(alpha_arg), "+s"(bias_arg));
  }
  constexpr int OL = TILE_O / 8;  // lanes across the output tile
  constexpr int R = NT / OL;      // row lanes
  static_assert(R >= 1 && NT % OL == 0, "tile shape");

  const int tid = (int)threadIdx.x;
  const int oblk = (int)(blockIdx.x % (unsigned)p.go);
  const int kblk = (int)(blockIdx.x / (unsigned)p.go);
  if ((int64_t)oblk * TILE_O >= p.d_out) return;  // a padding tile (whole workgroup)
  const int SL = p.slice;
  int tk_tau[B], tk_ist[B];  // Top-K mode: each row's cutoff, read with the other arguments
  if constexpr (MODE == kModeTopK) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int bb = b < p.batch ? b : 0;
      tk_tau[b] = p.cut[2 * bb];
      tk_ist[b] = p.cut[2 * bb + 1];
    }
  } else if constexpr (MODE == kModeTopKSel) {
    __shared__ SelLds sel_lds;
    constexpr int E = kTopkSelPerThread;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (b < p.batch) {
        const uint16_t* xb = p.x + (int64_t)b * p.d_in;
        uint16_t v[E];
        load_run<E>(xb, (int64_t)tid * E, p.d_in, (reinterpret_cast<uintptr_t>(xb) & 15u) == 0, v);
        wg_topk_cutoff<NT, E>(v, p.d_in, p.topk_k, sel_lds, tk_tau[b], tk_ist[b]);
      } else {
        tk_tau[b] = tk_tau[0];
        tk_ist[b] = tk_ist[0];
      }
    }
  }
  int* lk = reinterpret_cast<int*>(smem);
  float* lv = reinterpret_cast<float*>(smem + (size_t)SL * 4);
  // Batch > 1: the values are the activations' fp16 bits, [B][SLH] with SLH
  // even and > SL, so two consecutive kept entries are one 32-bit read; a
  // zero after the last kept entry pairs an odd count.
  constexpr bool kPairs = B > 1;
  const int SLH = (SL + 2) & ~1;
  uint16_t* lvh = reinterpret_cast<uint16_t*>(smem + (size_t)SL * 4);
  uint32_t* const ticket = p.tickets + (int64_t)oblk * kTicketStride;
  const int64_t o0 = (int64_t)oblk * TILE_O;
  // scored mode with the variance correction: alpha of the row (set below)
  __shared__ float s_alpha;
  // scored mode with VAR: per-wave sums of x'^2 ([0, NW)) and kept x'^2 ([NW, 2 NW))
  double* vred = nullptr;
  if constexpr (kScoredMode<MODE>) {
    __shared__ double vred_lds[2 * (NT / kWave)];
    vred = vred_lds;
  }
  const float* alpha_out = (kScoredMode<MODE> && p.var) ? &s_alpha : alpha_arg;
  __shared__ int s_last;

  // One pass per slice this workgroup computes: its own slice kblk, and only
  // where the tile's slices turned out to run on more than one XCD (see the
  // hand-off), every other slice of the tile as well.
  int kb = kblk;
  bool recompute = false;
  for (;;) {
    // ---------------- phase 1: kept rows of this workgroup -> LDS ----------
    int cnt = 0;
    double s_all = 0.0, s_kept = 0.0;  // scored mode: variance-correction sums
    const int64_t slice_k0 = (int64_t)kb * SL;
    const int64_t slice_span = (slice_k0 + SL < p.d_in ? slice_k0 + SL : p.d_in) - slice_k0;
    if constexpr (MODE == kModeList) {
      int64_t nn = p.nnz[0];
      const int64_t lim = p.cap < p.d_in ? p.cap : p.d_in;
      nn = nn < 0 ? 0 : (nn > lim ? lim : nn);
      const int64_t p0 = ((int64_t)kb * nn) / p.gk;
      const int64_t p1 = ((int64_t)(kb + 1) * nn) / p.gk;
      cnt = (int)(p1 - p0);
      for (int j = tid; j < cnt; j += NT) {
        const int32_t kk = p.idx[p0 + j];
        const bool ok = kk >= 0 && (int64_t)kk < p.d_in;
        lk[j] = ok ? kk : 0;
        lv[j] = ok ? h2f(p.val[p0 + j]) : 0.f;
      }
      __syncthreads();
    } else if constexpr (MODE == kModeListBatched) {
      // Rows of the slice present in any list: mark them in a dense LDS
      // staging area, then compact.
      const int64_t k0 = (int64_t)kb * SL;
      const int64_t k1 = (k0 + SL < p.d_in) ? k0 + SL : p.d_in;
      const int span = (int)(k1 - k0);
      int* flag = reinterpret_cast<int*>(smem + (size_t)SL * 4 + (size_t)B * SLH * 2);
      uint16_t* dv = reinterpret_cast<uint16_t*>(smem + (size_t)SL * 8 + (size_t)B * SLH * 2);
      for (int j = tid; j < SL; j += NT) {
        flag[j] = 0;
#pragma unroll
        for (int b = 0; b < B; ++b) dv[b * SL + j] = 0;
      }
      __syncthreads();
      const int w = tid / kWave;
      for (int b = w; b < p.batch; b += NT / kWave) {
        const int32_t* ib = p.idx + (int64_t)b * p.cap;
        const uint16_t* vb = p.val + (int64_t)b * p.cap;
        int64_t nn = p.nnz[b];
        const int64_t lim = p.cap < p.d_in ? p.cap : p.d_in;
        nn = nn < 0 ? 0 : (nn > lim ? lim : nn);
        const int64_t lo = wave_lower_bound(ib, nn, k0);
        const int64_t hi = wave_lower_bound(ib, nn, k1);
        for (int64_t q = lo + lane_id(); q < hi; q += kWave) {
          const int64_t kk = ib[q];
          if (kk >= k0 && kk < k1) {
            flag[kk - k0] = 1;
            dv[b * SL + (kk - k0)] = vb[q];
          }
        }
      }
      __syncthreads();
      for (int c = 0; c < span; c += NT) {
        const int j = c + tid;
        const bool keep = j < span && flag[j] != 0;
        int total;
        uint64_t wm;
        const int slot = chunk_slot<NT>(keep, wsum, total, wm);
        if (keep) {
          lk[cnt + slot] = (int)(k0 + j);
#pragma unroll
          for (int b = 0; b < B; ++b) lvh[b * SLH + cnt + slot] = dv[b * SL + j];
        }
        cnt += total;
      }
      __syncthreads();
    } else if (kOnePassChunks<B> > 0 && slice_span <= (int64_t)kOnePassChunks<B> * NT) {
      // One pass: every chunk's x (and mask word; SwiGLU: gate, up and norm)
      // loads are issued before any decision, so the slice costs one memory
      // round trip; the kept slots of all chunks come from one table of
      // per-chunk, per-wave ballot counts (one barrier).  Entry k0 + c*NT + tid
      // of chunk c; chunk-major order keeps the list ascending.
      constexpr int PC = kOnePassChunks<B> > 0 ? kOnePassChunks<B> : 1;
      constexpr int NW = NT / kWave;
      __shared__ int wtab[PC * NW];
      const int64_t k0 = (int64_t)kb * SL;
      const int64_t k1 = (k0 + SL < p.d_in) ? k0 + SL : p.d_in;
      const int64_t words = (p.d_in + 31) >> 5;
      const int nch = (int)((slice_span + NT - 1) / NT);  // chunks this slice has
      uint16_t xr[PC][B];
      uint32_t mw[PC][B];
      uint16_t ms[PC];  // scored: shift; SwiGLU: up
      double cs[PC];    // scored, SwiGLU mode 1: weight norm
      float hv[PC];     // SwiGLU: the kept value h
      // Every chunk's loads, also past the slice (clamped to its first entry):
      // leaving the loop early would put a wait for each load before the
      // branch, one round trip per chunk.
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        const int64_t k = k0 + (int64_t)c * NT + tid;
        const int64_t kc = k < k1 ? k : k0;
        if constexpr (MODE == kModeSwiglu) {
          xr[c][0] = p.g[kc];
          ms[c] = p.u[kc];
          cs[c] = p.swiglu_mode != 0 ? p.colnorm[kc] : 0.0;
        } else {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const int64_t bb = b < p.batch ? b : 0;
            xr[c][b] = p.x[bb * p.d_in + kc];
            if constexpr (MODE == kModeMasked) mw[c][b] = p.xmask[bb * words + (kc >> 5)];
          }
        }
        if constexpr (kScoredMode<MODE>) {
          ms[c] = p.mu != nullptr ? p.mu[kc] : (uint16_t)0;
          cs[c] = p.colnorm != nullptr ? p.colnorm[kc] : 1.0;
        }
      }
      const int w = tid / kWave;
      bool keep[PC];
      uint64_t bm[PC];
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        if (c > 0 && c >= nch) break;
        const int64_t k = k0 + (int64_t)c * NT + tid;
        bool any = false;
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const uint16_t xb = xr[c][b];
          bool kb = false;
          if constexpr (MODE == kModeScored) {
            kb = scored_keep(p, xr[c][b], ms[c], cs[c], b < p.batch && k < k1, s_all, s_kept);
          } else if constexpr (MODE == kModeScoredNM) {
            kb = scored_keep_nm(p, xr[c][b], ms[c], cs[c], b < p.batch && k < k1, s_all, s_kept);
          } else if constexpr (MODE == kModeSwiglu) {
            hv[c] = 0.f;
            kb = k < k1 && swiglu_keep(xb, ms[c], cs[c], p.swiglu_mode, p.t64, hv[c]);
          } else if (b < p.batch && k < k1) {
            if constexpr (MODE == kModeThreshold || MODE == kModeSquare) {
              kb = keep_entry<MODE>(xb, p.t);
            } else if constexpr (kTopKMode<MODE>) {
              kb = topk_keep(xb, k, tk_tau[b], tk_ist[b]);
            } else if constexpr (MODE == kModeMasked) {
              kb = ((mw[c][b] >> (k & 31)) & 1u) != 0;
            } else {
              kb = true;
            }
          }
          if (!kb) xr[c][b] = 0;  // what a skipped entry (or absent row) contributes
          any = any || kb;
        }
        keep[c] = any;
        bm[c] = __ballot(any);
        if (lane_id() == 0) wtab[c * NW + w] = (int)__popcll(bm[c]);
        if constexpr (MODE == kModeSwiglu) {
          // the mask: a wave covers 64 entries from a multiple of 64 (slices
          // are aligned to 64), so its two words are its own
          const int64_t kw = k0 + (int64_t)c * NT + (int64_t)w * kWave;
          if (p.out_mask != nullptr && oblk == 0 && lane_id() == 0 && kw < k1) {
            p.out_mask[kw >> 5] = (uint32_t)bm[c];
            if (kw + 32 < p.d_in) p.out_mask[(kw >> 5) + 1] = (uint32_t)(bm[c] >> 32);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        if (c > 0 && c >= nch) break;
        int before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const int v = wtab[c * NW + i];
          before += (i < w) ? v : 0;
          tot += v;
        }
        if (keep[c]) {
          const int slot = cnt + before + lanes_below(bm[c]);
          lk[slot] = (int)(k0 + (int64_t)c * NT + tid);
          if constexpr (kPairs) {
#pragma unroll
            for (int b = 0; b < B; ++b) lvh[b * SLH + slot] = xr[c][b];
          } else if constexpr (MODE == kModeSwiglu) {
            lv[slot] = hv[c];
          } else {
            lv[slot] = h2f(xr[c][0]);
          }
        }
        cnt += tot;
      }
      if constexpr (MODE == kModeSwiglu) {
        if (oblk == 0 && tid == 0) {
          if (p.gk == 1) {
            if (p.out_nnz != nullptr) p.out_nnz[0] = cnt;
          } else {
            store_handoff(p.slice_cnt + kb, (int32_t)cnt, LOCAL);
          }
        }
      }
      __syncthreads();
    } else {
      const int64_t k0 = (int64_t)kb * SL;
      const int64_t k1 = (k0 + SL < p.d_in) ? k0 + SL : p.d_in;
      const int64_t words = (p.d_in + 31) >> 5;
      for (int64_t c = k0; c < k1; c += NT) {
        const int64_t k = c + tid;
        const bool in = k < k1;
        float vb[B];
        uint16_t hb[B];  // fp16 bits of kept values (0 otherwise), batch > 1
        bool any = false;
        if constexpr (MODE == kModeSwiglu) {
          float hv = 0.f;
          any = in && swiglu_keep(p.g[k], p.u[k], p.swiglu_mode != 0 ? p.colnorm[k] : 0.0,
                                  p.swiglu_mode, p.t64, hv);
          vb[0] = hv;
        } else {
          // every row's load first, from in-range addresses (k0 < d_in), so
          // they are in flight together; then the decisions
          const int64_t kc = in ? k : k0;
          uint16_t xr[B];
          uint32_t mw[B];
          uint16_t ms = 0;  // scored: shift and weight norm
          double cs = 1.0;
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const int64_t bb = b < p.batch ? b : 0;
            xr[b] = p.x[bb * p.d_in + kc];
            if constexpr (MODE == kModeMasked) mw[b] = p.xmask[bb * words + (kc >> 5)];
          }
          if constexpr (kScoredMode<MODE>) {
            if (p.mu != nullptr) ms = p.mu[kc];
            if (p.colnorm != nullptr) cs = p.colnorm[kc];
          }
#pragma unroll
          for (int b = 0; b < B; ++b) {
            vb[b] = 0.f;
            hb[b] = 0;
            if constexpr (kScoredMode<MODE>) {
              const bool kp = MODE == kModeScored
                                  ? scored_keep(p, xr[b], ms, cs, in && b < p.batch, s_all, s_kept)
                                  : scored_keep_nm(p, xr[b], ms, cs, in && b < p.batch, s_all,
                                                   s_kept);
              if (kp) {
                vb[b] = h2f(xr[b]);
                hb[b] = xr[b];
                any = true;
              }
            } else if (b < p.batch && in) {
              const uint16_t xb = xr[b];
              bool kb;
              if constexpr (MODE == kModeThreshold || MODE == kModeSquare) {
                kb = keep_entry<MODE>(xb, p.t);
              } else if constexpr (kTopKMode<MODE>) {
                kb = topk_keep(xb, k, tk_tau[b], tk_ist[b]);
              } else if constexpr (MODE == kModeMasked) {
                kb = ((mw[b] >> (k & 31)) & 1u) != 0;
              } else {
                kb = true;
              }
              if (kb) {
                vb[b] = h2f(xb);
                hb[b] = xb;
              }
              any = any || kb;
            }
          }
          if constexpr (MODE == kModeDense) any = in;
        }
        int total;
        uint64_t wm;
        const int slot = chunk_slot<NT>(any, wsum, total, wm);
        if (any) {
          lk[cnt + slot] = (int)k;
          if constexpr (kPairs) {
#pragma unroll
            for (int b = 0; b < B; ++b) lvh[b * SLH + cnt + slot] = hb[b];
          } else {
            lv[cnt + slot] = vb[0];
          }
        }
        if constexpr (MODE == kModeSwiglu) {
          // each wave covers 64 consecutive entries starting at a multiple of 64
          if (p.out_mask != nullptr && oblk == 0 && lane_id() == 0) {
            const int64_t kw = c + (int64_t)(tid / kWave) * kWave;
            if (kw < k1) {
              p.out_mask[kw >> 5] = (uint32_t)wm;
              if (kw + 32 < p.d_in) p.out_mask[(kw >> 5) + 1] = (uint32_t)(wm >> 32);
            }
          }
        }
        cnt += total;
      }
      if constexpr (MODE == kModeSwiglu) {
        if (oblk == 0 && tid == 0) {
          if (p.gk == 1) {
            if (p.out_nnz != nullptr) p.out_nnz[0] = cnt;
          } else {
            store_handoff(p.slice_cnt + kb, (int32_t)cnt, LOCAL);
          }
        }
      }
      __syncthreads();
    }

    if constexpr (kPairs) {
      if (tid < B) lvh[tid * SLH + cnt] = 0;  // the pad after the last kept entry
      __syncthreads();
    }

    // ---------------- phase 2: stream the kept rows --------------------------
    const int o_lane = tid % OL;
    const int r_lane = tid / OL;
    const int64_t o = o0 + (int64_t)o_lane * 8;
    const bool o_ok = o < p.d_out;
    const uint16_t* __restrict__ wcol = p.wt + (o_ok ? o : 0);
    const int64_t ld = p.d_out;

    float acc[B][8];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[b][i] = 0.f;

    if constexpr (!kPairs) {
      // Rows j = r_lane, r_lane + R, ... in two halves of H rows: one half's
      // loads stay in flight while the other half is consumed.  Rows are added
      // in increasing j whatever U is.  Loads are unconditional (a branch per
      // load would make every wait a full drain): past the end of the list a
      // thread re-reads the list's last row, a cache hit, and consume() skips it.
      constexpr int H = U / 2;
      static_assert(U % 2 == 0, "two halves");
      auto issue = [&](half8 (&w)[H], int j0) {
    #pragma unroll
        for (int q = 0; q < H; ++q) {
          const int j = j0 + q * R;
          const int row = lk[j < cnt ? j : cnt - 1];
          w[q] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(wcol + (int64_t)row * ld));
        }
      };
      auto consume = [&](const half8 (&w)[H], int j0) {
    #pragma unroll
        for (int q = 0; q < H; ++q) {
          const int j = j0 + q * R;
          if (j < cnt) {
    #pragma unroll
            for (int b = 0; b < B; ++b) {
              const float vv = lv[b * SL + j];
    #pragma unroll
              for (int i = 0; i < 8; ++i) acc[b][i] = fmaf((float)w[q][i], vv, acc[b][i]);
            }
          }
        }
      };
      if constexpr (kScoredMode<MODE>) {
        // Scored mode with the variance correction: this slice's sums of x'^2
        // and kept x'^2, reduced per wave while the first rows are in flight
        // (every lane takes part); the workgroup's sum follows in phase 3.
        half8 wa[H], wb[H];
        const bool rows = r_lane < cnt;
        if (rows) {
          issue(wa, r_lane);
          issue(wb, r_lane + H * R);
        }
        if (p.var) {
#pragma unroll
          for (int off = kWave / 2; off >= 1; off >>= 1) {
            s_all += __shfl_xor(s_all, off, kWave);
            s_kept += __shfl_xor(s_kept, off, kWave);
          }
          if (lane_id() == 0) {
            vred[tid / kWave] = s_all;
            vred[NT / kWave + tid / kWave] = s_kept;
          }
        }
        if (rows) {
          for (int j0 = r_lane; j0 < cnt; j0 += U * R) {
            consume(wa, j0);
            issue(wa, j0 + U * R);
            consume(wb, j0 + H * R);
            issue(wb, j0 + U * R + H * R);
          }
        }
      } else {
        if (r_lane < cnt) {
          half8 wa[H], wb[H];
          issue(wa, r_lane);
          issue(wb, r_lane + H * R);
          for (int j0 = r_lane; j0 < cnt; j0 += U * R) {
            consume(wa, j0);
            issue(wa, j0 + U * R);
            consume(wb, j0 + H * R);
            issue(wb, j0 + U * R + H * R);
          }
        }
      }
    } else {
      // Batch > 1: kept entries in pairs (2m, 2m+1), m = r_lane, r_lane + R,
      // ...; v_dot2_f32_f16 adds both rows' products for one output and batch
      // row in one instruction (fp32 accumulate), half the VALU work of one
      // FMA per row.  An odd count pairs its last entry with the zero pad (the
      // row is read twice, its second value is 0).  Same halves as above.
      typedef _Float16 h2v __attribute__((ext_vector_type(2)));
      const int npair = (cnt + 1) >> 1;
      constexpr int HP = U / 4;  // pairs per half: U rows in flight
      static_assert(U % 4 == 0, "two halves of pairs");
      auto issue2 = [&](half8 (&wa)[HP], half8 (&wb)[HP], int m0) {
#pragma unroll
        for (int q = 0; q < HP; ++q) {
          const int m = m0 + q * R;
          const int mm = m < npair ? m : npair - 1;
          const int ja = 2 * mm, jb = 2 * mm + 1 < cnt ? 2 * mm + 1 : 2 * mm;
          wa[q] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(wcol + (int64_t)lk[ja] * ld));
          wb[q] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(wcol + (int64_t)lk[jb] * ld));
        }
      };
      auto consume2 = [&](const half8 (&wa)[HP], const half8 (&wb)[HP], int m0) {
#pragma unroll
        for (int q = 0; q < HP; ++q) {
          const int m = m0 + q * R;
          if (m < npair) {
            h2v wp[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) wp[i] = h2v{wa[q][i], wb[q][i]};
#pragma unroll
            for (int b = 0; b < B; ++b) {
              const h2v xp = *reinterpret_cast<const h2v*>(lvh + b * SLH + 2 * m);
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[b][i] = __builtin_amdgcn_fdot2(wp[i], xp, acc[b][i], false);
            }
          }
        }
      };
      if (r_lane < npair) {
        half8 a0[HP], b0[HP], a1[HP], b1[HP];
        issue2(a0, b0, r_lane);
        issue2(a1, b1, r_lane + HP * R);
        for (int m0 = r_lane; m0 < npair; m0 += 2 * HP * R) {
          consume2(a0, b0, m0);
          issue2(a0, b0, m0 + 2 * HP * R);
          consume2(a1, b1, m0 + HP * R);
          issue2(a1, b1, m0 + 2 * HP * R + HP * R);
        }
      }
    }

    // ---------------- phase 3: reduce row lanes, store the tile --------------
    __syncthreads();  // the kept list is no longer needed; reuse its LDS
    float* red = reinterpret_cast<float*>(smem);
    const bool single = p.gk == 1;
    const bool handoff = !single && p.tickets != nullptr;
    // Scored mode with VAR: the slice's sums.  One slice is the whole input:
    // alpha now (read after the barrier below).  Otherwise the sums go beside
    // this workgroup's partial, stored before its ticket, so the tile's last
    // workgroup reads every slice's sums with the partials.
    if constexpr (kScoredMode<MODE>) {
      if (p.var && tid == 0) {
        double a = 0.0, k = 0.0;
        for (int i = 0; i < NT / kWave; ++i) {
          a += vred[i];
          k += vred[NT / kWave + i];
        }
        if (single) {
          s_alpha = var_alpha(a, k);
        } else {
          double* dst = p.vsum + ((int64_t)kb * p.go + oblk) * 2;
          if (handoff) {
            store_handoff(dst, a, LOCAL);
            store_handoff(dst + 1, k, LOCAL);
          } else {
            dst[0] = a;
            dst[1] = k;
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (b >= p.batch) break;
#pragma unroll
      for (int i = 0; i < 8; ++i) red[r_lane * TILE_O + o_lane * 8 + i] = acc[b][i];
      __syncthreads();
      for (int oo = tid; oo < TILE_O; oo += NT) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) s += red[r * TILE_O + oo];
        const int64_t og = o0 + oo;
        if (og < p.d_out) {
          float* dst = p.part + ((int64_t)kb * B + b) * p.d_out + og;
          if (single)
            p.y[(int64_t)b * p.d_out + og] = finish(s, alpha_out, bias_arg, b, og);
          else if (handoff)
            store_handoff(dst, s, LOCAL);
          else
            *dst = s;
        }
      }
      __syncthreads();
    }
    if (!handoff) return;

    // ---------------- phase 4: one-launch hand-off ---------------------------
    if (!recompute) {
      wait_stores();
      __syncthreads();
      if (tid == 0) {
        if constexpr (LOCAL) {
          // fields: arrivals [5:0], sum x [15:6], sum x^2 [31:16]; every one
          // stays in its field up to the last arrival (gk <= kLocalMaxGk)
          const uint32_t x = xcd_id() ^ ((p.xcd_skew != 0 && kblk == 0) ? 1u : 0u);
          const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u | (x << 6) | ((x * x) << 16),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t gk = (uint32_t)p.gk;
          const uint32_t sx = ((prev >> 6) & 1023u) + x;
          const uint32_t sxx = (prev >> 16) + x * x;
          s_last = ((prev & 63u) != gk - 1) ? 0 : (sx == gk * x && sxx == gk * x * x) ? 1 : 2;
        } else {
          const unsigned prev =
              __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_last = (prev == (unsigned)(p.gk - 1)) ? 1 : 0;
        }
      }
      __syncthreads();
      if (s_last == 0) return;
      if (s_last == 1) break;
      // The tile's slices ran on more than one XCD (possible only in the L2
      // form): the other XCDs' partials sit in their own L2s, out of reach.
      // Recompute every other slice here instead, storing each partial into
      // this XCD's L2 exactly as its own workgroup would have: a partial is a
      // fixed function of the inputs, so the sum below comes out bit for bit
      // as it would have.  Slow, and never taken under round-robin dispatch.
      recompute = true;
      kb = -1;
    }
    kb = kb + 1 == kblk ? kb + 2 : kb + 1;
    if (kb >= p.gk) break;
    __syncthreads();
  }  // one pass per slice
  if (recompute) {  // the recomputed partials, visible to every wave of this workgroup
    wait_stores();
    __syncthreads();
  }
  handoff_reduce<TILE_O, NT, B, LOCAL, kScoredMode<MODE>>(p, o0, smem, alpha_out, bias_arg,
                                                         oblk, &s_alpha);
  if constexpr (MODE == kModeSwiglu) {
    if (oblk == 0 && p.out_nnz != nullptr) {
      int c = 0;
      for (int kk = tid; kk < p.gk; kk += NT)
        c += load_handoff(p.slice_cnt + kk, LOCAL);
      int tot;
      (void)block_exclusive_scan<NT>(c, wsum, tot);
      if (tid == 0) p.out_nnz[0] = tot;
    }
  }
  if (tid == 0) {  // ready for the next call
    if constexpr (LOCAL)  // in L2; written back when the kernel ends, before the next call
      __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    else
      store_coherent(ticket, 0u);
  }
}

// ---------------------------------------------------------------------------
// split-K, launch 2: y[b][o] = sum over slices in order of the partials.
// Thread (g, c) of a 256-thread workgroup adds slices g, g+16, ... of output
// quad c (float4 loads, all in flight), then the 16 groups are added in
// fixed order through LDS.
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int gk,
                                                int64_t d_out, uint16_t* __restrict__ y,
                                                const int32_t* __restrict__ slice_cnt,
                                                int32_t* __restrict__ out_nnz,
                                                const float* __restrict__ alpha,
                                                const uint16_t* __restrict__ bias,
                                                const double* __restrict__ vsum, int go) {
  constexpr int C = 16, G = kReduceGroups, kLoads = 16;
  __shared__ f4v red[G][C];
  __shared__ int scan[256 / kWave];
  __shared__ float s_alpha;
  const int tid = (int)threadIdx.x;
  if (vsum != nullptr) {
    // the variance correction of the (single) row from every slice's sums
    // (tile 0's copies; every tile's are the same)
    if (tid < kWave) {
      auto at = [&](int kk) {
        return make_double2(vsum[(int64_t)kk * go * 2], vsum[(int64_t)kk * go * 2 + 1]);
      };
      double a = 0.0, k = 0.0;
      if (tid < gk) {
        const double2 v = at(tid);
        a = v.x;
        k = v.y;
      }
      var_wave_sums(a, k, gk, at);
      if (tid == 0) s_alpha = var_alpha(a, k);
    }
    __syncthreads();
    alpha = &s_alpha;
  }
  const int c = tid % C;
  const int g = tid / C;
  const int b = (int)blockIdx.y;
  const int64_t o4 = ((int64_t)blockIdx.x * C + c) * 4;
  f4v s = {0.f, 0.f, 0.f, 0.f};
  if (o4 < d_out) {
    const float* base = part + (int64_t)b * d_out + o4;
    const int64_t stride = (int64_t)B * d_out;
    for (int k0 = g; k0 < gk; k0 += G * kLoads) {
      f4v tmp[kLoads];
#pragma unroll
      for (int q = 0; q < kLoads; ++q) {
        const int kk = k0 + q * G;
        tmp[q] = (kk < gk) ? *reinterpret_cast<const f4v*>(base + (int64_t)kk * stride)
                           : f4v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int q = 0; q < kLoads; ++q) s += tmp[q];
    }
  }
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && o4 < d_out) {
    f4v acc = red[0][c];
#pragma unroll
    for (int gg = 1; gg < G; ++gg) acc += red[gg][c];
    uint16_t* yo = y + (int64_t)b * d_out + o4;
#pragma unroll
    for (int i = 0; i < 4; ++i) yo[i] = finish(acc[i], alpha, bias, b, o4 + i);
  }
  if (out_nnz != nullptr && blockIdx.x == 0 && b == 0) {
    int cnt = 0;
    for (int kk = tid; kk < gk; kk += 256) cnt += slice_cnt[kk];
    int tot;
    (void)block_exclusive_scan<256>(cnt, scan, tot);
    if (tid == 0) out_nnz[0] = tot;
  }
}

// ---------------------------------------------------------------------------
// Full-K: no split of d_in, hence no partial tiles and one launch.  Each
// workgroup owns TO = 8*LPR outputs (LPR lanes x 16 bytes of every weight
// row) and walks every input index (or list entry), RL = NT/LPR rows at a
// time, U rows in flight per thread.  Entries that are not kept switch their
// lanes' loads off, so no compaction is needed.  Lanes are summed with a
// fixed xor butterfly and waves through LDS in fixed order.  Workgroups are
// renumbered so that consecutive output tiles -- which share 128-byte lines
// of every row -- run on the same XCD and share its L2.
// ---------------------------------------------------------------------------
template <int MODE, int NT, int LPR, int U, int B>
__global__ __launch_bounds__(NT) void k_gemv_fk(KParams p) {
  constexpr int TO = LPR * 8;
  constexpr int RL = NT / LPR;
  constexpr int NW = NT / kWave;
  static_assert(MODE != kModeSwiglu || LPR <= 2, "mask words need >= 32 indices per wave");
  const float* alpha_arg = nullptr;  // read with the other arguments (see k_gemv)
  const uint16_t* bias_arg = nullptr;
  if constexpr (kCorrected<MODE>) {
    alpha_arg = p.alpha;
    bias_arg = p.bias;
    asm volatile("" : "+s"(alpha_arg), "+s"(bias_arg));
  }
  __shared__ float red[NW][B][TO];
  __shared__ int wcnt[NW];
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const unsigned G = gridDim.x;
  const unsigned bi = blockIdx.x;
  const int oblk = (G % 8u == 0u) ? (int)((bi % 8u) * (G / 8u) + bi / 8u) : (int)bi;
  const int sub = tid % LPR;
  const int rl = tid / LPR;
  const int64_t o = (int64_t)oblk * TO + sub * 8;
  const bool o_ok = o < p.d_out;
  const uint16_t* __restrict__ wcol = p.wt + (o_ok ? o : 0);
  const int64_t ld = p.d_out;
  int tk_tau[B], tk_ist[B];  // Top-K mode: each row's cutoff
  if constexpr (MODE == kModeTopK) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int bb = b < p.batch ? b : 0;
      tk_tau[b] = p.cut[2 * bb];
      tk_ist[b] = p.cut[2 * bb + 1];
    }
  }
  const int64_t words = (p.d_in + 31) >> 5;

  int64_t n = p.d_in;
  if constexpr (MODE == kModeList) {
    const int64_t lim = p.cap < p.d_in ? p.cap : p.d_in;
    n = p.nnz[0];
    n = n < 0 ? 0 : (n > lim ? lim : n);
  }

  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[b][i] = 0.f;
  int kept_count = 0;  // SwiGLU: kept entries seen by this thread (sub 0 only)
  double s_all = 0.0, s_kept = 0.0;  // scored: variance-correction sums (sub 0 only)

  for (int64_t j0 = rl; j0 < n; j0 += (int64_t)RL * U) {
    int64_t row[U];
    float v[U][B];
    bool keep[U];
    // Every load of the U entries first, from in-range addresses (entry 0
    // past the end), so that they are in flight together; then the
    // decisions.  A load inside a divergent branch would wait before the
    // branch joins: one round trip per entry.
    uint16_t xa[U][B];  // x; list values; SwiGLU gate
    uint16_t xu[U];     // SwiGLU up; scored shift
    uint32_t mw[U][B];  // masked: mask words
    int32_t ix[U];      // list indices
    double cn[U];       // scored, SwiGLU mode 1: weight norms
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int64_t j = j0 + (int64_t)q * RL;
      const int64_t jc = j < n ? j : 0;
      if constexpr (MODE == kModeList) {
        ix[q] = p.idx[jc];
        xa[q][0] = p.val[jc];
      } else if constexpr (MODE == kModeSwiglu) {
        xa[q][0] = p.g[jc];
        xu[q] = p.u[jc];
        cn[q] = p.swiglu_mode != 0 ? p.colnorm[jc] : 0.0;
      } else if constexpr (MODE == kModeScored) {
        xa[q][0] = p.x[jc];
        xu[q] = p.mu != nullptr ? p.mu[jc] : (uint16_t)0;
        cn[q] = p.colnorm != nullptr ? p.colnorm[jc] : 1.0;
      } else {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int64_t bb = b < p.batch ? b : 0;
          xa[q][b] = p.x[bb * p.d_in + jc];
          if constexpr (MODE == kModeMasked) mw[q][b] = p.xmask[bb * words + (jc >> 5)];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int64_t j = j0 + (int64_t)q * RL;
      const bool in = j < n;
      row[q] = in ? j : 0;
      keep[q] = false;
#pragma unroll
      for (int b = 0; b < B; ++b) v[q][b] = 0.f;
      if constexpr (MODE == kModeList) {
        if (in) {
          const int32_t kk = ix[q];
          const bool ok = kk >= 0 && (int64_t)kk < p.d_in;
          row[q] = ok ? kk : 0;
          keep[q] = ok;
          v[q][0] = ok ? h2f(xa[q][0]) : 0.f;
        }
      } else if constexpr (MODE == kModeSwiglu) {
        float hv = 0.f;
        keep[q] = in && swiglu_keep(xa[q][0], xu[q], cn[q], p.swiglu_mode, p.t64, hv);
        v[q][0] = hv;
      } else if constexpr (MODE == kModeScored) {
        double a = 0.0, k = 0.0;
        keep[q] = scored_keep(p, xa[q][0], xu[q], cn[q], in, a, k);
        v[q][0] = keep[q] ? h2f(xa[q][0]) : 0.f;
        if (sub == 0) {
          s_all += a;
          s_kept += k;
        }
      } else {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          if (in && b < p.batch) {
            const uint16_t xb = xa[q][b];
            bool kb;
            if constexpr (MODE == kModeThreshold || MODE == kModeSquare) {
              kb = keep_entry<MODE>(xb, p.t);
            } else if constexpr (MODE == kModeTopK) {
              kb = topk_keep(xb, j, tk_tau[b], tk_ist[b]);
            } else if constexpr (MODE == kModeMasked) {
              kb = ((mw[q][b] >> (j & 31)) & 1u) != 0;
            } else {
              kb = true;
            }
            if (kb) v[q][b] = h2f(xb);
            keep[q] = keep[q] || kb;
          }
        }
      }
    }
    if constexpr (MODE == kModeSwiglu) {
      // mask words and kept count, written once (workgroup 0).  A wave's
      // sub-0 lanes cover 64/LPR consecutive indices starting at a multiple
      // of 64/LPR.
      if (bi == 0) {
#pragma unroll
        for (int q = 0; q < U; ++q) {
          const uint64_t m = __ballot(keep[q]);
          if (sub == 0 && keep[q]) ++kept_count;
          if (p.out_mask != nullptr && lane == 0) {
            const int64_t base = j0 - rl + (int64_t)q * RL + (int64_t)wv * (kWave / LPR);
            uint64_t bits = 0;
#pragma unroll
            for (int r = 0; r < kWave / LPR; ++r) bits |= ((m >> (r * LPR)) & 1ull) << r;
            for (int h = 0; h < (kWave / LPR) / 32; ++h)
              if (base + 32 * h < p.d_in) p.out_mask[(base >> 5) + h] = (uint32_t)(bits >> (32 * h));
          }
        }
      }
    }
    half8 w[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if (keep[q] && o_ok) {
        w[q] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(wcol + row[q] * ld));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[q][i] = (half_t)0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if (keep[q]) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[b][i] = fmaf((float)w[q][i], v[q][b], acc[b][i]);
      }
    }
  }

  // lanes with the same `sub` hold partial sums of the same outputs
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) acc[b][i] += __shfl_xor(acc[b][i], off, kWave);
  if (lane < LPR) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wv][b][lane * 8 + i] = acc[b][i];
  }
  if constexpr (MODE == kModeSwiglu) {
    if (bi == 0) {
      int c = kept_count;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) c += __shfl_xor(c, off, kWave);
      if (lane == 0) wcnt[wv] = c;
    }
  }
  __shared__ float s_alpha;
  __shared__ double vred[2][NW];
  const bool var = MODE == kModeScored && p.var != 0;
  if (var) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      s_all += __shfl_xor(s_all, off, kWave);
      s_kept += __shfl_xor(s_kept, off, kWave);
    }
    if (lane == 0) {
      vred[0][wv] = s_all;
      vred[1][wv] = s_kept;
    }
  }
  __syncthreads();
  if (var && tid == 0) {
    double a = 0.0, k = 0.0;
    for (int g = 0; g < NW; ++g) {
      a += vred[0][g];
      k += vred[1][g];
    }
    s_alpha = var_alpha(a, k);
  }
  if (var) __syncthreads();
  const float* alpha_out = var ? &s_alpha : alpha_arg;
  for (int e = tid; e < TO * B; e += NT) {
    const int b = e / TO;
    const int oo = e % TO;
    const int64_t og = (int64_t)oblk * TO + oo;
    if (b < p.batch && og < p.d_out) {
      float s = red[0][b][oo];
#pragma unroll
      for (int g = 1; g < NW; ++g) s += red[g][b][oo];
      p.y[(int64_t)b * p.d_out + og] = finish(s, alpha_out, bias_arg, b, og);
    }
  }
  if constexpr (MODE == kModeSwiglu) {
    if (bi == 0 && tid == 0 && p.out_nnz != nullptr) {
      int tot = 0;
      for (int g = 0; g < NW; ++g) tot += wcnt[g];
      p.out_nnz[0] = tot;
    }
  }
}

// out[k] = sqrt(sum_o WT[k][o]^2) in fp64, one wave per row, fixed-order
// butterfly reduction (deterministic).
__global__ __launch_bounds__(256) void k_col_norms(const uint16_t* __restrict__ wt, int64_t d_in,
                                                   int64_t d_out, double* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= d_in) return;  // uniform per wave
  const int lane = lane_id();
  const uint16_t* r = wt + row * d_out;
  double s = 0.0;
  for (int64_t o = (int64_t)lane * 8; o < d_out; o += 8 * kWave) {
    const half8 h = *reinterpret_cast<const half8*>(r + o);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double v = (double)(float)h[i];
      s += v * v;  // exact product: v has 11 significant bits
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
  if (lane == 0) out[row] = sqrt(s);
}

// ---------------------------------------------------------------------------
// dense GEMV on a row-major weight (the rank adapter's v = B x)
// ---------------------------------------------------------------------------
// One wave per output row: y[b][i] = sum_k W[i][k] x[b][k], W [d_out][d_in]
// row-major.  Lane l takes the 8-column chunks l, l + 64, ..., U at a time
// (16-byte loads of W and of each x row when VEC: d_in % 8 == 0 and 16-byte
// aligned bases; 2-byte loads with bounds otherwise), multiplies with packed
// fp16 dot products into fp32, and the wave's sum is taken with DPP row
// shifts.  Every output is one wave's own dot product: no partial sums, no
// hand-off, and each row's bytes are read once as contiguous 1 KB runs.
template <int B, bool VEC>
__global__ __launch_bounds__(256) void k_gemv_rows(const uint16_t* __restrict__ w, int64_t d_out,
                                                   int64_t d_in, const uint16_t* __restrict__ x,
                                                   int batch, uint16_t* __restrict__ y) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  constexpr int U = B <= 2 ? 8 : (B <= 4 ? 4 : 2);  // chunks in flight per lane
  const int lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * 4 + (int64_t)(threadIdx.x / kWave);
  if (row >= d_out) return;  // the whole wave
  const uint16_t* wr = w + row * d_in;
  const int64_t nch = (d_in + 7) / 8;  // 8-column chunks of a row
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.f;
  for (int64_t c0 = 0; c0 < nch; c0 += (int64_t)kWave * U) {
    u32x4 wv[U], xv[U][B];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * kWave + lane;
      if constexpr (VEC) {
        const int64_t cc = c < nch ? c : nch - 1;  // in range; its x is zeroed below
        wv[u] = *reinterpret_cast<const u32x4*>(wr + cc * 8);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int64_t bb = b < batch ? b : 0;
          const u32x4 t = *reinterpret_cast<const u32x4*>(x + bb * d_in + cc * 8);
          xv[u][b] = c < nch ? t : u32x4{0u, 0u, 0u, 0u};
        }
      } else {
        uint32_t wq[4], xq[B][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t k0 = c * 8 + 2 * e, k1 = k0 + 1;
          const uint32_t lo = k0 < d_in ? wr[k0] : 0u, hi = k1 < d_in ? wr[k1] : 0u;
          wq[e] = lo | (hi << 16);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const int64_t bb = b < batch ? b : 0;
            const uint32_t xl = k0 < d_in ? x[bb * d_in + k0] : 0u;
            const uint32_t xh = k1 < d_in ? x[bb * d_in + k1] : 0u;
            xq[b][e] = xl | (xh << 16);
          }
        }
        wv[u] = u32x4{wq[0], wq[1], wq[2], wq[3]};
#pragma unroll
        for (int b = 0; b < B; ++b) xv[u][b] = u32x4{xq[b][0], xq[b][1], xq[b][2], xq[b][3]};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the elements go through scalars: a bit cast of a vector element
          // taken in place would reinterpret element 0
          const uint32_t we = wv[u][e], xe = xv[u][b][e];
          acc[b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, we), __builtin_bit_cast(h2v, xe),
                                          acc[b], false);
        }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    // wave sum: rows of 16 by DPP row shifts, then the four row totals
    float s = acc[b];
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x111, 0xf, 0xf, true));
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x112, 0xf, 0xf, true));
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x114, 0xf, 0xf, true));
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x118, 0xf, 0xf, true));
    const float tot = (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 15)) +
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 31))) +
                      (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 47)) +
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 63)));
    if (lane == 0 && b < batch) y[(int64_t)b * d_out + row] = f2h(tot);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int batch_pad(int batch) { return batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t ticket_off, slicecnt_off, part_off, vsum_off, cut_off, total;
};

// Workspace: the hand-off counters (a fixed region, zero between calls: the
// caller zero-fills it once, every call leaves it zero), per-slice kept
// counts (SwiGLU) and the fp32 partial tiles [slice][batch][d_out].  The
// counts and partials are written before they are read within one call.
Layout ws_layout(int64_t d_out, int64_t d_in, int64_t batch) {
  const int64_t gk_max = d_in < kMaxGk ? d_in : kMaxGk;
  Layout L;
  L.ticket_off = 0;
  L.slicecnt_off = kTicketBytes;
  L.part_off = L.slicecnt_off + align256((size_t)gk_max * 4);
  L.vsum_off = L.part_off + align256((size_t)gk_max * (size_t)batch_pad((int)batch) *
                                     (size_t)d_out * 4);
  const size_t go_max = (size_t)((d_out + kMinSplitTileO - 1) / kMinSplitTileO);
  L.cut_off = L.vsum_off + align256((size_t)gk_max * go_max * 2 * sizeof(double));
  L.total = L.cut_off + 256;  // SA_MAX_BATCH (tau, i*) pairs of sparse_gemv_topk
  return L;
}

// LDS of the kept list: indices, then values (fp32 at batch 1; fp16 [B][SLH]
// at batch > 1), then for batched lists the dense staging (flags, fp16).
size_t list_lds_bytes(int mode, int slice, int B) {
  const size_t slh = (size_t)((slice + 2) & ~1);
  size_t b = (size_t)slice * 4 + (B > 1 ? (size_t)B * slh * 2 : (size_t)slice * 4);
  if (mode == kModeListBatched) b += (size_t)slice * 4 + (size_t)B * slice * 2;
  return b;
}

struct Plan {
  int go, gk, slice;
  size_t smem;
  int go_grid;  // output tiles of the grid: go, or go padded to a multiple of 8
};

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

namespace {

// The split-K kernel instance for a mode, tiling and batch (split-K tilings
// exist for batch 1 of the hot modes; everything else uses tiling 0).
using KFn = void (*)(KParams);

template <int MODE, int B, bool LOCAL>
KFn kernel_tiling_scope(int tiling) {
  if constexpr (B == 1 && (MODE == kModeThreshold || MODE == kModeDense || MODE == kModeList ||
                           kTopKMode<MODE>)) {
    switch (tiling) {
      case 1: return k_gemv<MODE, 256, 256, 8, B, LOCAL>;
      case 2: return k_gemv<MODE, 256, 512, 8, B, LOCAL>;
      case 3: return k_gemv<MODE, 128, 512, 8, B, LOCAL>;
      case 4: return k_gemv<MODE, 512, 256, 8, B, LOCAL>;
      case 5: return k_gemv<MODE, 128, 256, 16, B, LOCAL>;
      case 6: return k_gemv<MODE, 64, 256, 8, B, LOCAL>;
      case 7: return k_gemv<MODE, 256, 256, 4, B, LOCAL>;
      default: return k_gemv<MODE, 128, 256, 8, B, LOCAL>;
    }
  } else {
    (void)tiling;
    return k_gemv<MODE, 128, 256, 8, B, LOCAL>;
  }
}

template <int MODE, int B>
KFn kernel_tiling(int tiling, bool local) {
  if (local) return kernel_tiling_scope<MODE, B, true>(tiling);
  return kernel_tiling_scope<MODE, B, false>(tiling);
}

template <int MODE>
KFn kernel_batch(int tiling, int B, bool local) {
  switch (B) {
    case 1: return kernel_tiling<MODE, 1>(tiling, local);
    case 2: return kernel_tiling<MODE, 2>(tiling, local);
    case 4: return kernel_tiling<MODE, 4>(tiling, local);
    default: return kernel_tiling<MODE, 8>(tiling, local);
  }
}

KFn select_kernel(int mode, int tiling, int B, bool local = false) {
  switch (mode) {
    case kModeThreshold: return kernel_batch<kModeThreshold>(tiling, B, local);
    case kModeDense: return kernel_batch<kModeDense>(tiling, B, local);
    case kModeMasked: return kernel_batch<kModeMasked>(tiling, B, local);
    case kModeList: return kernel_tiling<kModeList, 1>(tiling, local);
    case kModeListBatched: return kernel_batch<kModeListBatched>(tiling, B, local);
    case kModeSwiglu: return kernel_tiling<kModeSwiglu, 1>(tiling, local);
    case kModeScored: return kernel_tiling<kModeScored, 1>(tiling, local);
    case kModeScoredNM: return kernel_tiling<kModeScoredNM, 1>(tiling, local);
    case kModeSquare: return kernel_batch<kModeSquare>(tiling, B, local);
    case kModeTopK: return kernel_batch<kModeTopK>(tiling, B, local);
    case kModeTopKSel:  // batch 1 only (launch_gemv_topk)
      return B == 1 ? kernel_tiling<kModeTopKSel, 1>(tiling, local) : nullptr;
    default: return nullptr;
  }
}

// Workgroups of `fn` that fit on one CU at once (cached).
int resident_per_cu(KFn fn, int nt, size_t smem) {
  static std::mutex mu;
  static struct {
    KFn fn;
    int nt;
    size_t smem;
    int dev, occ;
  } cache[32];
  static int next = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.fn == fn && e.nt == nt && e.smem == smem && e.dev == dev) return e.occ;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(fn), nt,
                                                   smem) != hipSuccess ||
      occ < 1)
    occ = 1;
  cache[next] = {fn, nt, smem, dev, occ};
  next = (next + 1) % 32;
  return occ;
}

// Split-K grid.  Streaming runs at a per-CU rate and the call ends when the
// most loaded CU does; each further workgroup on a CU adds fixed cost
// (x load, compaction, hand-off) of its own.  Measured over slice counts on
// this part, the best grids put k workgroups on every CU (or just under it),
// with k growing with the bytes a CU streams: about one workgroup per 64 KB,
// at least 2 and at most 4.  The bytes are estimated before the call (the
// sparse modes at half the weight), and no grid exceeds what is resident at
// once (a workgroup waiting for a free slot would start only after the
// others finish).  Weights up to kSmallSplitMaxWeightBytes take one
// workgroup per CU instead, and larger ones the best-balanced slice count
// up to k per CU (choose_plan).
Plan plan_for(int mode, int tiling, int64_t d_out, int64_t d_in, int B, int64_t gk_req) {
  Plan pl;
  const Tiling T = kTilings[tiling];
  pl.go = (int)((d_out + T.tile_o - 1) / T.tile_o);
  if (gk_req < 1) gk_req = 1;
  if (gk_req > kMaxGk) gk_req = kMaxGk;
  const int64_t align =
      mode == kModeSwiglu ? kSwigluSliceAlign : (mode == kModeScoredNM ? kScoredNMSliceAlign : 1);
  int64_t slice = (d_in + gk_req - 1) / gk_req;
  slice = (slice + align - 1) / align * align;
  // the kept list of a slice must fit the LDS budget
  const int64_t per_entry = (int64_t)list_lds_bytes(mode, 1, B);
  const int64_t max_slice = (int64_t)kMaxListLds / per_entry / align * align;
  if (slice > max_slice) slice = max_slice;
  pl.slice = (int)slice;
  pl.gk = (int)((d_in + slice - 1) / slice);
  size_t red = (size_t)T.threads * 8 * 4;
  const size_t red4 = (size_t)kReduceGroups * T.tile_o * 4;  // hand-off sum
  if (red4 > red) red = red4;
  const size_t lst = list_lds_bytes(mode, pl.slice, B);
  pl.smem = lst > red ? lst : red;
  pl.go_grid = pl.go;
  return pl;
}

// cus: compute units; resident: workgroups of the kernel that fit on one CU
// (0: ask the device).
Plan choose_plan(int mode, int tiling, int64_t d_out, int64_t d_in, int B, int64_t cus,
                 int resident) {
  const int nt = kTilings[tiling].threads;
  const int64_t go = (d_out + kTilings[tiling].tile_o - 1) / kTilings[tiling].tile_o;
  if (g_target_wgs > 0)  // tuning: the grid asked for
    return plan_for(mode, tiling, d_out, d_in, B, (g_target_wgs + go / 2) / go);
  const double bytes = 2.0 * (double)d_in * (double)d_out * (mode == kModeDense ? 1.0 : 0.5);
  int64_t k = (int64_t)(bytes / (double)cus / kBytesPerWorkgroup + 0.5);
  k = k < kMinWgsPerCu ? kMinWgsPerCu : (k > kMaxWgsPerCu ? kMaxWgsPerCu : k);
  int64_t gk_req = (k * cus) / go;
  if (2 * d_in * d_out <= kSmallSplitMaxWeightBytes) {
    gk_req = cus / go;
    const int64_t most = d_in / kSmallMinSlice;
    if (gk_req > most) gk_req = most;
  }
  const KFn fn = select_kernel(mode, tiling, B);
  Plan pl = plan_for(mode, tiling, d_out, d_in, B, gk_req);
  // Balance: streaming runs at a per-CU rate, so a call ends with its
  // busiest CU.  Of the slice counts up to the target, take the one with the
  // most workgroups per workgroup on the busiest CU (ties: more slices).
  // 22016 x 4096 at 50%: 4 slices (688 workgroups, at most 3 per CU) beat 5
  // (860, at most 4): 19.8 us against 21.0 us.
  if (2 * d_in * d_out > kSmallSplitMaxWeightBytes) {
    double best = 0.0;
    for (int64_t g = gk_req; g >= 1; --g) {
      const Plan c = plan_for(mode, tiling, d_out, d_in, B, g);
      const int64_t wgs = (int64_t)c.go * c.gk;
      const double per = (double)wgs / (double)((wgs + cus - 1) / cus);
      if (per > best * (1.0 + 1e-9)) {
        best = per;
        pl = c;
      }
    }
  }
  // at most one resident wave of workgroups
  for (int i = 0; i < 4 && pl.gk > 1; ++i) {
    const int64_t cap = (int64_t)(resident > 0 ? resident : resident_per_cu(fn, nt, pl.smem)) * cus;
    if ((int64_t)pl.go * pl.gk <= cap) break;
    pl = plan_for(mode, tiling, d_out, d_in, B, cap / go);
  }
  return pl;
}

// Plans are cached per call shape, so a steady stream of calls pays one
// lookup on the host.
Plan make_plan(int mode, int tiling, int64_t d_out, int64_t d_in, int B) {
  static std::mutex mu;
  struct Entry {
    int mode, tiling, B, target, dev;
    int64_t d_out, d_in;
    Plan pl;
    bool used;
  };
  static Entry cache[64];
  static int next = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : cache)
      if (e.used && e.mode == mode && e.tiling == tiling && e.B == B && e.d_out == d_out &&
          e.d_in == d_in && e.target == g_target_wgs && e.dev == dev)
        return e.pl;
  }
  const Plan pl = choose_plan(mode, tiling, d_out, d_in, B, device_cus(), 0);
  std::lock_guard<std::mutex> lock(mu);
  cache[next] = {mode, tiling, B, g_target_wgs, dev, d_out, d_in, pl, true};
  next = (next + 1) % 64;
  return pl;
}

hipError_t launch_split(KFn fn, int nt, const KParams& kp, const Plan& pl, hipStream_t s) {
  KParams arg = kp;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)(pl.go_grid * pl.gk)),
                         dim3(nt), args, pl.smem, s);
}

hipError_t launch_reduce(const KParams& kp, const Plan& pl, int B, bool with_nnz, hipStream_t s) {
  const dim3 grid((unsigned)((kp.d_out / 4 + 15) / 16), (unsigned)kp.batch);
  int32_t* nnz_out = with_nnz ? kp.out_nnz : nullptr;
  switch (B) {
    case 1:
      hipLaunchKernelGGL(k_reduce<1>, grid, dim3(256), 0, s, kp.part, pl.gk, kp.d_out, kp.y,
                         kp.slice_cnt, nnz_out, kp.alpha, kp.bias, kp.vsum, kp.go);
      break;
    case 2:
      hipLaunchKernelGGL(k_reduce<2>, grid, dim3(256), 0, s, kp.part, pl.gk, kp.d_out, kp.y,
                         kp.slice_cnt, nnz_out, kp.alpha, kp.bias, kp.vsum, kp.go);
      break;
    case 4:
      hipLaunchKernelGGL(k_reduce<4>, grid, dim3(256), 0, s, kp.part, pl.gk, kp.d_out, kp.y,
                         kp.slice_cnt, nnz_out, kp.alpha, kp.bias, kp.vsum, kp.go);
      break;
    default:
      hipLaunchKernelGGL(k_reduce<8>, grid, dim3(256), 0, s, kp.part, pl.gk, kp.d_out, kp.y,
                         kp.slice_cnt, nnz_out, kp.alpha, kp.bias, kp.vsum, kp.go);
      break;
  }
  return hipGetLastError();
}

template <int MODE, int NT, int LPR, int U, int B>
hipError_t launch_fk(const KParams& kp, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_fk<MODE, NT, LPR, U, B>), dim3(grid), dim3(NT), 0, s, kp);
  return hipGetLastError();
}

template <int MODE, int B>
hipError_t dispatch_fk(const KParams& kp, int tiling, unsigned grid, hipStream_t s) {
  switch (tiling) {
    case 9: return launch_fk<MODE, 512, 2, 16, B>(kp, grid, s);
    case 10: return launch_fk<MODE, 512, 1, 16, B>(kp, grid, s);
    default: return launch_fk<MODE, 1024, 2, 8, B>(kp, grid, s);
  }
}

}  // namespace

size_t gemv_workspace_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  return ws_layout(d_out, d_in, batch).total;
}

size_t gemv_workspace_cut_offset(int64_t d_out, int64_t d_in, int64_t batch) {
  return ws_layout(d_out, d_in, batch).cut_off;
}

size_t gemv_workspace_zero_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  (void)d_out;
  (void)d_in;
  (void)batch;
  return kTicketBytes;  // the hand-off counters; the rest is written before it is read
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (sparse_gemv_threshold_noalloc):
// a fixed array in device memory, one copy per GPU the library runs on, held
// until the process ends.  It is used exactly as a caller's workspace: its
// first kTicketBytes are the hand-off counters, zero from load time (static
// storage) and left zero by every call; the partial sums follow.  Host code
// reaches it only through the address hipGetSymbolAddress gives for the
// current device (the array's name is not a device address on the host).
// ---------------------------------------------------------------------------
namespace {
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes > kTicketBytes, "room for partials after the counters");

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};
}  // namespace

hipError_t gemv_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

// The kernel and decomposition of one call shape.  cus / resident: the
// device's compute units and the split-K kernel's workgroups per CU (0: ask
// the device); make_plan's cache serves the launcher's own calls.
struct Decision {
  int mode;  // internal mode (batched lists have their own)
  int B;     // compiled batch
  int tiling;
  bool full_k;
  Plan pl;  // split-K only
  bool one_launch;
  bool local;
};

Decision decide_gemv(int mode, int64_t d_out, int64_t d_in, int64_t batch, int64_t cus,
                     int resident, bool cached) {
  Decision d{};
  if (mode == kModeList && batch > 1) mode = kModeListBatched;
  const int B = (mode == kModeSwiglu || mode == kModeList) ? 1 : batch_pad((int)batch);
  // Full-K serves batch <= 2 of every mode except batched lists and the
  // in-workgroup Top-K select, for small weights whose grid fills the chip
  // or whose walk is short.
  const bool sel = mode == kModeTopKSel;
  const bool fk_ok = B <= 2 && mode != kModeListBatched && !sel && mode != kModeScoredNM;
  int tiling = g_tiling;
  const bool hot = B == 1 && (mode == kModeThreshold || mode == kModeDense ||
                              mode == kModeList || mode == kModeTopK || sel);
  if (tiling < 0) {
    const int64_t wbytes = d_in * d_out * 2;
    const bool fk_fills = (d_out + kTilings[kDefaultFullK].tile_o - 1) /
                              kTilings[kDefaultFullK].tile_o >= cus ||
                          d_in <= kFullKShortDin;
    if (fk_ok && wbytes <= kFullKMaxWeightBytes && fk_fills)
      tiling = kDefaultFullK;
    else if (hot)
      tiling = (wbytes <= kSmallSplitMaxWeightBytes && d_out <= kSmallNarrowDout)
                   ? kSplitNarrowTiling
                   : kDefaultSplitKHot;
    else
      tiling = kDefaultSplitK;
  }
  if (kTilings[tiling].full_k && !fk_ok) tiling = kDefaultSplitK;
  if (!kTilings[tiling].full_k && !hot)
    tiling = kDefaultSplitK;  // split-K variants exist for the batch-1 hot modes only
  d.mode = mode;
  d.B = B;
  d.tiling = tiling;
  d.full_k = kTilings[tiling].full_k != 0;
  if (d.full_k) return d;
  d.pl = cached ? make_plan(mode, tiling, d_out, d_in, B)
                : choose_plan(mode, tiling, d_out, d_in, B, cus, resident);
  // One launch at batch 1.  The last workgroup's final sum grows with
  // slices x rows, so at batch 2 one launch pays only with the partials in
  // L2 and few slices, and from batch 3 (padded to 4) a second launch is
  // faster (measured: 11008 x 4096 batch 2, 86 tiles, 17.0 us two launches,
  // 17.6 us one; 12288 x 4096 batch 2, in L2, 17.9 against 18.3 us).
  const bool l2_ok = d.pl.go % 8 == 0 && d.pl.gk <= kLocalMaxGk;
  const bool auto_one = B == 1 || (B == 2 && l2_ok && d.pl.gk <= kBatch2OneLaunchMaxGk);
  d.one_launch = d.pl.gk > 1 && (g_handoff == 0 ? auto_one : g_handoff >= 2);
  // At batch 1 a tile count that is not a multiple of 8 is padded to one:
  // the padding tiles' workgroups exit at once, and every slice of a real
  // tile then shares one XCD too.  Only with at least 8 tiles (the padded
  // count stays within the workspace's per-tile sums) and while the grid
  // still fits one resident wave.
  bool padded = false;
  if (B == 1 && !l2_ok && d.pl.go >= 8 && d.pl.gk <= kLocalMaxGk && d.one_launch &&
      g_handoff != 2) {
    const int go8 = (d.pl.go + 7) / 8 * 8;
    const int nt = kTilings[tiling].threads;
    const int per = resident > 0 ? resident
                                 : resident_per_cu(select_kernel(mode, tiling, B, true), nt,
                                                   d.pl.smem);
    if ((int64_t)go8 * d.pl.gk <= (int64_t)per * cus) {
      d.pl.go_grid = go8;
      padded = true;
    }
  }
  // partials kept in L2 when every slice of a tile runs on one XCD
  d.local = d.one_launch && g_handoff != 2 && (l2_ok || padded);
  return d;
}

}  // namespace

hipError_t launch_gemv(const GemvCall& c, hipStream_t s) {
  const Decision dc = decide_gemv(c.mode, c.d_out, c.d_in, c.batch, device_cus(), 0, true);
  const int mode = dc.mode;
  const int B = dc.B;
  const int tiling = dc.tiling;

  KParams kp{};
  kp.wt = c.wt;
  kp.d_out = c.d_out;
  kp.d_in = c.d_in;
  kp.x = c.x;
  kp.xmask = c.xmask;
  kp.t = c.t;
  kp.idx = c.idx;
  kp.val = c.val;
  kp.nnz = c.nnz;
  kp.cap = c.cap;
  kp.g = c.g;
  kp.u = c.u;
  kp.colnorm = c.colnorm;
  kp.t64 = c.t64;
  kp.swiglu_mode = c.swiglu_mode;
  kp.out_mask = c.out_mask;
  kp.out_nnz = c.out_nnz;
  kp.y = c.y;
  kp.batch = c.batch;
  kp.alpha = c.alpha;
  kp.bias = c.bias;
  kp.mu = c.mu;
  kp.cut = c.cut;
  kp.topk_k = c.topk_k;
  kp.var = ((mode == kModeScored || mode == kModeScoredNM) && c.var) ? 1 : 0;
  kp.sn = c.sn;
  kp.sm = c.sm;

  if (dc.full_k) {
    const unsigned grid = (unsigned)((c.d_out + kTilings[tiling].tile_o - 1) /
                                     kTilings[tiling].tile_o);
    switch (mode) {
      case kModeThreshold:
        return B == 1 ? dispatch_fk<kModeThreshold, 1>(kp, tiling, grid, s)
                      : dispatch_fk<kModeThreshold, 2>(kp, tiling, grid, s);
      case kModeDense:
        return B == 1 ? dispatch_fk<kModeDense, 1>(kp, tiling, grid, s)
                      : dispatch_fk<kModeDense, 2>(kp, tiling, grid, s);
      case kModeMasked:
        return B == 1 ? dispatch_fk<kModeMasked, 1>(kp, tiling, grid, s)
                      : dispatch_fk<kModeMasked, 2>(kp, tiling, grid, s);
      case kModeList: return dispatch_fk<kModeList, 1>(kp, tiling, grid, s);
      case kModeSwiglu: return dispatch_fk<kModeSwiglu, 1>(kp, tiling, grid, s);
      case kModeScored: return dispatch_fk<kModeScored, 1>(kp, tiling, grid, s);
      case kModeSquare:
        return B == 1 ? dispatch_fk<kModeSquare, 1>(kp, tiling, grid, s)
                      : dispatch_fk<kModeSquare, 2>(kp, tiling, grid, s);
      case kModeTopK:
        return B == 1 ? dispatch_fk<kModeTopK, 1>(kp, tiling, grid, s)
                      : dispatch_fk<kModeTopK, 2>(kp, tiling, grid, s);
      default: return hipErrorInvalidValue;
    }
  }

  const Plan& pl = dc.pl;
  const Layout L = ws_layout(c.d_out, c.d_in, c.batch);
  if (pl.gk > 1 && (c.ws == nullptr || c.ws_bytes < L.total)) return hipErrorInvalidValue;
  if (pl.gk > kMaxGk) return hipErrorInvalidValue;  // the workspace holds kMaxGk slices
  unsigned char* ws = static_cast<unsigned char*>(c.ws);
  kp.slice_cnt = ws ? reinterpret_cast<int32_t*>(ws + L.slicecnt_off) : nullptr;
  kp.part = ws ? reinterpret_cast<float*>(ws + L.part_off) : nullptr;
  kp.vsum = (kp.var && ws) ? reinterpret_cast<double*>(ws + L.vsum_off) : nullptr;
  const bool one_launch = dc.one_launch;
  const bool local = dc.local;
  kp.tickets = one_launch ? reinterpret_cast<uint32_t*>(ws + L.ticket_off) : nullptr;
  kp.xcd_skew = g_test_hooks & 1;
  kp.go = pl.go_grid;
  kp.gk = pl.gk;
  kp.slice = pl.slice;

  const KFn fn = select_kernel(mode, tiling, B, local);
  if (fn == nullptr) return hipErrorInvalidValue;
  const hipError_t e = launch_split(fn, kTilings[tiling].threads, kp, pl, s);
  if (e != hipSuccess || pl.gk == 1 || one_launch) return e;
  return launch_reduce(kp, pl, B, mode == kModeSwiglu && c.out_nnz != nullptr, s);
}

namespace {
// The fused Top-K mode of a call: the in-workgroup select applies to a
// split-K plan at batch 1 whose workgroups can hold the row (d_in <= threads
// x kTopkSelPerThread); 0 where it does not.  Measured at 50%: 11008 x 4096
// 15.45 us in one launch against 17.16 us in two.  At batch 2 each workgroup
// would select two rows one after the other, and the two-launch form
// measured as fast (22.18 against 22.32 us).  Longer rows (48 entries per
// thread) made every workgroup's select slower than the separate launch:
// 4096 x 11008, 19.67 against 17.06 us.
int topk_fused_mode(int64_t d_out, int64_t d_in, int64_t batch, int64_t cus, int resident,
                    bool cached, Decision* out) {
  if (batch != 1 || (g_test_hooks & 2) != 0) return 0;
  const Decision d = decide_gemv(kModeTopKSel, d_out, d_in, batch, cus, resident, cached);
  if (d.full_k || d_in > (int64_t)kTilings[d.tiling].threads * kTopkSelPerThread) return 0;
  if (out) *out = d;
  return kModeTopKSel;
}
}  // namespace

hipError_t launch_gemv_topk(const GemvCall& c, int32_t* cut, hipStream_t s) {
  GemvCall g = c;
  const int fused = topk_fused_mode(c.d_out, c.d_in, c.batch, device_cus(), 0, true, nullptr);
  if (fused != 0) {
    g.mode = fused;
    return launch_gemv(g, s);
  }
  const hipError_t e = launch_sparsify_topk(c.x, c.batch, c.d_in, c.topk_k, nullptr, nullptr,
                                            nullptr, nullptr, 0, cut, s);
  if (e != hipSuccess) return e;
  g.mode = kModeTopK;
  g.cut = cut;
  return launch_gemv(g, s);
}

namespace {
template <int B>
void launch_rows_b(bool vec, dim3 grid, const uint16_t* w, int64_t d_out, int64_t d_in,
                   const uint16_t* x, int batch, uint16_t* y, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((k_gemv_rows<B, true>), grid, dim3(256), 0, s, w, d_out, d_in, x, batch, y);
  else
    hipLaunchKernelGGL((k_gemv_rows<B, false>), grid, dim3(256), 0, s, w, d_out, d_in, x, batch,
                       y);
}
}  // namespace

hipError_t launch_gemv_rows(const uint16_t* w, int64_t d_out, int64_t d_in, const uint16_t* x,
                            int batch, uint16_t* y, hipStream_t s) {
  const bool vec = (d_in % 8) == 0 && (reinterpret_cast<uintptr_t>(w) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  const dim3 grid((unsigned)((d_out + 3) / 4));
  switch (batch_pad(batch)) {
    case 1: launch_rows_b<1>(vec, grid, w, d_out, d_in, x, batch, y, s); break;
    case 2: launch_rows_b<2>(vec, grid, w, d_out, d_in, x, batch, y, s); break;
    case 4: launch_rows_b<4>(vec, grid, w, d_out, d_in, x, batch, y, s); break;
    default: launch_rows_b<8>(vec, grid, w, d_out, d_in, x, batch, y, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_col_norms(const uint16_t* wt, int64_t d_in, int64_t d_out, double* out,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_col_norms, dim3((unsigned)((d_in + 3) / 4)), dim3(256), 0, s, wt, d_in,
                     d_out, out);
  return hipGetLastError();
}

int gemv_plan(int mode, int64_t d_out, int64_t d_in, int64_t batch, int cus, int resident,
              int* kernel, int* tile_o, int* go, int* gk, int* handoff) {
  const int64_t n = cus > 0 ? cus : device_cus();
  Decision d = decide_gemv(mode, d_out, d_in, batch, n, resident, false);
  if (mode == kModeTopK) {  // what launch_gemv_topk runs
    Decision f{};
    if (topk_fused_mode(d_out, d_in, batch, n, resident, false, &f) != 0) d = f;
  }
  const Tiling& T = kTilings[d.tiling];
  *kernel = d.full_k ? 1 : 0;
  *tile_o = T.tile_o;
  *go = d.full_k ? (int)((d_out + T.tile_o - 1) / T.tile_o) : d.pl.go;
  *gk = d.full_k ? 1 : d.pl.gk;
  *handoff = (d.full_k || d.pl.gk == 1) ? 0 : (!d.one_launch ? 1 : (d.local ? 3 : 2));
  return 0;
}

int gemv_set_test_hooks(int flags) {
  if (flags < 0 || flags > 3) return 1;
  g_test_hooks = flags;
  return 0;
}

int gemv_set_tuning(int tiling, int target_wgs, int handoff) {
  if (tiling < -1 || tiling >= kNumTilings || target_wgs < 0 || handoff < 0 || handoff > 3)
    return 1;
  g_tiling = tiling;
  g_target_wgs = target_wgs;
  g_handoff = handoff;
  return 0;
}

int gemv_tiling_info(int i, int* tile_o, int* threads, int* unroll) {
  // tile_o of a full-K tiling is reported negated so callers can tell them apart
  if (i < 0 || i >= kNumTilings) return 1;
  if (tile_o) *tile_o = kTilings[i].full_k ? -kTilings[i].tile_o : kTilings[i].tile_o;
  if (threads) *threads = kTilings[i].threads;
  if (unroll) *unroll = kTilings[i].unroll;
  return 0;
}

}  // namespace sa
