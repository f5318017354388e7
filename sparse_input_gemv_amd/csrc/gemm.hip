// MFMA matmuls for gfx950: the dense GEMM baseline and the batched N:M
// activation-sparse GEMM.
//
// Y[T][d_out] = X[T][d_in] * WT[d_in][d_out], fp16 in, fp32 accumulate,
// fp16 out.  (Q-Sparse author replies, answer on batched inference: for
// large batches the activations of every token are N:M sparse -- Block
// Q-Sparse -- and the product is measured against a dense matmul.)
//
// Three engines live here: the pipelined engine (k_gemm_pipe: dense, 2:4 on
// the sparse MFMA, and the whole-tile gather of tile-shared N:M), the
// per-32-row-block gather of tile-shared N:M (k_gemm_shared), and the
// staged-register engine described next (k_gemm), which takes every shape
// the others do not.
//
// Staged-register engine: a 256-thread workgroup computes a BM x 128 output
// tile (BM = 256 or 128) with four waves (2 x 2), each wave (BM/2) x 64 =
// (BM/64) x 2 blocks of 32 x 32.  The K loop steps by 32 with double-buffered
// LDS tiles:
//   B (WT, contiguous along the output index) is transposed into LDS as
//     [n][k] while being staged, two k rows packed per 32-bit LDS word, so
//     each lane's MFMA B operand is one or two 16-byte LDS reads;
//   A is staged as [m][k]:
//     dense      -- X rows as they are;
//     N:M        -- the compressed kept values are scattered into a zero-filled
//                   tile by their mask bits ("gathered dense sub-tiles"), then
//                   the dense MFMA runs (v_mfma_f32_32x32x16_f16);
//     2:4        -- the compressed values stay compressed and the mask bits
//                   become the 2-bit position codes of the gfx950 sparse MFMA
//                   (v_smfmac_f32_32x32x32_f16), halving the MFMA work.
// Lane layouts (checked on the device): 32x32x16 -- lane l holds A[l%32]
// [8(l/32)..+8] and B[8(l/32)..+8][l%32]; result register r of lane l is
// row 8(r/4)+4(l/32)+r%4, column l%32.  Sparse 32x32x32 -- lane l holds the
// 8 kept values of A row l%32 over dense k in [16(l/32), +16) (position
// code of group q in bits 4q..4q+3: first position | second << 2), and B
// rows 8(l/32)..+8 and 16+8(l/32)..+8 of column l%32.
#include "common.hpp"
#include "launch.hpp"

namespace sa {
namespace {

constexpr int BN = 128, BK = 32, NTH = 256;
constexpr int LDA = BK + 8;  // halves per LDS row of A (padding against bank conflicts)
constexpr int LDB = BK + 8;  // halves per LDS row of B^T

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f16v __attribute__((ext_vector_type(16)));

enum AKind : int { kADense = 0, kANM = 1, kA24 = 2, kANMVec = 3, kAGather = 4 };

struct GParams {
  const uint16_t* x;      // dense: X [T][d_in]; sparse: compressed values [T][d_in*n/m]
  const uint32_t* mask;   // sparse: [T][d_in/32]; tile-shared: [ceil(T/tt)][d_in/32]
  const uint16_t* wt;     // [d_in][d_out]
  uint16_t* y;            // [T][d_out]
  int64_t T, d_in, d_out;
  int n, m;
  int tt;                 // tile-shared: rows per pattern
};

// ---- B staging: 32 k rows x 128 n columns -> LDS Bs[n][k] ------------------
// Thread (c = tid % 16, r = tid / 16) loads WT rows k0+2r and k0+2r+1 at
// columns n0 + 8c .. +8 and writes 8 packed (k, k+1) pairs.
struct BRegs {
  u32x4 lo, hi;
};

__device__ __forceinline__ void load_b(const GParams& p, int64_t k0, int64_t n0, BRegs& r) {
  const int tid = (int)threadIdx.x;
  const int c = tid % 16, rr = tid / 16;
  const int64_t n = n0 + 8 * c;
  const int64_t k = k0 + 2 * rr;
  const bool n_ok = n < p.d_out;  // d_out % 8 == 0: the 8 columns are all in or all out
  r.lo = (n_ok && k < p.d_in) ? *reinterpret_cast<const u32x4*>(p.wt + k * p.d_out + n)
                              : u32x4{0u, 0u, 0u, 0u};
  r.hi = (n_ok && k + 1 < p.d_in) ? *reinterpret_cast<const u32x4*>(p.wt + (k + 1) * p.d_out + n)
                                  : u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void store_b(uint16_t* Bs, const BRegs& r) {
  const int tid = (int)threadIdx.x;
  const int c = tid % 16, rr = tid / 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = r.lo[i], b = r.hi[i];
    // columns 8c + 2i and 8c + 2i + 1; each word packs (k, k+1)
    const uint32_t w0 = (a & 0xffffu) | (b << 16);
    const uint32_t w1 = (a >> 16) | (b & 0xffff0000u);
    *reinterpret_cast<uint32_t*>(Bs + (8 * c + 2 * i) * LDB + 2 * rr) = w0;
    *reinterpret_cast<uint32_t*>(Bs + (8 * c + 2 * i + 1) * LDB + 2 * rr) = w1;
  }
}

// ---- A staging ---------------------------------------------------------------
// Work items of a BM x 32 tile, spread over the 256 threads:
//   dense   -- (row, 8-wide chunk): BM*4 items, 16-byte loads;
//   N:M     -- (row, 16-wide half): BM*2 items; the mask bits and the kept
//              values before the half give where its values start;
//   2:4     -- (row, half): the 8 compressed values and the 16-bit position
//              code of the sparse MFMA;
//   N:M with m | 4n (every pattern of the workloads) -- one row per item: a
//              32-wide row tile holds exactly 32n/m kept values, a whole number
//              of 16-byte words at a 16-byte aligned offset, loaded as vectors
//              and scattered by the set bits of the row's mask word.
template <int AK>
struct AItems;
template <>
struct AItems<kADense> {
  static constexpr int kPerRow = 4;
};
template <>
struct AItems<kANM> {
  static constexpr int kPerRow = 2;
};
template <>
struct AItems<kA24> {
  static constexpr int kPerRow = 2;
};
template <>
struct AItems<kANMVec> {
  static constexpr int kPerRow = 1;
};

template <int AK, int BM>
struct ARegs {
  static constexpr int kItems = (BM * AItems<AK>::kPerRow + NTH - 1) / NTH;
  static constexpr int kWords = (AK == kANMVec) ? 4 : (AK == kANM ? 2 : 1);
  u32x4 v[kItems][kWords];
  uint32_t bits[kItems];
};

template <int AK, int BM>
__device__ __forceinline__ void load_a(const GParams& p, int64_t m0, int64_t k0,
                                       ARegs<AK, BM>& r) {
  constexpr int PR = AItems<AK>::kPerRow;
  const int tid = (int)threadIdx.x;
  const int64_t kc = (AK == kADense) ? 0 : p.d_in * p.n / p.m;  // compressed row length
#pragma unroll
  for (int it = 0; it < ARegs<AK, BM>::kItems; ++it) {
    const int item = tid + it * NTH;
    const int lrow = item / PR;
    const int part = item % PR;
    const int64_t row = m0 + lrow;
#pragma unroll
    for (int q = 0; q < ARegs<AK, BM>::kWords; ++q) r.v[it][q] = u32x4{0u, 0u, 0u, 0u};
    r.bits[it] = 0;
    if (lrow >= BM || row >= p.T || k0 >= p.d_in) continue;
    if constexpr (AK == kADense) {
      const int64_t k = k0 + 8 * part;
      if (k < p.d_in) r.v[it][0] = *reinterpret_cast<const u32x4*>(p.x + row * p.d_in + k);
    } else if constexpr (AK == kANMVec) {
      const int C = 32 * p.n / p.m;  // multiple of 8
      r.bits[it] = p.mask[row * (p.d_in / 32) + k0 / 32];
      const uint16_t* src = p.x + row * kc + k0 * p.n / p.m;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (8 * q < C) r.v[it][q] = *reinterpret_cast<const u32x4*>(src + 8 * q);
    } else {
      const int half = part;
      const uint32_t w = p.mask[row * (p.d_in / 32) + k0 / 32];
      const uint32_t bits = half ? (w >> 16) : (w & 0xffffu);
      r.bits[it] = bits;
      if constexpr (AK == kA24) {
        // exactly 8 kept values per 16 dense k; 16-byte aligned because
        // kc % 16 == 0 and k0/2 + 8*half is a multiple of 8
        r.v[it][0] = *reinterpret_cast<const u32x4*>(p.x + row * kc + k0 / 2 + 8 * half);
      } else {
        // kept values of this row before dense k0 + 16*half: k0 is a
        // multiple of 32 and of m, so exactly k0*n/m precede the tile.  The
        // counts are clamped to the row so a malformed mask cannot read past it.
        int64_t before = k0 * p.n / p.m + (half ? __popc(w & 0xffffu) : 0);
        if (before > kc) before = kc;
        int cnt = __popc(bits);
        if (cnt > kc - before) cnt = (int)(kc - before);
        const uint16_t* src = p.x + row * kc + before;
        uint16_t vals[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) vals[e] = (e < cnt) ? src[e] : (uint16_t)0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r.v[it][0][i] = (uint32_t)vals[2 * i] | ((uint32_t)vals[2 * i + 1] << 16);
          r.v[it][1][i] = (uint32_t)vals[8 + 2 * i] | ((uint32_t)vals[8 + 2 * i + 1] << 16);
        }
      }
    }
  }
}

// Scatter the kept values (word-packed, position order) to the set bits of
// `bits` in dst[0..W), after zero-filling it.
template <int W, int NV>
__device__ __forceinline__ void scatter_row(uint16_t* dst, uint32_t bits, const u32x4 (&v)[NV]) {
#pragma unroll
  for (int q = 0; q < W / 8; ++q) *reinterpret_cast<u32x4*>(dst + 8 * q) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int sidx = 0; sidx < W; ++sidx) {
    const uint32_t word = v[sidx / 8][(sidx % 8) / 2];  // static register index
    const uint16_t hv = (uint16_t)((sidx & 1) ? (word >> 16) : (word & 0xffffu));
    if (bits != 0u) {
      dst[__builtin_ctz(bits)] = hv;
      bits &= bits - 1u;
    }
  }
}

template <int AK, int BM>
__device__ __forceinline__ void store_a(uint16_t* As, uint32_t* Aidx, const ARegs<AK, BM>& r) {
  constexpr int PR = AItems<AK>::kPerRow;
  const int tid = (int)threadIdx.x;
#pragma unroll
  for (int it = 0; it < ARegs<AK, BM>::kItems; ++it) {
    const int item = tid + it * NTH;
    const int lrow = item / PR;
    const int part = item % PR;
    if (lrow >= BM) continue;
    if constexpr (AK == kADense) {
      *reinterpret_cast<u32x4*>(As + lrow * LDA + 8 * part) = r.v[it][0];
    } else if constexpr (AK == kANMVec) {
      scatter_row<32, 4>(As + lrow * LDA, r.bits[it], r.v[it]);
    } else if constexpr (AK == kANM) {
      scatter_row<16, 2>(As + lrow * LDA + 16 * part, r.bits[it], r.v[it]);
    } else {
      // compressed values: 8 halves per (row, half) -> As[row][8*half .. +8]
      *reinterpret_cast<u32x4*>(As + lrow * LDA + 8 * part) = r.v[it][0];
      // position code: per group of 4, first set position | second << 2
      uint32_t code = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t nib = (r.bits[it] >> (4 * g)) & 0xfu;
        const uint32_t p0 = nib ? (uint32_t)__builtin_ctz(nib) : 0u;
        const uint32_t rest = nib & (nib - 1u);
        const uint32_t p1 = rest ? (uint32_t)__builtin_ctz(rest) : (p0 == 3u ? 3u : p0 + 1u);
        code |= (p0 | (p1 << 2)) << (4 * g);
      }
      Aidx[lrow * 2 + part] = code;
    }
  }
}

template <int AK, int BM>
__global__ __launch_bounds__(NTH) void k_gemm(GParams p) {
  constexpr int MB = BM / 64;  // 32-row MFMA blocks per wave
  __shared__ __align__(16) uint16_t As[2][BM * LDA];
  __shared__ __align__(16) uint16_t Bs[2][BN * LDB];
  __shared__ uint32_t Aidx[2][AK == kA24 ? BM * 2 : 1];
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;  // 2 x 2 waves, (BM/2) x 64 each

  // tile order: all M tiles of one N strip are consecutive, so the strip of
  // WT stays in cache while they run
  const int64_t mt = (p.T + BM - 1) / BM;
  const int64_t m0 = (int64_t)(blockIdx.x % mt) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x / mt) * BN;

  f16v acc[MB][2];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nk = (p.d_in + BK - 1) / BK;
  ARegs<AK, BM> ar;
  BRegs br;
  load_a<AK, BM>(p, m0, 0, ar);
  load_b(p, 0, n0, br);
  store_a<AK, BM>(As[0], Aidx[0], ar);
  store_b(Bs[0], br);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) {
      load_a<AK, BM>(p, m0, (kt + 1) * BK, ar);
      load_b(p, (kt + 1) * BK, n0, br);
    }
    const uint16_t* as = As[cur];
    const uint16_t* bs = Bs[cur];
    if constexpr (AK == kA24) {
      h16 bop[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int col = wn * 64 + b * 32 + lane % 32;
        const h8 lo = *reinterpret_cast<const h8*>(bs + col * LDB + 8 * (lane / 32));
        const h8 hi = *reinterpret_cast<const h8*>(bs + col * LDB + 16 + 8 * (lane / 32));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bop[b][e] = lo[e];
          bop[b][8 + e] = hi[e];
        }
      }
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const int row = wm * (BM / 2) + a * 32 + lane % 32;
        const h8 aop = *reinterpret_cast<const h8*>(as + row * LDA + 8 * (lane / 32));
        const int code = (int)Aidx[cur][row * 2 + lane / 32];
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(aop, bop[b], acc[a][b], code, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        h8 aop[MB], bop[2];
#pragma unroll
        for (int a = 0; a < MB; ++a) {
          const int row = wm * (BM / 2) + a * 32 + lane % 32;
          aop[a] = *reinterpret_cast<const h8*>(as + row * LDA + kk + 8 * (lane / 32));
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int col = wn * 64 + b * 32 + lane % 32;
          bop[b] = *reinterpret_cast<const h8*>(bs + col * LDB + kk + 8 * (lane / 32));
        }
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[a], bop[b], acc[a][b], 0, 0, 0);
      }
    }
    if (more) {
      store_a<AK, BM>(As[cur ^ 1], Aidx[cur ^ 1], ar);
      store_b(Bs[cur ^ 1], br);
    }
    __syncthreads();
  }

  // epilogue: fp16 stores; register r of lane l is row 8(r/4)+4(l/32)+r%4
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row < p.T && col < p.d_out) p.y[row * p.d_out + col] = f2h(acc[a][b][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Pipelined engine (dense and 2:4 A, d_in a multiple of the kind's K step,
// 16-byte aligned rows).  A 256-thread workgroup computes a BM x 128 output
// tile (BM = 256 or 128, chosen per call at launch), four waves of BM/2 x 64;
// the K loop steps through NS LDS stages (three unless tuned).  Tiles go from
// global memory to LDS with direct loads (global_load_lds: lane l's bytes
// land at the instruction's LDS base + size * l), NS - 1 K steps ahead, so no
// registers hold staged data and the loads of step t+2 overlap the MFMAs of
// step t.
// Two or three workgroups share a CU wherever LDS and registers allow, so
// one's barrier and load waits are covered by the others' MFMAs.
//   Dense: K steps of 32 (72 KB of LDS at BM = 256: two workgroups per CU;
//     measured 8% faster than steps of 64 with one).  X rows, K-contiguous,
//     are stored [m][32] with 16-byte chunks XOR-swizzled by the row (chosen
//     through each lane's source address) so the 32 rows one operand read
//     touches fall in distinct banks.
//   2:4: K steps of 64 (steps of 32 leave too few sparse MFMAs per barrier:
//     measured slower); 128-row tiles take 75 KB, two workgroups per CU.
//     The compressed values, [m][32] (64-byte rows, swizzled as the dense
//     A), and the row's two 32-bit mask words [m][2]; each lane turns its 16
//     mask bits into the position code of the sparse MFMA.
//   B (WT, N-contiguous) is stored [k][128] as it lies in memory (chunks
//     swizzled by k); the MFMA B operand -- consecutive k of one column --
//     comes from LDS transpose reads (ds_read_b64_tr_b16): within a 16-lane
//     group, source lane s addresses 4 halves of row k0 + s/4 at column
//     c0 + 4 (s % 4), and lane i receives column c0 + i of rows k0 .. k0+3
//     (layout checked on the device).
// A stage is reused only after a barrier that follows every wave's reads of
// it; each wait names the exact number of later loads allowed in flight.
// The MFMA sequence per output block is the staged-register engine's, so
// both engines give identical results.
// ---------------------------------------------------------------------------
constexpr int PBN = 128;

typedef short s4v __attribute__((ext_vector_type(4)));
#define SA_LDS4(ptr) ((__attribute__((address_space(3))) s4v*)(ptr))

template <int AK, int BM>
struct Pipe;
template <int BM>
struct Pipe<kADense, BM> {
  static constexpr int kBK = 32;                       // K step
  static constexpr int kMB = BM / 64;                  // 32-row A blocks per wave
  static constexpr int kAHalves = BM * kBK;            // [BM][32]
  static constexpr int kMaskWords = 0;
  static constexpr int kLoadsPerWave = BM / 64 + 2;    // A, B
  static constexpr int kWgsByRegs = BM == 256 ? 2 : 3;  // workgroups per CU the registers allow
};
template <int BM>
struct Pipe<kA24, BM> {
  static constexpr int kBK = 64;
  static constexpr int kMB = BM / 64;
  static constexpr int kAHalves = BM * kBK / 2;        // [BM][32] compressed
  static constexpr int kMaskWords = BM * 2;            // [BM][2]
  static constexpr int kLoadsPerWave = BM / 64 + 4 + BM / 128;  // A, B, mask
  static constexpr int kWgsByRegs = 2;
};
// Tile-shared N:M with one pattern for the whole row tile: the dense engine
// on the compressed values and the kept rows of WT (see pipe_issue).
template <int BM>
struct Pipe<kAGather, BM> : Pipe<kADense, BM> {};
// The tile's pattern in LDS, 4 KB: a byte per kept entry (its position in
// its 32-column mask word) when d_in n / m <= 4096, else the mask row
// itself (d_in <= 32768), searched per load.
constexpr int kGatherMaskWords = 1024;
constexpr int kGatherTableBytes = 4 * kGatherMaskWords;

template <int AK, int BM>
constexpr int pipe_stage_halves() {
  return Pipe<AK, BM>::kAHalves + Pipe<AK, BM>::kBK * PBN + 2 * Pipe<AK, BM>::kMaskWords;
}
// Workgroups per CU with NS stages: what the 160 KB of LDS (the stages plus
// the 2:4 code table) and the registers both allow.
template <int AK, int BM, int NS>
constexpr int pipe_wgs_per_cu() {
  constexpr int lds = NS * pipe_stage_halves<AK, BM>() * 2 + (AK == kA24 ? 256 : 0) +
                      (AK == kAGather ? 4 * kGatherMaskWords : 0);
  constexpr int by_lds = 160 * 1024 / lds;
  static_assert(by_lds >= 1, "stages exceed the LDS");
  return by_lds < Pipe<AK, BM>::kWgsByRegs ? by_lds : Pipe<AK, BM>::kWgsByRegs;
}

// 16-byte chunk swizzles: A rows of 64 bytes (dense and 2:4), B rows of 256
// bytes.  Each spreads the rows one operand read touches over distinct banks
// for 32 or 64 LDS banks.
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int k) { return 4 * (k & 3); }

// s_waitcnt encoding (gfx9 family): vmcnt in bits 3:0 and 15:14, expcnt 6:4
// (7 = no wait), lgkmcnt 11:8 (0 = all LDS reads done)
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One global_load_lds of 16 (or 4) bytes per lane: from `src` to LDS at
// lds_base + 16 * lane (4 * lane).  Written as inline asm so that the
// compiler's automatic waits do not treat the load as a pending write to
// every LDS array (it cannot tell the stages apart and would drain all loads
// before each read); the waits are stated by stage_barrier instead.  The
// instruction has no result register, and the memory clobber keeps LDS
// reads on their side of it.  The LDS base goes in M0 as an input operand
// (the compiler writes M0 itself, so no reserved register is clobbered);
// the s_nop covers the wait state between an M0 write and the load.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ void load_to_lds16(const void* src, const void* lds_base) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "{m0}"(lds_addr(lds_base))
      : "memory");
}
__device__ __forceinline__ void load_to_lds4(const void* src, const void* lds_base) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "{m0}"(lds_addr(lds_base))
      : "memory");
}

// Position of the r-th set bit (r from 0) of a field of at most 32 bits, by
// halving; a field with fewer set bits gives some position below 32.
__device__ __forceinline__ int select_bit(uint32_t b, int r) {
  int pos = 0;
#pragma unroll
  for (int half = 16; half >= 1; half /= 2) {
    const int c = __builtin_popcount(b & ((1u << half) - 1u));
    if (r >= c) {
      r -= c;
      b >>= half;
      pos += half;
    }
  }
  return pos;
}

// This wave's share of the loads of the K step starting at k0 into one stage
// (A, then B, then for 2:4 the mask words).  Rows past T and columns past
// d_out read clamped (valid) addresses; their results are never stored.
template <int AK, int BM>
__device__ __forceinline__ void pipe_issue(const GParams& p, int64_t m0, int64_t n0, int64_t k0,
                                           uint16_t* S, const uint32_t* mrow) {
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  uint16_t* As = S;
  uint16_t* Bs = S + Pipe<AK, BM>::kAHalves;
  constexpr int BK = Pipe<AK, BM>::kBK;
  constexpr int AI = BM / 64;  // A instructions per wave
  // gather, byte-table mode: this lane's two B rows of the step in one read,
  // issued before the A loads so that its latency overlaps them
  static_assert(AK != kAGather || BK / 16 == 2, "two B loads per lane and step");
  uint32_t pair = 0;
  const bool table = AK == kAGather && p.d_in / p.m * p.n <= kGatherTableBytes;
  if constexpr (AK == kAGather) {
    if (table)
      pair = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(mrow) + k0 +
                                                 8 * w + 2 * (lane / 16));
  }
  if constexpr (AK == kADense || AK == kAGather) {
    // gather: A rows are the compressed values, d_in n / m long
    const int64_t lda = AK == kAGather ? p.d_in / p.m * p.n : p.d_in;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int rb = (w * AI + i) * 16;  // 16 rows of 64 bytes per instruction
      const int r = rb + lane / 4;
      const int gc = (lane % 4) ^ swz_a(r);
      int64_t row = m0 + r;
      if (row >= p.T) row = p.T - 1;
      load_to_lds16(p.x + row * lda + k0 + 8 * gc, As + rb * BK);
    }
  } else {
    const int64_t kc = p.d_in / 2;  // compressed row length
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int rb = (w * AI + i) * 16;  // 16 rows of 64 bytes per instruction
      const int r = rb + lane / 4;
      const int gc = (lane % 4) ^ swz_a(r);
      int64_t row = m0 + r;
      if (row >= p.T) row = p.T - 1;
      load_to_lds16(p.x + row * kc + k0 / 2 + 8 * gc, As + rb * (BK / 2));
    }
    uint32_t* Ms = reinterpret_cast<uint32_t*>(Bs + BK * PBN);
    const int64_t words = p.d_in / 32;
    constexpr int MI = BM / 128;  // mask instructions per wave
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int rb = (w * MI + i) * 32;  // 32 rows of 2 words per instruction
      const int r = rb + lane / 2;
      int64_t row = m0 + r;
      if (row >= p.T) row = p.T - 1;
      load_to_lds4(p.mask + row * words + k0 / 32 + (lane % 2), Ms + rb * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < BK / 16; ++i) {
    const int kb = (w * (BK / 16) + i) * 4;  // 4 k rows of 256 bytes per instruction
    const int k = kb + lane / 16;
    const int gc = (lane % 16) ^ swz_b(k);
    int64_t n = n0 + 8 * gc;
    if (n >= p.d_out) n = p.d_out - 8;
    int64_t row = k0 + k;
    if constexpr (AK == kAGather) {
      // compressed entry j = k0 + k: mask word j / per (per = 32 n / m kept
      // entries per word, a power of two), its (j mod per)-th set bit, read
      // from the byte table or found in the mask word
      const int lper = __builtin_ctz((unsigned)(32 / p.m * p.n));
      const int64_t wd = row >> lper;
      const int pos = table ? (int)((pair >> (8 * i)) & 0xffu)
                            : select_bit(mrow[wd], (int)(row & ((1 << lper) - 1)));
      row = 32 * wd + pos;
      if (row > p.d_in - 1) row = p.d_in - 1;
    }
    load_to_lds16(p.wt + row * p.d_out + n, Bs + kb * PBN);
  }
}

// Four consecutive k (kq .. kq+3, plus 8 for lanes 32..63) of this lane's
// column of the 32-column block starting at c0, by one transpose read.
__device__ __forceinline__ s4v b_quad(const uint16_t* Bs, int kq, int c0) {
  const int lane = lane_id();
  const int g = lane / 16, i = lane % 16;
  const int k = kq + 8 * (g >> 1) + (i >> 2);
  const int n = c0 + 16 * (g & 1) + 4 * (i & 3);
  const uint16_t* ptr = Bs + k * PBN + 8 * ((n / 8) ^ swz_b(k)) + 4 * ((n / 4) & 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(SA_LDS4(ptr));
}

// Sparse MFMA position code of 16 mask bits: per group of 4, the first kept
// position | the second << 2 (as the staged-register engine forms it).
__device__ __forceinline__ int code_of(uint32_t bits) {
  uint32_t code = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t nib = (bits >> (4 * g)) & 0xfu;
    const uint32_t p0 = nib ? (uint32_t)__builtin_ctz(nib) : 0u;
    const uint32_t rest = nib & (nib - 1u);
    const uint32_t p1 = rest ? (uint32_t)__builtin_ctz(rest) : (p0 == 3u ? 3u : p0 + 1u);
    code |= (p0 | (p1 << 2)) << (4 * g);
  }
  return (int)code;
}

template <int AK, int BM>
__device__ __forceinline__ void pipe_compute(const uint16_t* S, const uint8_t* code_lut,
                                             f16v (&acc)[Pipe<AK, BM>::kMB][2], int wm, int wn) {
  const int lane = lane_id();
  constexpr int BK = Pipe<AK, BM>::kBK;
  constexpr int MB = Pipe<AK, BM>::kMB;
  const uint16_t* As = S;
  const uint16_t* Bs = S + Pipe<AK, BM>::kAHalves;
  if constexpr (AK == kADense || AK == kAGather) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      h8 aop[MB], bop[2];
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const int m = wm * (BM / 2) + 32 * a + lane % 32;
        const int q = 2 * kk + lane / 32;
        aop[a] = *reinterpret_cast<const h8*>(As + m * BK + 8 * (q ^ swz_a(m)));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int c0 = wn * 64 + 32 * b;
        const s4v q0 = b_quad(Bs, kk * 16, c0), q1 = b_quad(Bs, kk * 16 + 4, c0);
        typedef short s8v __attribute__((ext_vector_type(8)));
        const s8v both = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        bop[b] = __builtin_bit_cast(h8, both);
      }
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[a], bop[b], acc[a][b], 0, 0, 0);
    }
  } else {
    const uint32_t* Ms = reinterpret_cast<const uint32_t*>(Bs + BK * PBN);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      h8 aop[MB];
      int code[MB];
      h16 bop[2];
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const int m = wm * (BM / 2) + 32 * a + lane % 32;
        const int q = 2 * kk + lane / 32;
        aop[a] = *reinterpret_cast<const h8*>(As + m * (BK / 2) + 8 * (q ^ swz_a(m)));
        // position code of this lane's 16 mask bits, a byte at a time
        const uint32_t bits = Ms[m * 2 + kk] >> (16 * (lane / 32));
        code[a] = (int)code_lut[bits & 0xffu] | ((int)code_lut[(bits >> 8) & 0xffu] << 8);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int c0 = wn * 64 + 32 * b;
        const s4v q0 = b_quad(Bs, kk * 32, c0), q1 = b_quad(Bs, kk * 32 + 4, c0);
        const s4v q2 = b_quad(Bs, kk * 32 + 16, c0), q3 = b_quad(Bs, kk * 32 + 20, c0);
        typedef short s16v __attribute__((ext_vector_type(16)));
        const s16v all = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3],
                          q2[0], q2[1], q2[2], q2[3], q3[0], q3[1], q3[2], q3[3]};
        bop[b] = __builtin_bit_cast(h16, all);
      }
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] =
              __builtin_amdgcn_smfmac_f32_32x32x32_f16(aop[a], bop[b], acc[a][b], code[a], 0, 0);
    }
  }
}

// Stage wait with a run-time count: all but min(n, N) later stages' loads
// landed (n is uniform, so the choice is a scalar branch).
template <int LPW, int N>
__device__ __forceinline__ void stage_barrier_upto(int n) {
  if constexpr (N == 0) {
    stage_barrier<0>();
  } else {
    if (n >= N)
      stage_barrier<N * LPW>();
    else
      stage_barrier_upto<LPW, N - 1>(n);
  }
}

// The whole K loop over NS stages, loads NS - 1 steps ahead.  Step t waits
// for its own stage (t % NS), refills stage (t - 1) % NS -- read by step t - 1,
// which every wave finished before the barrier -- with step t + NS - 1, and
// computes (the gather kind computes first, then refills).  The main loop runs while every refill exists, with no branch
// inside; the last steps (fewer than 2 NS - 1) run in the tail, each waiting
// for exactly the later loads that exist.
template <int AK, int BM, int NS>
__device__ __forceinline__ void pipe_k_loop(const GParams& p, int64_t m0, int64_t n0, uint16_t* S,
                                            const uint8_t* code_lut, const uint32_t* mrow,
                                            f16v (&acc)[Pipe<AK, BM>::kMB][2], int wm, int wn) {
  constexpr int LPW = Pipe<AK, BM>::kLoadsPerWave;
  constexpr int BK = Pipe<AK, BM>::kBK;
  constexpr int SH = pipe_stage_halves<AK, BM>();
  constexpr int D = NS - 1;  // prefetch distance in steps
  static_assert(NS >= 3 && (D - 1) * LPW < 64, "stage count / vmcnt range");
  const int64_t nk = (AK == kAGather ? p.d_in / p.m * p.n : p.d_in) / BK;
  // gather: the B rows need a table lookup before their loads; issued after
  // the step's MFMAs, that latency overlaps them instead of delaying them
  constexpr bool kIssueLate = AK == kAGather;
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) pipe_issue<AK, BM>(p, m0, n0, j * BK, S + j * SH, mrow);
  int64_t kt = 0;
  for (; kt + NS + D - 1 < nk; kt += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      stage_barrier<(D - 1) * LPW>();
      if constexpr (kIssueLate) {
        pipe_compute<AK, BM>(S + j * SH, code_lut, acc, wm, wn);
        pipe_issue<AK, BM>(p, m0, n0, (kt + j + D) * BK, S + ((j + D) % NS) * SH, mrow);
      } else {
        pipe_issue<AK, BM>(p, m0, n0, (kt + j + D) * BK, S + ((j + D) % NS) * SH, mrow);
        pipe_compute<AK, BM>(S + j * SH, code_lut, acc, wm, wn);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NS + D - 1; ++j) {
    const int64_t t = kt + j;
    if (t < nk) {
      const int64_t later = nk - 1 - t;
      stage_barrier_upto<LPW, D - 1>(later < D - 1 ? (int)later : D - 1);
      if (!kIssueLate && t + D < nk)
        pipe_issue<AK, BM>(p, m0, n0, (t + D) * BK, S + ((j + D) % NS) * SH, mrow);
      pipe_compute<AK, BM>(S + (j % NS) * SH, code_lut, acc, wm, wn);
      if (kIssueLate && t + D < nk)
        pipe_issue<AK, BM>(p, m0, n0, (t + D) * BK, S + ((j + D) % NS) * SH, mrow);
    }
  }
}

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the
// 8 XCDs, so workgroup b runs on XCD b % 8; each XCD is given a contiguous
// run of a grouped tile order (kGroupM row tiles across all column tiles,
// row tile fastest), so the workgroups one XCD runs together share their A
// row tiles and B column tiles in its L2.  Any dispatch order gives the
// same results (the map is a bijection); this one only places the reuse.
constexpr int64_t kGroupM = 4;
__device__ __forceinline__ void pipe_tile(int64_t b, int64_t mt, int64_t ntl, int64_t& m,
                                          int64_t& n) {
  const int64_t G = mt * ntl;
  const int64_t x = b % 8, l = b / 8;
  const int64_t per = G / 8, rem = G % 8;
  const int64_t t = x * per + (x < rem ? x : rem) + l;  // position in the grouped order
  const int64_t gsz = kGroupM * ntl;
  const int64_t first = (t / gsz) * kGroupM;
  const int64_t gm = (mt - first < kGroupM) ? mt - first : kGroupM;
  m = first + (t % gsz) % gm;
  n = (t % gsz) / gm;
}

template <int AK, int BM, int NS>
__global__ __launch_bounds__(NTH, (pipe_wgs_per_cu<AK, BM, NS>())) void k_gemm_pipe(GParams p) {
  constexpr int MB = Pipe<AK, BM>::kMB;
  __shared__ __align__(16) uint16_t S[NS * pipe_stage_halves<AK, BM>()];
  const int lane = lane_id();
  const int wave = (int)threadIdx.x / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int64_t mt = (p.T + BM - 1) / BM;
  const int64_t ntl = (p.d_out + PBN - 1) / PBN;
  int64_t mi, ni;
  pipe_tile(blockIdx.x, mt, ntl, mi, ni);
  const int64_t m0 = mi * BM, n0 = ni * PBN;

  f16v acc[MB][2];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // 2:4: position code of every mask byte (two groups of 4), built once;
  // the first stage barrier orders these writes before any read
  __shared__ uint8_t code_lut[AK == kA24 ? 256 : 1];
  if constexpr (AK == kA24) code_lut[threadIdx.x] = (uint8_t)code_of(threadIdx.x);
  // gather: the row tile's pattern (one for all its rows), read by every B
  // load of the K loop: the byte table of kept positions, built here one
  // mask word per thread (a word holds per = 32 n / m kept entries, at a
  // fixed offset of the table), or the mask row itself
  __shared__ uint32_t mrow[AK == kAGather ? kGatherMaskWords : 1];
  if constexpr (AK == kAGather) {
    const int64_t wpr = p.d_in / 32;
    const uint32_t* src = p.mask + (m0 / p.tt) * wpr;
    if (p.d_in / p.m * p.n <= kGatherTableBytes) {
      // entry j at byte (j & ~7) | (j & 3) << 1 | (j >> 2) & 1: the entries
      // j and j + 4 that one lane loads in a step sit side by side
      const int per = 32 / p.m * p.n;
      uint8_t* tab = reinterpret_cast<uint8_t*>(mrow);
      for (int64_t i = threadIdx.x; i < wpr; i += NTH) {
        uint32_t bits = src[i];
        for (int e = 0; e < per; ++e) {
          const int64_t j = i * per + e;
          tab[(j & ~7) | ((j & 3) << 1) | ((j >> 2) & 1)] =
              (uint8_t)(bits ? __builtin_ctz(bits) : 31);
          bits &= bits - 1u;
        }
      }
    } else {
      for (int64_t i = threadIdx.x; i < wpr; i += NTH) mrow[i] = src[i];
    }
    __syncthreads();
  }
  pipe_k_loop<AK, BM, NS>(p, m0, n0, S, code_lut, mrow, acc, wm, wn);

#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row < p.T && col < p.d_out) p.y[row * p.d_out + col] = f2h(acc[a][b][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Wide dense engine (k_gemm_wide): 256 x 256 output tiles, eight waves of the
// pipelined engine's 128 x 64 wave tile, K steps of 32 through NS stages of
// 32 KB (A [256][32] and B [32][256], swizzled as in k_gemm_pipe; one
// workgroup per CU).  A K step moves 32 KB into LDS for 4.2 MFLOP where the
// 256 x 128 tile moves 24 KB for 2.1 MFLOP, so the load path -- what bounds
// the pipelined engine -- carries a third less per FLOP, and the eight waves
// on a CU share one set of barriers.  Every output block gets the same MFMA
// sequence as in the other engines: identical results.
// ---------------------------------------------------------------------------
constexpr int WBM = 256, WBN = 256, WNT = 512;
constexpr int kWideAHalves = WBM * BK;
constexpr int kWideStageHalves = kWideAHalves + BK * WBN;
constexpr int kWideLoadsPerWave = 4;  // two A and two B instructions of 1 KB
constexpr int kWideMaxStages = 160 * 1024 / (2 * kWideStageHalves);
static_assert(kWideMaxStages >= 3, "three wide stages must fit the LDS");

// This wave's share of one K step's loads: A as 16 rows of 64 bytes and B as
// 2 k rows of 512 bytes per instruction.  Rows past T and columns past d_out
// read clamped (valid) addresses; their results are never stored.
__device__ __forceinline__ void wide_issue(const GParams& p, int64_t m0, int64_t n0, int64_t k0,
                                           uint16_t* S) {
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  uint16_t* As = S;
  uint16_t* Bs = S + kWideAHalves;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rb = (w * 2 + i) * 16;
    const int r = rb + lane / 4;
    const int gc = (lane % 4) ^ swz_a(r);
    int64_t row = m0 + r;
    if (row >= p.T) row = p.T - 1;
    load_to_lds16(p.x + row * p.d_in + k0 + 8 * gc, As + rb * BK);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kb = (w * 2 + i) * 2;
    const int k = kb + lane / 32;
    const int gc = (lane % 32) ^ swz_b(k);
    int64_t n = n0 + 8 * gc;
    if (n >= p.d_out) n = p.d_out - 8;
    load_to_lds16(p.wt + (k0 + k) * p.d_out + n, Bs + kb * WBN);
  }
}

// b_quad on 256-column B rows.
__device__ __forceinline__ s4v wide_b_quad(const uint16_t* Bs, int kq, int c0) {
  const int lane = lane_id();
  const int g = lane / 16, i = lane % 16;
  const int k = kq + 8 * (g >> 1) + (i >> 2);
  const int n = c0 + 16 * (g & 1) + 4 * (i & 3);
  const uint16_t* ptr = Bs + k * WBN + 8 * ((n / 8) ^ swz_b(k)) + 4 * ((n / 4) & 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(SA_LDS4(ptr));
}

// One K step of a wave's 128 x 64 tile (pipe_compute's dense branch).
__device__ __forceinline__ void wide_compute(const uint16_t* S, f16v (&acc)[4][2], int wm,
                                             int wn) {
  const int lane = lane_id();
  const uint16_t* As = S;
  const uint16_t* Bs = S + kWideAHalves;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    h8 aop[4], bop[2];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int m = wm * 128 + 32 * a + lane % 32;
      const int q = 2 * kk + lane / 32;
      aop[a] = *reinterpret_cast<const h8*>(As + m * BK + 8 * (q ^ swz_a(m)));
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int c0 = wn * 64 + 32 * b;
      const s4v q0 = wide_b_quad(Bs, kk * 16, c0), q1 = wide_b_quad(Bs, kk * 16 + 4, c0);
      typedef short s8v __attribute__((ext_vector_type(8)));
      const s8v both = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
      bop[b] = __builtin_bit_cast(h8, both);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[a], bop[b], acc[a][b], 0, 0, 0);
  }
}

template <int NS>
__global__ __launch_bounds__(WNT, 1) void k_gemm_wide(GParams p) {
  static_assert(NS >= 3 && NS <= kWideMaxStages, "wide stage count");
  __shared__ __align__(16) uint16_t S[NS * kWideStageHalves];
  const int lane = lane_id();
  const int wave = (int)threadIdx.x / kWave;
  const int wm = wave / 4, wn = wave % 4;
  const int64_t mt = (p.T + WBM - 1) / WBM;
  const int64_t ntl = (p.d_out + WBN - 1) / WBN;
  int64_t mi, ni;
  pipe_tile(blockIdx.x, mt, ntl, mi, ni);
  const int64_t m0 = mi * WBM, n0 = ni * WBN;
  f16v acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // the pipelined engine's K loop: loads D = NS - 1 steps ahead, a stage
  // refilled only after the barrier that follows every wave's reads of it
  constexpr int D = NS - 1;
  const int64_t nk = p.d_in / BK;
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) wide_issue(p, m0, n0, j * BK, S + j * kWideStageHalves);
  int64_t kt = 0;
  for (; kt + NS + D - 1 < nk; kt += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      stage_barrier<(D - 1) * kWideLoadsPerWave>();
      wide_issue(p, m0, n0, (kt + j + D) * BK, S + ((j + D) % NS) * kWideStageHalves);
      wide_compute(S + j * kWideStageHalves, acc, wm, wn);
    }
  }
#pragma unroll
  for (int j = 0; j < NS + D - 1; ++j) {
    const int64_t t = kt + j;
    if (t < nk) {
      const int64_t later = nk - 1 - t;
      stage_barrier_upto<kWideLoadsPerWave, D - 1>(later < D - 1 ? (int)later : D - 1);
      if (t + D < nk)
        wide_issue(p, m0, n0, (t + D) * BK, S + ((j + D) % NS) * kWideStageHalves);
      wide_compute(S + (j % NS) * kWideStageHalves, acc, wm, wn);
    }
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row < p.T && col < p.d_out) p.y[row * p.d_out + col] = f2h(acc[a][b][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Wide 2:4 engine (k_gemm_wide24): the wide engine's 256 x 256 tiles and
// eight 128 x 64 wave tiles on the sparse MFMA.  A K step covers 64 dense k:
// A holds 32 compressed values per row ([256][32], 64-byte rows swizzled as
// the dense A) and the row's two mask words ([256][2]); B holds 64 k rows of
// 256 columns ([64][256], as the wide B).  A stage is 50 KB, three fit the
// LDS (one workgroup per CU).  Per 64 dense k a 128 x 128 2:4 tile stages
// 25 KB for 1.05 MFLOP of sparse MFMA work and a wide tile 50 KB for 4.2, so
// the load path carries half as much per FLOP.  The MFMA sequence per output
// block is the pipelined 2:4 engine's: identical results.
// ---------------------------------------------------------------------------
constexpr int kW24BK = 64;
constexpr int kW24AHalves = WBM * kW24BK / 2;   // [256][32] compressed
constexpr int kW24MaskWords = WBM * 2;          // [256][2]
constexpr int kW24StageHalves = kW24AHalves + kW24BK * WBN + 2 * kW24MaskWords;
constexpr int kW24LoadsPerWave = 7;  // two A, four B, one mask instruction
constexpr int kW24Stages = 3;
static_assert(kW24Stages * kW24StageHalves * 2 + 256 <= 160 * 1024, "wide 2:4 stages fit the LDS");

__device__ __forceinline__ void wide24_issue(const GParams& p, int64_t m0, int64_t n0, int64_t k0,
                                             uint16_t* S) {
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  uint16_t* As = S;
  uint16_t* Bs = S + kW24AHalves;
  uint32_t* Ms = reinterpret_cast<uint32_t*>(Bs + kW24BK * WBN);
  const int64_t kc = p.d_in / 2;  // compressed row length
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rb = (w * 2 + i) * 16;  // 16 rows of 64 bytes per instruction
    const int r = rb + lane / 4;
    const int gc = (lane % 4) ^ swz_a(r);
    int64_t row = m0 + r;
    if (row >= p.T) row = p.T - 1;
    load_to_lds16(p.x + row * kc + k0 / 2 + 8 * gc, As + rb * (kW24BK / 2));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kb = (w * 4 + i) * 2;  // 2 k rows of 512 bytes per instruction
    const int k = kb + lane / 32;
    const int gc = (lane % 32) ^ swz_b(k);
    int64_t n = n0 + 8 * gc;
    if (n >= p.d_out) n = p.d_out - 8;
    load_to_lds16(p.wt + (k0 + k) * p.d_out + n, Bs + kb * WBN);
  }
  {
    const int rb = w * 32;  // 32 rows of 2 words per instruction
    const int r = rb + lane / 2;
    int64_t row = m0 + r;
    if (row >= p.T) row = p.T - 1;
    load_to_lds4(p.mask + row * (p.d_in / 32) + k0 / 32 + (lane % 2), Ms + rb * 2);
  }
}

// One K step of a wave's 128 x 64 tile (pipe_compute's 2:4 branch).
__device__ __forceinline__ void wide24_compute(const uint16_t* S, const uint8_t* code_lut,
                                               f16v (&acc)[4][2], int wm, int wn) {
  const int lane = lane_id();
  const uint16_t* As = S;
  const uint16_t* Bs = S + kW24AHalves;
  const uint32_t* Ms = reinterpret_cast<const uint32_t*>(Bs + kW24BK * WBN);
#pragma unroll
  for (int kk = 0; kk < kW24BK / 32; ++kk) {
    h8 aop[4];
    int code[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int m = wm * 128 + 32 * a + lane % 32;
      const int q = 2 * kk + lane / 32;
      aop[a] = *reinterpret_cast<const h8*>(As + m * (kW24BK / 2) + 8 * (q ^ swz_a(m)));
      const uint32_t bits = Ms[m * 2 + kk] >> (16 * (lane / 32));
      code[a] = (int)code_lut[bits & 0xffu] | ((int)code_lut[(bits >> 8) & 0xffu] << 8);
    }
    // one column block at a time: a single 16-value B operand is live
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int c0 = wn * 64 + 32 * b;
      const s4v q0 = wide_b_quad(Bs, kk * 32, c0), q1 = wide_b_quad(Bs, kk * 32 + 4, c0);
      const s4v q2 = wide_b_quad(Bs, kk * 32 + 16, c0), q3 = wide_b_quad(Bs, kk * 32 + 20, c0);
      typedef short s16v __attribute__((ext_vector_type(16)));
      const s16v all = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3],
                        q2[0], q2[1], q2[2], q2[3], q3[0], q3[1], q3[2], q3[3]};
      const h16 bop = __builtin_bit_cast(h16, all);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        acc[a][b] =
            __builtin_amdgcn_smfmac_f32_32x32x32_f16(aop[a], bop, acc[a][b], code[a], 0, 0);
    }
  }
}

__global__ __launch_bounds__(WNT, 1) void k_gemm_wide24(GParams p) {
  constexpr int NS = kW24Stages;
  __shared__ __align__(16) uint16_t S[NS * kW24StageHalves];
  __shared__ uint8_t code_lut[256];
  const int lane = lane_id();
  const int wave = (int)threadIdx.x / kWave;
  const int wm = wave / 4, wn = wave % 4;
  const int64_t mt = (p.T + WBM - 1) / WBM;
  const int64_t ntl = (p.d_out + WBN - 1) / WBN;
  int64_t mi, ni;
  pipe_tile(blockIdx.x, mt, ntl, mi, ni);
  const int64_t m0 = mi * WBM, n0 = ni * WBN;
  f16v acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  // position code of every mask byte; the first stage barrier orders these
  // writes before any read
  if (threadIdx.x < 256) code_lut[threadIdx.x] = (uint8_t)code_of(threadIdx.x);

  constexpr int D = NS - 1;
  const int64_t nk = p.d_in / kW24BK;
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) wide24_issue(p, m0, n0, j * kW24BK, S + j * kW24StageHalves);
  int64_t kt = 0;
  for (; kt + NS + D - 1 < nk; kt += NS) {
    // stages rolled, not unrolled: one set of LDS addresses stays live
#pragma unroll 1
    for (int j = 0; j < NS; ++j) {
      stage_barrier<(D - 1) * kW24LoadsPerWave>();
      wide24_issue(p, m0, n0, (kt + j + D) * kW24BK, S + ((j + D) % NS) * kW24StageHalves);
      wide24_compute(S + j * kW24StageHalves, code_lut, acc, wm, wn);
    }
  }
#pragma unroll
  for (int j = 0; j < NS + D - 1; ++j) {
    const int64_t t = kt + j;
    if (t < nk) {
      const int64_t later = nk - 1 - t;
      stage_barrier_upto<kW24LoadsPerWave, D - 1>(later < D - 1 ? (int)later : D - 1);
      if (t + D < nk)
        wide24_issue(p, m0, n0, (t + D) * kW24BK, S + ((j + D) % NS) * kW24StageHalves);
      wide24_compute(S + (j % NS) * kW24StageHalves, code_lut, acc, wm, wn);
    }
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row < p.T && col < p.d_out) p.y[row * p.d_out + col] = f2h(acc[a][b][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Tile-shared N:M on 32-row tiles (k_gemm_g32): the whole-tile gather for
// tiles of tt rows with tt a multiple of 32 (VW32 is tt = 32).  A 256-thread
// workgroup computes a 32 x 128 output tile, one 32-row block of one pattern:
// each wave one 32 x 32 block (wave w: columns 32 w .. 32 w + 31).  The K
// loop runs over the d_in n / m compressed entries in steps of 32 through NS
// stages of 10 KB: A [32][32] (the compressed values, rows swizzled as the
// dense A) and B [32][128], the kept WT rows of the pattern only (as in the
// whole-tile gather), so B bytes fall to n / m of dense.  Small stages let
// five workgroups share a CU, whose loads cover each other's latency.
//   Loads per step: A is 2 KB, one instruction each for waves 0 and 1; B is
//   two instructions per wave.  A wave's stage wait counts its own loads.
// The MFMA sequence per output block is the whole-tile gather's (compressed
// k in order, 16 per MFMA): identical results.
// ---------------------------------------------------------------------------
constexpr int kG32BK = 32;
constexpr int kG32AHalves = 32 * kG32BK;  // [32][32]
constexpr int kG32GroupM = 16;  // row tiles grouped across the column tiles (L2 reuse of B)
// Per tile width BN (128 or 256 columns): stage size and B loads per wave
// and step (1 KB instructions of 4 rows of 256 bytes, or 2 rows of 512).
template <int BN>
struct G32 {
  static_assert(BN == 128 || BN == 256, "tile width");
  static constexpr int kStageHalves = kG32AHalves + kG32BK * BN;
  static constexpr int kBLoads = kG32BK * BN * 2 / 1024 / 4;
  static constexpr int kBlocks = BN / 128;  // 32 x 32 blocks per wave
};

// Pattern table entry of compressed entry j.  At 128 columns a lane loads
// entries j and j + 4 of a step, stored side by side; at 256 columns the
// table is in entry order.
template <int BN>
__device__ __forceinline__ int g32_slot(int64_t j) {
  if constexpr (BN == 128)
    return (int)((j & ~7) | ((j & 3) << 1) | ((j >> 2) & 1));
  else
    return (int)j;
}

template <int BN>
__device__ __forceinline__ void g32_issue(const GParams& p, int64_t m0, int64_t n0, int64_t k0,
                                          uint16_t* S, const uint32_t* mrow, bool table) {
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  uint16_t* As = S;
  uint16_t* Bs = S + kG32AHalves;
  const uint8_t* tab = reinterpret_cast<const uint8_t*>(mrow);
  // this lane's B rows of the step, read from the table before the A load
  // so that their latency overlaps it
  constexpr int BL = G32<BN>::kBLoads;
  int pos[BL];
  if constexpr (BN == 128) {
    // entries k0 + 8 w + lane / 16 and + 4: one 16-bit read
    const uint32_t pair =
        table ? *reinterpret_cast<const uint16_t*>(tab + k0 + 8 * w + 2 * (lane / 16)) : 0u;
    pos[0] = (int)(pair & 0xffu);
    pos[1] = (int)(pair >> 8);
  } else {
#pragma unroll
    for (int i = 0; i < BL; ++i) pos[i] = table ? (int)tab[k0 + (w * BL + i) * 2 + lane / 32] : 0;
  }
  const int64_t lda = p.d_in / p.m * p.n;
  if (w < 2) {
    const int rb = w * 16;  // 16 rows of 64 bytes
    const int r = rb + lane / 4;
    const int gc = (lane % 4) ^ swz_a(r);
    int64_t row = m0 + r;
    if (row >= p.T) row = p.T - 1;
    load_to_lds16(p.x + row * lda + k0 + 8 * gc, As + rb * kG32BK);
  }
  const int lper = __builtin_ctz((unsigned)(32 / p.m * p.n));
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    constexpr int RPI = 1024 / (2 * BN);  // k rows per instruction
    constexpr int CPR = BN / 8;           // 16-byte chunks per row
    const int kb = (w * BL + i) * RPI;
    const int k = kb + lane / CPR;
    const int gc = (lane % CPR) ^ swz_b(k);
    int64_t n = n0 + 8 * gc;
    if (n >= p.d_out) n = p.d_out - 8;
    const int64_t j = k0 + k;  // compressed entry
    const int64_t wd = j >> lper;
    const int ps = table ? pos[i] : select_bit(mrow[wd], (int)(j & ((1 << lper) - 1)));
    int64_t row = 32 * wd + ps;
    if (row > p.d_in - 1) row = p.d_in - 1;
    load_to_lds16(p.wt + row * p.d_out + n, Bs + kb * BN);
  }
}

template <int BN>
__device__ __forceinline__ void g32_compute(const uint16_t* S, f16v (&acc)[G32<BN>::kBlocks],
                                            int w) {
  const int lane = lane_id();
  const uint16_t* As = S;
  const uint16_t* Bs = S + kG32AHalves;
#pragma unroll
  for (int kk = 0; kk < kG32BK / 16; ++kk) {
    const int m = lane % 32;
    const int q = 2 * kk + lane / 32;
    const h8 aop = *reinterpret_cast<const h8*>(As + m * kG32BK + 8 * (q ^ swz_a(m)));
#pragma unroll
    for (int b = 0; b < G32<BN>::kBlocks; ++b) {
      const int c0 = w * (BN / 4) + 32 * b;
      s4v q0, q1;
      if constexpr (BN == 128) {
        q0 = b_quad(Bs, kk * 16, c0);
        q1 = b_quad(Bs, kk * 16 + 4, c0);
      } else {
        q0 = wide_b_quad(Bs, kk * 16, c0);
        q1 = wide_b_quad(Bs, kk * 16 + 4, c0);
      }
      typedef short s8v __attribute__((ext_vector_type(8)));
      const s8v both = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
      acc[b] =
          __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, __builtin_bit_cast(h8, both), acc[b], 0, 0, 0);
    }
  }
}

// Stage wait of wave w: waves 0 and 1 also load A, one more load per step.
template <int BL, int LATER>
__device__ __forceinline__ void g32_barrier(int w) {
  if (w < 2)
    stage_barrier<LATER * (BL + 1)>();
  else
    stage_barrier<LATER * BL>();
}
template <int BL>
__device__ __forceinline__ void g32_barrier_upto(int w, int later) {
  if (later >= 2)
    g32_barrier<BL, 2>(w);
  else if (later == 1)
    g32_barrier<BL, 1>(w);
  else
    g32_barrier<BL, 0>(w);
}

// TB: bytes of the pattern table, sized to the call (512, 2048 or 4096
// kept entries) so that more workgroups fit a CU; at 4096 the table also
// holds the mask row for longer patterns.
template <int NS, int TB, int BN>
__global__ __launch_bounds__(NTH) void k_gemm_g32(GParams p) {
  static_assert(NS == 3 || NS == 4, "the waits cover a prefetch distance of 2 or 3 steps");
  static_assert(TB % 4 == 0 && TB <= kGatherTableBytes, "table size");
  constexpr int D = NS - 1;
  constexpr int SH = G32<BN>::kStageHalves;
  constexpr int NB = G32<BN>::kBlocks;
  __shared__ __align__(16) uint16_t S[NS * SH];
  __shared__ uint32_t mrow[TB / 4];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int64_t mt = (p.T + 31) / 32;
  const int64_t ntl = (p.d_out + BN - 1) / BN;
  // grouped order, kG32GroupM row tiles across all column tiles, row tile
  // fastest; each XCD takes a contiguous run of it (as pipe_tile)
  int64_t mi, ni;
  {
    const int64_t b = blockIdx.x;
    const int64_t G = mt * ntl;
    const int64_t x = b % 8, l = b / 8;
    const int64_t per = G / 8, rem = G % 8;
    const int64_t t = x * per + (x < rem ? x : rem) + l;
    const int64_t gsz = kG32GroupM * ntl;
    const int64_t first = (t / gsz) * kG32GroupM;
    const int64_t gm = (mt - first < kG32GroupM) ? mt - first : kG32GroupM;
    mi = first + (t % gsz) % gm;
    ni = (t % gsz) / gm;
  }
  const int64_t m0 = mi * 32, n0 = ni * BN;
  // the tile's pattern: the byte table of kept positions (as k_gemm_pipe's
  // gather) or the mask row itself
  const int64_t wpr = p.d_in / 32;
  const uint32_t* src = p.mask + (m0 / p.tt) * wpr;
  const bool table = p.d_in / p.m * p.n <= TB;  // else TB = 4096: the mask row (<= 1024 words)
  if (table) {
    const int per = 32 / p.m * p.n;
    uint8_t* tab = reinterpret_cast<uint8_t*>(mrow);
    for (int64_t i = threadIdx.x; i < wpr; i += NTH) {
      uint32_t bits = src[i];
      for (int e = 0; e < per; ++e) {
        tab[g32_slot<BN>(i * per + e)] = (uint8_t)(bits ? __builtin_ctz(bits) : 31);
        bits &= bits - 1u;
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < wpr; i += NTH) mrow[i] = src[i];
  }
  __syncthreads();

  f16v acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  const int nk = (int)(p.d_in / p.m * p.n / kG32BK);
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) g32_issue<BN>(p, m0, n0, j * kG32BK, S + j * SH, mrow, table);
  for (int t = 0; t < nk; ++t) {
    // wait for step t's loads, leaving the later steps' in flight (at most
    // D - 1 of them), then refill the stage step t - 1 used
    const int later = nk - 1 - t;
    g32_barrier_upto<G32<BN>::kBLoads>(w, later < D - 1 ? later : D - 1);
    if (t + D < nk)
      g32_issue<BN>(p, m0, n0, (int64_t)(t + D) * kG32BK, S + ((t + D) % NS) * SH, mrow, table);
    g32_compute<BN>(S + (t % NS) * SH, acc, w);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t col = n0 + w * (BN / 4) + 32 * b + lane % 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
      if (row < p.T && col < p.d_out) p.y[row * p.d_out + col] = f2h(acc[b][r]);
    }
  }
}

// ---------------------------------------------------------------------------
// Tile-shared N:M engine.  Every 32-row block of tokens lies in one tile of
// tt rows (tt a multiple of 32), so its rows share one N:M pattern; over one
// K step the block's product is a dense MFMA product of the compressed values
// (32 per row per step) with the kept rows of WT.  A K step covers KB =
// 32 m / n dense rows of WT, staged whole as the dense engine stages B, and
// 32 compressed values of each A row.  The gather costs no extra LDS reads:
// the MFMA B operand comes from transpose reads in which every source lane
// addresses its own row, so a lane points at the kept row of its k slot
// rather than at the slot's own row.  Per K step each wave turns its row
// blocks' mask words into a table of kept-row offsets, one lane per kept
// slot (the r-th set bit of its group), stored so that the four offsets a
// lane reads in a step share one 32-bit word.
//   Stage: A [BM][32] (64-byte rows, swizzled as the dense A), B [KB][128]
//   (as the dense B), and one 64-word mask area per wave (lane l of wave w
//   loads word l % (KB/32) of its row block l / (KB/32)).
// Only the MFMA work shrinks (to n/m of dense): every step still stages the
// whole WT slab, and B operands are read per 32-row block (no reuse across
// the blocks of a wave), so the engine pays off where MFMAs, not loads, bound
// the dense product.
// ---------------------------------------------------------------------------
template <int KB, int BM>
struct Shared {
  static constexpr int kMB = BM / 64;               // 32-row blocks per wave
  static constexpr int kAHalves = BM * 32;
  static constexpr int kBHalves = KB * PBN;
  static constexpr int kMaskWords = 4 * 64;         // one 64-word area per wave
  static constexpr int kStageHalves = kAHalves + kBHalves + 2 * kMaskWords;
  static constexpr int kLoadsPerWave = BM / 64 + KB / 16 + 1;
  static constexpr int kStages = 3;
  static constexpr int kLdsBytes = kStages * kStageHalves * 2 + 4 * kMB * 32;
  static constexpr int kWgsPerCu = (160 * 1024 / kLdsBytes) < 2 ? (160 * 1024 / kLdsBytes) : 2;
  static_assert(kWgsPerCu >= 1, "stages exceed the LDS");
};

template <int KB, int BM>
__device__ __forceinline__ void shared_issue(const GParams& p, int64_t m0, int64_t n0,
                                             int64_t step, uint16_t* S) {
  using C = Shared<KB, BM>;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  uint16_t* As = S;
  uint16_t* Bs = S + C::kAHalves;
  uint32_t* Ms = reinterpret_cast<uint32_t*>(Bs + C::kBHalves) + 64 * w;
  const int64_t kc = p.d_in / KB * 32;  // compressed row length
  constexpr int AI = BM / 64;
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int rb = (w * AI + i) * 16;  // 16 rows of 64 bytes per instruction
    const int r = rb + lane / 4;
    const int gc = (lane % 4) ^ swz_a(r);
    int64_t row = m0 + r;
    if (row >= p.T) row = p.T - 1;
    load_to_lds16(p.x + row * kc + step * 32 + 8 * gc, As + rb * 32);
  }
#pragma unroll
  for (int i = 0; i < KB / 16; ++i) {
    const int kb = (w * (KB / 16) + i) * 4;  // 4 k rows of 256 bytes per instruction
    const int k = kb + lane / 16;
    const int gc = (lane % 16) ^ swz_b(k);
    int64_t n = n0 + 8 * gc;
    if (n >= p.d_out) n = p.d_out - 8;
    load_to_lds16(p.wt + (step * KB + k) * p.d_out + n, Bs + kb * PBN);
  }
  constexpr int W = KB / 32;  // mask words per row block per step
  int bl = lane / W;
  if (bl >= C::kMB) bl = C::kMB - 1;  // spare lanes repeat a valid word
  int64_t row = m0 + (w / 2) * (BM / 2) + 32 * bl;
  if (row >= p.T) row = p.T - 1;
  const int64_t words = p.d_in / 32;
  load_to_lds4(p.mask + (row / p.tt) * words + step * W + lane % W, Ms);
}

// This wave's kept-row offsets for the step: lane -> (block a, slot j).
// Slot j = 16 kk + 8 h + 4 q + r (MFMA kk, lane half h, quad q, row r of
// the quad) is stored at byte 4 (4 h + r) + 2 kk + q of the block's 32.
template <int KB, int BM>
__device__ __forceinline__ void shared_positions(const GParams& p, const uint32_t* Ms,
                                                 uint8_t* tab) {
  using C = Shared<KB, BM>;
  const int lane = lane_id();
  const int ln = __builtin_ctz((unsigned)p.n), lm = __builtin_ctz((unsigned)p.m);
  const uint32_t fmask = p.m == 32 ? 0xffffffffu : ((1u << p.m) - 1u);
#pragma unroll
  for (int a0 = 0; a0 < C::kMB; a0 += 2) {
    const int a = a0 + lane / 32, j = lane % 32;
    const int bit0 = (j >> ln) << lm;  // first dense row of the slot's group
    const uint32_t bits = (Ms[a * (KB / 32) + bit0 / 32] >> (bit0 % 32)) & fmask;
    int off = bit0 + select_bit(bits, j & (p.n - 1));
    if (off > KB - 1) off = KB - 1;
    const int kk = j >> 4, h = (j >> 3) & 1, q = (j >> 2) & 1, r = j & 3;
    tab[a * 32 + 4 * (4 * h + r) + 2 * kk + q] = (uint8_t)off;
  }
}

// Four halves of row k (this lane's own source row) for a transpose read.
__device__ __forceinline__ s4v b_quad_row(const uint16_t* Bs, int k, int c0) {
  const int lane = lane_id();
  const int g = lane / 16, i = lane % 16;
  const int n = c0 + 16 * (g & 1) + 4 * (i & 3);
  const uint16_t* ptr = Bs + k * PBN + 8 * ((n / 8) ^ swz_b(k)) + 4 * ((n / 4) & 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(SA_LDS4(ptr));
}

template <int KB, int BM>
__device__ __forceinline__ void shared_compute(const uint16_t* S, const uint8_t* tab,
                                               f16v (&acc)[Shared<KB, BM>::kMB][2], int wm,
                                               int wn) {
  using C = Shared<KB, BM>;
  constexpr int MB = C::kMB;
  const int lane = lane_id();
  const uint16_t* As = S;
  const uint16_t* Bs = S + C::kAHalves;
  uint32_t P[MB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
    P[a] = *reinterpret_cast<const uint32_t*>(tab + a * 32 + 4 * (4 * (lane / 32) + (lane % 16) / 4));
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    h8 aop[MB];
#pragma unroll
    for (int a = 0; a < MB; ++a) {
      const int m = wm * (BM / 2) + 32 * a + lane % 32;
      const int q = 2 * kk + lane / 32;
      aop[a] = *reinterpret_cast<const h8*>(As + m * 32 + 8 * (q ^ swz_a(m)));
    }
#pragma unroll
    for (int a = 0; a < MB; ++a) {
      const int r0 = (int)((P[a] >> (16 * kk)) & 0xffu), r1 = (int)((P[a] >> (16 * kk + 8)) & 0xffu);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int c0 = wn * 64 + 32 * b;
        const s4v q0 = b_quad_row(Bs, r0, c0), q1 = b_quad_row(Bs, r1, c0);
        typedef short s8v __attribute__((ext_vector_type(8)));
        const s8v both = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[a], __builtin_bit_cast(h8, both),
                                                           acc[a][b], 0, 0, 0);
      }
    }
  }
}

template <int KB, int BM>
__global__ __launch_bounds__(NTH, (Shared<KB, BM>::kWgsPerCu)) void k_gemm_shared(GParams p) {
  using C = Shared<KB, BM>;
  constexpr int MB = C::kMB;
  constexpr int SH = C::kStageHalves;
  constexpr int LPW = C::kLoadsPerWave;
  __shared__ __align__(16) uint16_t S[C::kStages * SH];
  __shared__ __align__(4) uint8_t tabs[4 * MB * 32];
  const int lane = lane_id();
  const int wave = (int)threadIdx.x / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int64_t mt = (p.T + BM - 1) / BM;
  const int64_t ntl = (p.d_out + PBN - 1) / PBN;
  int64_t mi, ni;
  pipe_tile(blockIdx.x, mt, ntl, mi, ni);
  const int64_t m0 = mi * BM, n0 = ni * PBN;
  uint8_t* tab = tabs + wave * MB * 32;

  f16v acc[MB][2];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Three stages, loads two steps ahead (the dense engine's loop).  After
  // each stage wait the wave builds its offset table from its own mask words
  // (its own loads, so the wait alone orders them), then computes.
  auto step = [&](int64_t t, int stage) {
    const uint16_t* St = S + stage * SH;
    shared_positions<KB, BM>(p, reinterpret_cast<const uint32_t*>(St + C::kAHalves + C::kBHalves) +
                                    64 * wave, tab);
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    shared_compute<KB, BM>(St, tab, acc, wm, wn);
    (void)t;
  };
  const int64_t nk = p.d_in / KB;
  shared_issue<KB, BM>(p, m0, n0, 0, S);
  if (nk > 1) shared_issue<KB, BM>(p, m0, n0, 1, S + SH);
  for (int64_t t = 0; t < nk; ++t) {
    const int stage = (int)(t % 3);
    if (t + 1 < nk)
      stage_barrier<LPW>();
    else
      stage_barrier<0>();
    if (t + 2 < nk) shared_issue<KB, BM>(p, m0, n0, t + 2, S + ((stage + 2) % 3) * SH);
    step(t, stage);
  }

#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row < p.T && col < p.d_out) p.y[row * p.d_out + col] = f2h(acc[a][b][r]);
      }
    }
}

template <int AK>
bool pipe_ok(const GParams& p) {
  return p.d_in % Pipe<AK, 256>::kBK == 0 && p.d_out % 8 == 0 && p.d_out >= 8 && p.T >= 1 &&
         (reinterpret_cast<uintptr_t>(p.x) & 15u) == 0 &&
         (reinterpret_cast<uintptr_t>(p.wt) & 15u) == 0 &&
         (reinterpret_cast<uintptr_t>(p.mask) & 3u) == 0;
}

// ---------------------------------------------------------------------------
// N:M patterns other than 2:4, two-pass path: the compressed values are
// expanded into a zero-filled dense [T][d_in] copy (the "gathered dense"
// operand written out once), then the pipelined dense engine runs on it.
// One thread per 32-entry mask word: a word holds exactly 32n/m kept values
// (m divides 32), at a fixed offset of the compressed array; they are
// scattered to their set bits in an LDS tile and the workgroup's run of the
// dense copy is written with 16-byte stores.  A mask word with more set bits
// than that places only the first 32n/m values (no read past its run).
// Token t reads mask row t / tt (tt = 1: per-token masks; tt > 1: one mask
// row per tile of tt tokens).
// ---------------------------------------------------------------------------
constexpr int kExpandThreads = 256;

template <int NV>  // 16-byte vectors of kept values per word (per = 8 NV); 0 = scalar loads
__global__ __launch_bounds__(kExpandThreads) void k_nm_expand(const uint16_t* __restrict__ xval,
                                                              const uint32_t* __restrict__ mask,
                                                              int64_t nwords, int64_t wpr,
                                                              int tt, int per,
                                                              uint16_t* __restrict__ xd) {
  __shared__ __align__(16) uint16_t tile[kExpandThreads * 32];
  const int tid = (int)threadIdx.x;
  const int64_t w0 = (int64_t)blockIdx.x * kExpandThreads;
  const int64_t w = w0 + tid;
  uint16_t* mine = tile + tid * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(mine + 8 * q) = u32x4{0u, 0u, 0u, 0u};
  if (w < nwords) {
    const int64_t t = w / wpr;
    uint32_t bits = mask[tt == 1 ? w : (t / tt) * wpr + (w - t * wpr)];
    const uint16_t* src = xval + w * per;
    if constexpr (NV > 0) {
      u32x4 v[NV];
#pragma unroll
      for (int q = 0; q < NV; ++q) v[q] = *reinterpret_cast<const u32x4*>(src + 8 * q);
#pragma unroll
      for (int r = 0; r < 8 * NV; ++r) {
        const uint32_t word = v[r / 8][(r % 8) / 2];  // static register index
        if (bits != 0u) {
          mine[__builtin_ctz(bits)] = (uint16_t)((r & 1) ? (word >> 16) : (word & 0xffffu));
          bits &= bits - 1u;
        }
      }
    } else {
      for (int r = 0; r < per && bits != 0u; ++r) {
        mine[__builtin_ctz(bits)] = src[r];
        bits &= bits - 1u;
      }
    }
  }
  __syncthreads();
  const int64_t left = nwords - w0;
  const int nthr = left < kExpandThreads ? (int)left : kExpandThreads;
  uint16_t* dst = xd + w0 * 32;
  for (int i = tid; i < nthr * 4; i += kExpandThreads)
    *reinterpret_cast<u32x4*>(dst + 8 * i) = *reinterpret_cast<const u32x4*>(tile + 8 * i);
}

hipError_t launch_nm_expand(const uint16_t* xval, const uint32_t* mask, int64_t T, int64_t d_in,
                            int n, int m, int tt, uint16_t* xd, hipStream_t s) {
  const int64_t wpr = d_in / 32;
  const int64_t nwords = T * wpr;
  const int per = 32 * n / m;
  const int64_t blocks = (nwords + kExpandThreads - 1) / kExpandThreads;
  if (blocks > 0x7fffffffLL) return hipErrorNotSupported;
  const dim3 grid((unsigned)blocks), block(kExpandThreads);
#define SA_EXPAND(NV) \
  hipLaunchKernelGGL(k_nm_expand<NV>, grid, block, 0, s, xval, mask, nwords, wpr, tt, per, xd)
  switch (per % 8 == 0 ? per / 8 : 0) {
    case 1: SA_EXPAND(1); break;
    case 2: SA_EXPAND(2); break;
    case 3: SA_EXPAND(3); break;
    case 4: SA_EXPAND(4); break;
    default: SA_EXPAND(0);
  }
#undef SA_EXPAND
  return hipGetLastError();
}

int g_gemm_bm = 0;      // tuning override of the tile height: 0 = automatic, else 128 or 256
int g_gemm_engine = 0;  // tuning override: 0 = automatic, 1 = staged-register engine,
                        // 2 = pipelined 256 x 128 / 128 x 128 tiles, 3 = wide (dense only)
int g_gemm_stages = 0;  // tuning override of the pipelined stage count: 0 = automatic, else 3..6
constexpr int kMaxStages = 6;

template <int AK, int BM, int NS>
constexpr bool pipe_fits() {
  return NS * pipe_stage_halves<AK, BM>() * 2 + (AK == kA24 ? 256 : 0) <= 160 * 1024;
}

// Launch with ns stages (clamped down to the most the tile's LDS holds).
template <int AK, int BM, int NS = 3>
hipError_t launch_pipe_stages(const GParams& p, int64_t tiles, int ns, hipStream_t s) {
  if constexpr (NS < kMaxStages && pipe_fits<AK, BM, NS + 1>()) {
    if (ns > NS) return launch_pipe_stages<AK, BM, NS + 1>(p, tiles, ns, s);
  }
  hipLaunchKernelGGL((k_gemm_pipe<AK, BM, NS>), dim3((unsigned)tiles), dim3(NTH), 0, s, p);
  return hipGetLastError();
}

template <int NS = 3>
hipError_t launch_wide_stages(const GParams& p, int64_t tiles, int ns, hipStream_t s) {
  if constexpr (NS < kWideMaxStages) {
    if (ns > NS) return launch_wide_stages<NS + 1>(p, tiles, ns, s);
  }
  hipLaunchKernelGGL((k_gemm_wide<NS>), dim3((unsigned)tiles), dim3(WNT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wide(const GParams& p, hipStream_t s) {
  const int64_t tiles = ((p.T + WBM - 1) / WBM) * ((p.d_out + WBN - 1) / WBN);
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  return launch_wide_stages(p, tiles, g_gemm_stages ? g_gemm_stages : kWideMaxStages, s);
}

// Wide or 256 x 128 tiles, from rates measured at K = 4096 (2048..8192 rows,
// 4096..22016 outputs): a CU finishes one wide tile in ~115 us, and two
// 256 x 128 tiles sharing it in ~150 us, i.e. the wide engine does ~1.29x
// the work per CU.  But the wide engine runs in whole rounds of one tile per
// CU, while the narrow engine's time grows about linearly with its tile
// count (a CU's second slot refills as tiles finish).  So the wide engine
// pays when its rounds take less than the narrow tiles at 1.29x the rate:
// rounds <= 1.29 * narrow tiles / (2 * CUs).  It picked the faster engine at
// each of the 17 shapes measured (losses of 2-7% avoided at 1.1-1.3 rounds
// and just past 2; gains of 6-15% elsewhere).
// 2:4 on wide tiles or on 128 x 128 tiles (two per CU).  Measured at
// K = 4096: a round of wide tiles takes ~108 us and a round of 128 x 128
// tiles ~71 us, so per unit of work the wide engine is ~1.3x faster, but it
// runs in whole rounds of one tile per CU.  The wide engine is taken when
// its rounds stay within 1.5x its tile count per CU: 344 tiles (2 rounds;
// 190 against 206 us), 256, 688, 896 and 1376 tiles take it; 64 and 128
// tiles (a round mostly idle: 28 against 16 us, 99 against 75 us) do not.
bool wide24_pays(int64_t T, int64_t d_out, int64_t cus) {
  const int64_t wide = ((T + WBM - 1) / WBM) * ((d_out + WBN - 1) / WBN);
  const int64_t rounds = (wide + cus - 1) / cus;
  return 100 * rounds * cus <= 150 * wide;
}

bool wide_pays(int64_t T, int64_t d_out, int64_t cus) {
  const int64_t wide = ((T + WBM - 1) / WBM) * ((d_out + WBN - 1) / WBN);
  const int64_t narrow = ((T + 255) / 256) * ((d_out + PBN - 1) / PBN);
  const int64_t rounds = (wide + cus - 1) / cus;
  return 200 * rounds * cus <= 129 * narrow;
}

hipError_t launch_wide24(const GParams& p, hipStream_t s) {
  const int64_t tiles = ((p.T + WBM - 1) / WBM) * ((p.d_out + WBN - 1) / WBN);
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  hipLaunchKernelGGL(k_gemm_wide24, dim3((unsigned)tiles), dim3(WNT), 0, s, p);
  return hipGetLastError();
}

// 2:4 on the wide engine: when asked for (engine 3), or automatically where
// it pays (wide24_pays).
bool wide24_pays(int64_t T, int64_t d_out, int64_t cus);
bool wide24_chosen(int64_t T, int64_t d_out, int64_t cus) {
  return g_gemm_engine == 3 || (g_gemm_engine == 0 && g_gemm_bm == 0 && wide24_pays(T, d_out, cus));
}

// Dense on the pipelined engines: the wide one where it pays (automatic
// choice) or when asked for (engine 3).
bool pipe_wide(int ak, int64_t T, int64_t d_out, int64_t cus) {
  return ak == kADense &&
         (g_gemm_engine == 3 || (g_gemm_engine == 0 && g_gemm_bm == 0 && wide_pays(T, d_out, cus)));
}

// Pipelined engine tile height (measured): dense 256 rows, or 128 when
// 256-row tiles would give fewer workgroups than the device has CUs; 2:4
// always 128, where two workgroups share a CU (faster at both configured
// shapes).
int pipe_bm(int ak, int64_t T, int64_t d_out, int64_t cus) {
  const int64_t tiles256 = ((T + 255) / 256) * ((d_out + PBN - 1) / PBN);
  return g_gemm_bm ? g_gemm_bm : ((ak == kA24 || tiles256 < cus) ? 128 : 256);
}

template <int AK>
hipError_t launch_pipe(const GParams& p, hipStream_t s) {
  const int64_t cus = device_cus();
  if (pipe_wide(AK, p.T, p.d_out, cus)) return launch_wide(p, s);
  const int64_t ntl = (p.d_out + PBN - 1) / PBN;
  const int bm = pipe_bm(AK, p.T, p.d_out, cus);
  const int64_t tiles = ((p.T + bm - 1) / bm) * ntl;
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  const int ns = g_gemm_stages ? g_gemm_stages : 3;
  if (bm == 256) return launch_pipe_stages<AK, 256>(p, tiles, ns, s);
  return launch_pipe_stages<AK, 128>(p, tiles, ns, s);
}

template <int AK, int BM>
hipError_t launch_tile(const GParams& p, hipStream_t s) {
  const int64_t tiles = ((p.T + BM - 1) / BM) * ((p.d_out + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  hipLaunchKernelGGL((k_gemm<AK, BM>), dim3((unsigned)tiles), dim3(NTH), 0, s, p);
  return hipGetLastError();
}


// 256-row tiles when there are enough of them to fill the chip, 128 otherwise.
// The zero-filled N:M staging (any pattern but 2:4) needs more registers per
// row and measured slower at 256 rows, so it stays at 128 unless overridden.
int kind_bm(int ak, int64_t T, int64_t d_out) {
  const int64_t tiles256 = ((T + 255) / 256) * ((d_out + BN - 1) / BN);
  const bool tall_ok = (ak == kADense || ak == kA24) && tiles256 >= 256;
  return g_gemm_bm ? g_gemm_bm : (tall_ok ? 256 : 128);
}

template <int AK>
hipError_t launch_kind(const GParams& p, hipStream_t s) {
  if (kind_bm(AK, p.T, p.d_out) == 256) return launch_tile<AK, 256>(p, s);
  return launch_tile<AK, 128>(p, s);
}

// Tile-shared engine: K step KB = 32 m / n dense rows (64 or 128), tile
// height as the dense engine picks it (256 rows when they fill the CUs).
bool shared_engine_ok(int64_t d_in, int n, int m, int tt) {
  if (tt % 32 != 0 || n < 1 || 32 % n != 0 || (m != 2 * n && m != 4 * n)) return false;
  return d_in % (32 * m / n) == 0;
}

template <int KB>
hipError_t launch_shared_kb(const GParams& p, hipStream_t s) {
  const int64_t ntl = (p.d_out + PBN - 1) / PBN;
  const int64_t tiles256 = ((p.T + 255) / 256) * ntl;
  const int bm = g_gemm_bm ? g_gemm_bm : (tiles256 < device_cus() ? 128 : 256);
  const int64_t tiles = ((p.T + bm - 1) / bm) * ntl;
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  if (bm == 256)
    hipLaunchKernelGGL((k_gemm_shared<KB, 256>), dim3((unsigned)tiles), dim3(NTH), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm_shared<KB, 128>), dim3((unsigned)tiles), dim3(NTH), 0, s, p);
  return hipGetLastError();
}

// Whole-tile gather (one pattern per row tile: tt a multiple of 128): the
// dense engine over d_in n / m compressed K, loading only the kept WT rows.
bool gather_shape_ok(int64_t d_in, int n, int m, int tt) {
  return tt % 128 == 0 && n >= 1 && 32 % n == 0 && n <= m && d_in % m == 0 &&
         d_in <= 32 * kGatherMaskWords && (d_in / m * n) % 32 == 0;
}

// 32-row tiles of one pattern (tt a multiple of 32), only the kept WT rows.
bool g32_shape_ok(int64_t d_in, int n, int m, int tt) {
  return tt % 32 == 0 && n >= 1 && 32 % n == 0 && n <= m && d_in % m == 0 &&
         d_in <= 32 * kGatherMaskWords && (d_in / m * n) % kG32BK == 0;
}

template <int BN>
hipError_t launch_g32_bn(const GParams& p, hipStream_t s) {
  const int64_t tiles = ((p.T + 31) / 32) * ((p.d_out + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  const int64_t kept = p.d_in / p.m * p.n;
  const dim3 grid((unsigned)tiles);
  if (g_gemm_stages >= 4)
    hipLaunchKernelGGL((k_gemm_g32<4, kGatherTableBytes, BN>), grid, dim3(NTH), 0, s, p);
  else if (kept <= 512)
    hipLaunchKernelGGL((k_gemm_g32<3, 512, BN>), grid, dim3(NTH), 0, s, p);
  else if (kept <= 2048)
    hipLaunchKernelGGL((k_gemm_g32<3, 2048, BN>), grid, dim3(NTH), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm_g32<3, kGatherTableBytes, BN>), grid, dim3(NTH), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_g32(const GParams& p, hipStream_t s) {
  if (g_gemm_engine == 3) return launch_g32_bn<256>(p, s);
  return launch_g32_bn<128>(p, s);
}

hipError_t launch_gather(const GParams& p, hipStream_t s) {
  const int64_t ntl = (p.d_out + PBN - 1) / PBN;
  const int64_t tiles256 = ((p.T + 255) / 256) * ntl;
  int bm = g_gemm_bm ? g_gemm_bm : ((p.tt % 256 == 0 && tiles256 >= device_cus()) ? 256 : 128);
  if (p.tt % bm != 0) bm = 128;  // a tile of rows must share one pattern
  const int64_t tiles = ((p.T + bm - 1) / bm) * ntl;
  if (tiles > 0x7fffffffLL) return hipErrorNotSupported;
  const int ns = g_gemm_stages ? g_gemm_stages : 3;
  if (bm == 256) return launch_pipe_stages<kAGather, 256>(p, tiles, ns, s);
  return launch_pipe_stages<kAGather, 128>(p, tiles, ns, s);
}

}  // namespace

size_t nm_shared_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m, int tt) {
  if (gather_shape_ok(d_in, n, m, tt) || g32_shape_ok(d_in, n, m, tt) ||
      shared_engine_ok(d_in, n, m, tt))
    return 0;
  return (size_t)T * (size_t)d_in * 2;
}

hipError_t launch_nm_shared_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T,
                                 int64_t d_in, int n, int m, int tt, const uint16_t* wt,
                                 int64_t d_out, uint16_t* y, void* ws, size_t ws_bytes,
                                 hipStream_t s) {
  GParams p{};
  p.x = xval;
  p.mask = mask;
  p.wt = wt;
  p.y = y;
  p.T = T;
  p.d_in = d_in;
  p.d_out = d_out;
  p.n = n;
  p.m = m;
  p.tt = tt;
  if (gather_shape_ok(d_in, n, m, tt)) return launch_gather(p, s);
  // 32-row tiles, unless a tile height is asked for and the per-block
  // gather can take the shape
  if (g32_shape_ok(d_in, n, m, tt) && (g_gemm_bm == 0 || !shared_engine_ok(d_in, n, m, tt)))
    return launch_g32(p, s);
  if (shared_engine_ok(d_in, n, m, tt)) {
    if (32 * m / n == 64) return launch_shared_kb<64>(p, s);
    return launch_shared_kb<128>(p, s);
  }
  // any other tile or pattern: expand into the workspace, then dense
  if (ws == nullptr || ws_bytes < nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt))
    return hipErrorInvalidValue;
  GParams pd = p;
  pd.x = static_cast<const uint16_t*>(ws);
  pd.mask = nullptr;
  hipError_t e = launch_nm_expand(xval, mask, T, d_in, n, m, tt, static_cast<uint16_t*>(ws), s);
  if (e != hipSuccess) return e;
  if (g_gemm_engine != 1 && pipe_ok<kADense>(pd)) return launch_pipe<kADense>(pd, s);
  return launch_kind<kADense>(pd, s);
}

int gemm_plan(int op, int64_t T, int64_t d_in, int64_t d_out, int n, int m, int64_t cus,
              int* engine, int* tile_rows, int* tile_cols, int64_t* tiles) {
  // the shape conditions of pipe_ok (16-byte aligned operands assumed)
  auto pipe_shape = [&](int bk) { return d_in % bk == 0 && d_out % 8 == 0 && d_out >= 8; };
  int ak = kADense;
  bool pipe = false;
  if (op == 0) {
    pipe = g_gemm_engine != 1 && pipe_shape(Pipe<kADense, 256>::kBK);
  } else if (n == 2 && m == 4) {
    ak = kA24;
    pipe = g_gemm_engine != 1 && pipe_shape(Pipe<kA24, 256>::kBK);
  } else {  // the expanded copy on the dense engine, with a workspace
    pipe = g_gemm_engine != 1 && pipe_shape(Pipe<kADense, 256>::kBK);
    if (!pipe) ak = (4 * n) % m == 0 ? kANMVec : kANM;
  }
  if (pipe && (pipe_wide(ak, T, d_out, cus) || (ak == kA24 && wide24_chosen(T, d_out, cus)))) {
    *engine = 3;
    *tile_rows = WBM;
    *tile_cols = WBN;
  } else if (pipe) {
    *engine = 2;
    *tile_rows = pipe_bm(ak, T, d_out, cus);
    *tile_cols = PBN;
  } else {
    *engine = 1;
    *tile_rows = kind_bm(ak, T, d_out);
    *tile_cols = BN;
  }
  *tiles = ((T + *tile_rows - 1) / *tile_rows) * ((d_out + *tile_cols - 1) / *tile_cols);
  return 0;
}

int gemm_set_tuning(int bm, int engine, int stages) {
  if ((bm != 0 && bm != 128 && bm != 256) || engine < 0 || engine > 3 ||
      (stages != 0 && (stages < 3 || stages > kMaxStages)) || (engine == 3 && bm == 128))
    return 1;
  g_gemm_bm = bm;
  g_gemm_engine = engine;
  g_gemm_stages = stages;
  return 0;
}

hipError_t launch_dense_gemm(const uint16_t* x, int64_t T, int64_t d_in, const uint16_t* wt,
                             int64_t d_out, uint16_t* y, hipStream_t s) {
  GParams p{};
  p.x = x;
  p.wt = wt;
  p.y = y;
  p.T = T;
  p.d_in = d_in;
  p.d_out = d_out;
  if (g_gemm_engine != 1 && pipe_ok<kADense>(p)) return launch_pipe<kADense>(p, s);
  return launch_kind<kADense>(p, s);
}

size_t nm_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m) {
  if (n == 2 && m == 4) return 0;
  return (size_t)T * (size_t)d_in * 2;
}

hipError_t launch_nm_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T, int64_t d_in,
                          int n, int m, const uint16_t* wt, int64_t d_out, uint16_t* y,
                          void* ws, size_t ws_bytes, hipStream_t s) {
  GParams p{};
  p.x = xval;
  p.mask = mask;
  p.wt = wt;
  p.y = y;
  p.T = T;
  p.d_in = d_in;
  p.d_out = d_out;
  p.n = n;
  p.m = m;
  // 2:4 on the sparse MFMA; every other pattern through zero-filled dense
  // tiles (vector loads when m divides 4n)
  if (n == 2 && m == 4) {
    if (g_gemm_engine != 1 && pipe_ok<kA24>(p)) {
      if (wide24_chosen(T, d_out, device_cus())) return launch_wide24(p, s);
      return launch_pipe<kA24>(p, s);
    }
    return launch_kind<kA24>(p, s);
  }
  // two passes through the dense pipelined engine when a workspace is given
  if (g_gemm_engine != 1 && ws != nullptr && ws_bytes >= nm_spmm_workspace_bytes(T, d_in, n, m) &&
      (reinterpret_cast<uintptr_t>(ws) & 15u) == 0) {
    GParams pd = p;
    pd.x = static_cast<const uint16_t*>(ws);
    pd.mask = nullptr;
    if (pipe_ok<kADense>(pd)) {
      hipError_t e =
          launch_nm_expand(xval, mask, T, d_in, n, m, 1, static_cast<uint16_t*>(ws), s);
      if (e != hipSuccess) return e;
      return launch_pipe<kADense>(pd, s);
    }
  }
  if ((4 * n) % m == 0) return launch_kind<kANMVec>(p, s);
  return launch_kind<kANM>(p, s);
}

}  // namespace sa
