// Host-side launchers implemented in the .hip files and called by abi.cpp
// after argument validation.  Each returns a HIP error code (0 = success).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// ---- sparsifiers (sparsify.hip) -------------------------------------------
hipError_t launch_sparsify_threshold(const uint16_t* x, int64_t rows, int64_t d, float t,
                                     uint32_t* mask, int32_t* idx, uint16_t* val,
                                     int32_t* nnz, int64_t cap, hipStream_t s);
hipError_t launch_sparsify_scored(const uint16_t* x, int64_t rows, int64_t d,
                                  const uint16_t* mu, const double* colnorm, int n, int m,
                                  double t, uint32_t* mask, int32_t* idx, uint16_t* val,
                                  int32_t* nnz, float* alpha, int64_t cap, hipStream_t s);
// cut (may be NULL): per row the pair (tau, i*) of the selection; mask, idx
// and val may all be NULL (then only cut and nnz are written).
hipError_t launch_sparsify_topk(const uint16_t* x, int64_t rows, int64_t d, int64_t k,
                                uint32_t* mask, int32_t* idx, uint16_t* val, int32_t* nnz,
                                int64_t cap, int32_t* cut, hipStream_t s);
hipError_t launch_sparsify_nm(const uint16_t* x, int64_t rows, int64_t d, int n, int m,
                              uint32_t* mask, uint16_t* val, hipStream_t s);
hipError_t launch_sparsify_nm_shared(const uint16_t* x, int64_t rows, int64_t d, int n, int m,
                                     int tt, uint32_t* mask, uint16_t* val, hipStream_t s);

// ---- calibration (calibrate.hip) ------------------------------------------
hipError_t launch_calibrate(const uint16_t* samples, int64_t n, double s, float* t_out,
                            hipStream_t st);

// ---- GEMV family (gemv.hip) -------------------------------------------------
enum GemvMode : int {
  kModeThreshold = 0,  // x + t: fused threshold
  kModeDense = 1,      // every column
  kModeMasked = 2,     // x + bitmask
  kModeList = 3,       // idx/val/nnz lists
  kModeSwiglu = 4,     // CATS / RaNA masked SwiGLU down
  kModeScored = 6,     // x + shift + weight norms: weight-aware threshold (batch 1)
  kModeSquare = 7,     // x + t: keep x_k iff x_k^2 >= t (the rank adapter's masker)
  kModeTopK = 8,       // x + per-row (tau, i*) from the Top-K select: keep iff
                       // key > tau, or key == tau and k <= i*
  kModeTopKSel = 9,    // kModeTopK with each workgroup selecting (tau, i*) itself
  kModeScoredNM = 10,  // kModeScored with n of every m entries kept by score (batch 1)
};

struct GemvCall {
  int mode = 0;
  const uint16_t* wt = nullptr;
  int64_t d_out = 0, d_in = 0;
  int batch = 1;
  // threshold / dense / masked
  const uint16_t* x = nullptr;
  const uint32_t* xmask = nullptr;
  float t = 0.f;
  const uint16_t* mu = nullptr;  // scored mode: static shift [d_in] (or none)
  const int32_t* cut = nullptr;  // Top-K mode: [batch][2] (tau, i*)
  int64_t topk_k = 0;            // kModeTopKSel: entries kept per row
  int var = 0;                   // scored mode: apply the variance correction
  int sn = 0, sm = 0;            // scored N:M mode: n kept of every m
  // lists
  const int32_t* idx = nullptr;
  const uint16_t* val = nullptr;
  const int32_t* nnz = nullptr;
  int64_t cap = 0;
  // swiglu
  const uint16_t* g = nullptr;
  const uint16_t* u = nullptr;
  const double* colnorm = nullptr;
  double t64 = 0.0;
  int swiglu_mode = 0;
  uint32_t* out_mask = nullptr;
  int32_t* out_nnz = nullptr;
  // output correction (null: none): y[b][o] = alpha[b] * sum + bias[o]
  const float* alpha = nullptr;
  const uint16_t* bias = nullptr;
  // output and scratch
  uint16_t* y = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

// Hand-off counters at the head of the GEMV workspace: one per output tile
// (d_out <= 524288, split-K tiles of >= 64 outputs), 128 bytes apart.
constexpr int kTicketStride = 32;  // uint32 words
constexpr int kMinSplitTileO = 64;
constexpr size_t kGemvTicketBytes = (size_t)(524288 / kMinSplitTileO) * kTicketStride * 4;

size_t gemv_workspace_bytes(int64_t d_out, int64_t d_in, int64_t batch);
// Offset in that workspace of SA_MAX_BATCH (tau, i*) pairs for sparse_gemv_topk.
size_t gemv_workspace_cut_offset(int64_t d_out, int64_t d_in, int64_t batch);
// Dense y[b] = W x[b] for a row-major W [d_out][d_in] (one wave per output;
// no workspace).  batch in 1..8.
hipError_t launch_gemv_rows(const uint16_t* w, int64_t d_out, int64_t d_in, const uint16_t* x,
                            int batch, uint16_t* y, hipStream_t s);
// Leading bytes of that workspace that must be zero before a call (and are
// zero after it): the hand-off counters, the status word and the slots.
size_t gemv_workspace_zero_bytes(int64_t d_out, int64_t d_in, int64_t batch);
// The allocation-free entry point's scratch: a static device array of
// kNoAllocScratchBytes per GPU; *ptr gets the current device's copy (looked
// up once per device).  Allocates nothing.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t gemv_noalloc_scratch(void** ptr);
// Returns hipErrorInvalidValue if the workspace is too small for the launch
// (checked by abi.cpp beforehand, so this is a second line of defence).
hipError_t launch_gemv(const GemvCall& c, hipStream_t s);
// Top-K GEMV (c.mode kModeTopK, c.topk_k; cut the [batch][2] cutoff pairs'
// place in the workspace): one launch in which every workgroup selects the
// row's cutoff itself where the in-workgroup select applies (split-K, batch
// 1, d_in <= the workgroup's threads x kTopkSelPerThread), else the select
// kernel writes cut and the GEMV reads it.
constexpr int kTopkSelPerThread = 16;
hipError_t launch_gemv_topk(const GemvCall& c, int32_t* cut, hipStream_t s);
hipError_t launch_col_norms(const uint16_t* wt, int64_t d_in, int64_t d_out, double* out,
                            hipStream_t s);
int gemv_set_tuning(int tiling, int target_wgs, int handoff);
int gemv_set_test_hooks(int flags);
// The decomposition launch_gemv would use (cus, resident: 0 = ask the device).
int gemv_plan(int mode, int64_t d_out, int64_t d_in, int64_t batch, int cus, int resident,
              int* kernel, int* tile_o, int* go, int* gk, int* handoff);
int gemv_tiling_info(int i, int* tile_o, int* threads, int* unroll);

// ---- read-stream calibration (stream.hip) -----------------------------------
constexpr int kReadStreamBlocks = 2048;  // measured best grid for a 45 MB read
constexpr int kReadStreamThreads = 256;
constexpr int kReadStreamMaxBlocks = 16384;
hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s);

// ---- MFMA matmuls (gemm.hip) ------------------------------------------------
// Compute units of the current device (cached per device).
int device_cus();

hipError_t launch_dense_gemm(const uint16_t* x, int64_t T, int64_t d_in, const uint16_t* wt,
                             int64_t d_out, uint16_t* y, hipStream_t s);
// The engine and tile a matmul call takes (op 0 dense_gemm, 1 nm_act_spmm
// with a workspace), on `cus` compute units, under the current tuning.
int gemm_plan(int op, int64_t T, int64_t d_in, int64_t d_out, int n, int m, int64_t cus,
              int* engine, int* tile_rows, int* tile_cols, int64_t* tiles);
size_t nm_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m);
hipError_t launch_nm_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T, int64_t d_in,
                          int n, int m, const uint16_t* wt, int64_t d_out, uint16_t* y,
                          void* ws, size_t ws_bytes, hipStream_t s);
size_t nm_shared_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m, int tt);
hipError_t launch_nm_shared_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T,
                                 int64_t d_in, int n, int m, int tt, const uint16_t* wt,
                                 int64_t d_out, uint16_t* y, void* ws, size_t ws_bytes,
                                 hipStream_t s);
int gemm_set_tuning(int bm, int engine, int stages);

}  // namespace sa
