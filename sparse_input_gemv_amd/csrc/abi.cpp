// extern "C" entry points of libsparse_act.so (declared in
// include/sparse_act.h): validate on the host, then enqueue on the caller's
// stream.  No allocation, no synchronisation, no exceptions across the ABI.
#include <hip/hip_runtime_api.h>

#include "../../include/sparse_act.h"
#include "launch.hpp"
#include "validate.hpp"

namespace {

int hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return SA_OK;
  sa::set_error("%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  return SA_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    default: return "SA_ERR_UNKNOWN";
  }
}

const char* sa_last_error(void) { return sa::last_error(); }

int sa_version(void) { return 100; }

int act_sparsify_threshold(const uint16_t* x, int64_t rows, int64_t d, float t, uint32_t* mask,
                           int32_t* idx, uint16_t* val, int32_t* nnz, int64_t cap,
                           void* stream) {
  sa::clear_error();
  int st = sa::check_threshold(x, rows, d, t, mask, idx, val, nnz, cap);
  if (st != SA_OK) return st;
  if (rows == 0) return SA_OK;
  return hip_status(
      sa::launch_sparsify_threshold(x, rows, d, t, mask, idx, val, nnz, cap, as_stream(stream)),
      "act_sparsify_threshold");
}

int act_sparsify_scored(const uint16_t* x, int64_t rows, int64_t d, const uint16_t* mu,
                        const double* colnorm, int n, int m, double t, uint32_t* mask,
                        int32_t* idx, uint16_t* val, int32_t* nnz, int64_t cap, float* alpha,
                        void* stream) {
  sa::clear_error();
  int st = sa::check_scored(x, rows, d, mu, colnorm, n, m, t, mask, idx, val, nnz, cap, alpha);
  if (st != SA_OK) return st;
  if (rows == 0) return SA_OK;
  return hip_status(sa::launch_sparsify_scored(x, rows, d, mu, colnorm, n, m, t, mask, idx, val,
                                               nnz, alpha, cap, as_stream(stream)),
                    "act_sparsify_scored");
}

int act_sparsify_topk(const uint16_t* x, int64_t rows, int64_t d, int64_t k, uint32_t* mask,
                      int32_t* idx, uint16_t* val, int32_t* nnz, int64_t cap, void* stream) {
  sa::clear_error();
  int st = sa::check_topk(x, rows, d, k, mask, idx, val, nnz, cap);
  if (st != SA_OK) return st;
  if (rows == 0) return SA_OK;
  return hip_status(sa::launch_sparsify_topk(x, rows, d, k, mask, idx, val, nnz, cap, nullptr,
                                             as_stream(stream)),
                    "act_sparsify_topk");
}

int act_topk_cutoff(const uint16_t* x, int64_t rows, int64_t d, int64_t k, int32_t* cut,
                    void* stream) {
  sa::clear_error();
  int st = sa::check_topk_cutoff(x, rows, d, k, cut, "act_topk_cutoff");
  if (st != SA_OK) return st;
  if (rows == 0) return SA_OK;
  return hip_status(sa::launch_sparsify_topk(x, rows, d, k, nullptr, nullptr, nullptr, nullptr,
                                             0, cut, as_stream(stream)),
                    "act_topk_cutoff");
}

int act_sparsify_nm(const uint16_t* x, int64_t rows, int64_t d, int n, int m, uint32_t* mask,
                    uint16_t* val, void* stream) {
  sa::clear_error();
  int st = sa::check_nm(x, rows, d, n, m, mask, val);
  if (st != SA_OK) return st;
  if (rows == 0) return SA_OK;
  return hip_status(sa::launch_sparsify_nm(x, rows, d, n, m, mask, val, as_stream(stream)),
                    "act_sparsify_nm");
}

int act_sparsify_nm_shared(const uint16_t* x, int64_t rows, int64_t d, int n, int m, int tt,
                           uint32_t* mask, uint16_t* val, void* stream) {
  sa::clear_error();
  int st = sa::check_nm_shared(x, rows, d, n, m, tt, mask, val);
  if (st != SA_OK) return st;
  if (rows == 0) return SA_OK;
  hipError_t e =
      sa::launch_sparsify_nm_shared(x, rows, d, n, m, tt, mask, val, as_stream(stream));
  if (e == hipErrorNotSupported) {
    sa::set_error("act_sparsify_nm_shared: shape not supported by the compiled kernels");
    return SA_ERR_UNSUPPORTED;
  }
  return hip_status(e, "act_sparsify_nm_shared");
}

int act_calibrate_threshold(const uint16_t* samples, int64_t n, double s, float* t_out,
                            void* stream) {
  sa::clear_error();
  int st = sa::check_calibrate(samples, n, s, t_out);
  if (st != SA_OK) return st;
  return hip_status(sa::launch_calibrate(samples, n, s, t_out, as_stream(stream)),
                    "act_calibrate_threshold");
}

static_assert(SA_WS_TICKET_BYTES == sa::kGemvTicketBytes, "header and library agree");

size_t sa_workspace_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  if (d_out < 1 || d_in < 1) return 0;
  if (batch < 1) batch = 1;
  if (batch > SA_MAX_BATCH) batch = SA_MAX_BATCH;
  return sa::gemv_workspace_bytes(d_out, d_in, batch);
}

size_t sparse_gemv_workspace_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  return sa_workspace_bytes(d_out, d_in, batch);
}

size_t sa_workspace_zero_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  if (d_out < 1 || d_in < 1) return 0;
  if (batch < 1) batch = 1;
  if (batch > SA_MAX_BATCH) batch = SA_MAX_BATCH;
  return sa::gemv_workspace_zero_bytes(d_out, d_in, batch);
}

static int run_gemv(const sa::GemvCall& c, const char* fn, void* stream) {
  if (c.batch == 0) return SA_OK;
  return hip_status(sa::launch_gemv(c, as_stream(stream)), fn);
}

int sparse_gemv(const uint16_t* wt, int64_t d_out, int64_t d_in, const int32_t* idx,
                const uint16_t* val, const int32_t* nnz, int64_t batch, int64_t cap,
                uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_sparse_gemv(idx, val, nnz, batch, cap);
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeList;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.idx = idx;
  c.val = val;
  c.nnz = nnz;
  c.cap = cap;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "sparse_gemv", stream);
}

int sparse_gemv_threshold(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x,
                          int64_t batch, float t, uint16_t* y, void* ws, size_t ws_bytes,
                          void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_activation(x, "sparse_gemv_threshold: x");
  if (st == SA_OK) st = sa::check_threshold_value(t);
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeThreshold;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.x = x;
  c.t = t;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "sparse_gemv_threshold", stream);
}

int sparse_gemv_scored(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x,
                       const uint16_t* mu, const double* colnorm, double t, int var,
                       const uint16_t* bias, uint16_t* y, void* ws, size_t ws_bytes,
                       void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, 1);
  int st = sa::check_gemv_common(wt, d_out, d_in, 1, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_activation(x, "sparse_gemv_scored: x");
  if (st == SA_OK && (!(t >= 0.0) || t > 1e300 || (reinterpret_cast<uintptr_t>(mu) & 1u) != 0 ||
                      (reinterpret_cast<uintptr_t>(colnorm) & 7u) != 0 ||
                      (reinterpret_cast<uintptr_t>(bias) & 1u) != 0)) {
    sa::set_error("sparse_gemv_scored: t must be finite and >= 0; mu, colnorm, bias aligned");
    st = SA_ERR_INVALID_ARG;
  }
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeScored;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = 1;
  c.x = x;
  c.mu = mu;
  c.colnorm = colnorm;
  c.t64 = t;
  c.var = var != 0;
  c.bias = bias;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "sparse_gemv_scored", stream);
}

int sparse_gemv_scored_nm(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x,
                          const uint16_t* mu, const double* colnorm, int n, int m, int var,
                          const uint16_t* bias, uint16_t* y, void* ws, size_t ws_bytes,
                          void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, 1);
  int st = sa::check_gemv_common(wt, d_out, d_in, 1, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_activation(x, "sparse_gemv_scored_nm: x");
  if (st == SA_OK && (!(m == 4 || m == 8 || m == 16 || m == 32) || n < 1 || n > m ||
                      d_in % m != 0)) {
    sa::set_error("sparse_gemv_scored_nm: need m in {4, 8, 16, 32}, 1 <= n <= m, d_in % m == 0");
    st = SA_ERR_INVALID_ARG;
  }
  if (st == SA_OK && ((reinterpret_cast<uintptr_t>(mu) & 1u) != 0 ||
                      (reinterpret_cast<uintptr_t>(colnorm) & 7u) != 0 ||
                      (reinterpret_cast<uintptr_t>(bias) & 1u) != 0)) {
    sa::set_error("sparse_gemv_scored_nm: mu, colnorm, bias must be aligned");
    st = SA_ERR_INVALID_ARG;
  }
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeScoredNM;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = 1;
  c.x = x;
  c.mu = mu;
  c.colnorm = colnorm;
  c.sn = n;
  c.sm = m;
  c.var = var != 0;
  c.bias = bias;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "sparse_gemv_scored_nm", stream);
}

static_assert(SA_NOALLOC_SCRATCH_BYTES == sa::kNoAllocScratchBytes, "header and library agree");

int sparse_gemv_topk(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x,
                     int64_t batch, int64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                     void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, ws, ws_bytes, need);
  // the cutoff pairs live in the workspace (checked above when batch > 0)
  int32_t* cut = (st == SA_OK && batch > 0)
                     ? reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) +
                                                  sa::gemv_workspace_cut_offset(d_out, d_in, batch))
                     : nullptr;
  if (st == SA_OK) st = sa::check_topk_cutoff(x, batch, d_in, k, cut, "sparse_gemv_topk");
  if (st != SA_OK || batch == 0) return st;
  sa::GemvCall c;
  c.mode = sa::kModeTopK;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.x = x;
  c.topk_k = k;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return hip_status(sa::launch_gemv_topk(c, cut, as_stream(stream)), "sparse_gemv_topk");
}

int sparse_gemv_threshold_noalloc(const uint16_t* wt, int64_t d_out, int64_t d_in,
                                  const uint16_t* x, int64_t batch, float t, uint16_t* y,
                                  void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  // sizes are checked before the scratch is looked up: an oversized call
  // returns at once
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, nullptr, 0, 0);
  if (st == SA_OK) st = sa::check_activation(x, "sparse_gemv_threshold_noalloc: x");
  if (st == SA_OK) st = sa::check_threshold_value(t);
  if (st == SA_OK) st = sa::check_noalloc_size(need, sa::kNoAllocScratchBytes);
  if (st != SA_OK) return st;
  if (batch == 0) return SA_OK;
  void* ws = nullptr;
  const hipError_t e = sa::gemv_noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "sparse_gemv_threshold_noalloc");
  sa::GemvCall c;
  c.mode = sa::kModeThreshold;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.x = x;
  c.t = t;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = sa::kNoAllocScratchBytes;
  return run_gemv(c, "sparse_gemv_threshold_noalloc", stream);
}

int sparse_gemv_corrected(const uint16_t* wt, int64_t d_out, int64_t d_in, const int32_t* idx,
                          const uint16_t* val, const int32_t* nnz, int64_t batch, int64_t cap,
                          const float* alpha, const uint16_t* bias, uint16_t* y, void* ws,
                          size_t ws_bytes, void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_sparse_gemv(idx, val, nnz, batch, cap);
  if (st == SA_OK &&
      ((reinterpret_cast<uintptr_t>(alpha) & 3u) != 0 || (reinterpret_cast<uintptr_t>(bias) & 1u) != 0)) {
    sa::set_error("sparse_gemv_corrected: misaligned alpha or bias");
    st = SA_ERR_INVALID_ARG;
  }
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeList;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.idx = idx;
  c.val = val;
  c.nnz = nnz;
  c.cap = cap;
  c.alpha = alpha;
  c.bias = bias;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "sparse_gemv_corrected", stream);
}

int rana_adapter_gemv(const uint16_t* b, int64_t r, int64_t d_in, const uint16_t* at,
                      int64_t d_out, const uint16_t* x, int64_t batch, float t, uint16_t* v,
                      uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, r, batch < 1 ? 1 : batch);
  int st = sa::check_rows_gemv(b, r, d_in, batch, v, "rana_adapter_gemv");
  if (st == SA_OK) st = sa::check_gemv_common(at, d_out, r, batch, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_activation(x, "rana_adapter_gemv: x");
  if (st == SA_OK) st = sa::check_threshold_value(t);
  if (st != SA_OK) return st;
  if (batch == 0) return SA_OK;
  st = hip_status(sa::launch_gemv_rows(b, r, d_in, x, (int)batch, v, as_stream(stream)),
                  "rana_adapter_gemv");
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeSquare;
  c.wt = at;
  c.d_out = d_out;
  c.d_in = r;
  c.batch = (int)batch;
  c.x = v;
  c.t = t;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "rana_adapter_gemv", stream);
}

int masked_gemv(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x,
                const uint32_t* mask, int64_t batch, uint16_t* y, void* ws, size_t ws_bytes,
                void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_activation(x, "masked_gemv: x");
  if (st == SA_OK && (mask == nullptr || (reinterpret_cast<uintptr_t>(mask) & 3u) != 0)) {
    sa::set_error("masked_gemv: mask must be a non-NULL 4-byte aligned pointer");
    st = SA_ERR_INVALID_ARG;
  }
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeMasked;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.x = x;
  c.xmask = mask;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "masked_gemv", stream);
}

int dense_gemv(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x, int64_t batch,
               uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_out, d_in, batch < 1 ? 1 : batch);
  int st = sa::check_gemv_common(wt, d_out, d_in, batch, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_activation(x, "dense_gemv: x");
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeDense;
  c.wt = wt;
  c.d_out = d_out;
  c.d_in = d_in;
  c.batch = (int)batch;
  c.x = x;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "dense_gemv", stream);
}

int masked_swiglu_down(const uint16_t* g, const uint16_t* u, const uint16_t* wdt,
                       const double* colnorm, int64_t d_ff, int64_t d_model, double t, int mode,
                       uint16_t* y, uint32_t* mask, int32_t* nnz, void* ws, size_t ws_bytes,
                       void* stream) {
  sa::clear_error();
  const size_t need = sa::gemv_workspace_bytes(d_model, d_ff, 1);
  int st = sa::check_gemv_common(wdt, d_model, d_ff, 1, y, ws, ws_bytes, need);
  if (st == SA_OK) st = sa::check_swiglu(g, u, colnorm, d_ff, t, mode);
  if (st == SA_OK && ((reinterpret_cast<uintptr_t>(mask) & 3u) != 0 ||
                      (reinterpret_cast<uintptr_t>(nnz) & 3u) != 0)) {
    sa::set_error("masked_swiglu_down: mask and nnz must be 4-byte aligned");
    st = SA_ERR_INVALID_ARG;
  }
  if (st != SA_OK) return st;
  sa::GemvCall c;
  c.mode = sa::kModeSwiglu;
  c.wt = wdt;
  c.d_out = d_model;
  c.d_in = d_ff;
  c.batch = 1;
  c.g = g;
  c.u = u;
  c.colnorm = colnorm;
  c.t64 = t;
  c.swiglu_mode = mode;
  c.out_mask = mask;
  c.out_nnz = nnz;
  c.y = y;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  return run_gemv(c, "masked_swiglu_down", stream);
}

int weight_col_norms(const uint16_t* wt, int64_t d_in, int64_t d_out, double* out,
                     void* stream) {
  sa::clear_error();
  int st = sa::check_col_norms(wt, d_in, d_out, out);
  if (st != SA_OK) return st;
  if (d_in == 0) return SA_OK;
  return hip_status(sa::launch_col_norms(wt, d_in, d_out, out, as_stream(stream)),
                    "weight_col_norms");
}

static_assert(SA_READ_STREAM_SINK_WORDS == sa::kReadStreamBlocks * sa::kReadStreamThreads / 64,
              "one sink word per wave of the read-stream grid");

int sa_read_stream_grid(const void* src, size_t bytes, uint32_t* sink, int blocks,
                        void* stream) {
  sa::clear_error();
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) {
    sa::set_error("sa_read_stream: src and sink must be non-NULL and aligned, bytes a positive "
                  "multiple of 16");
    return SA_ERR_INVALID_ARG;
  }
  if (blocks < 1 || blocks > sa::kReadStreamMaxBlocks) {
    sa::set_error("sa_read_stream_grid: blocks must be in [1, %d]", sa::kReadStreamMaxBlocks);
    return SA_ERR_INVALID_ARG;
  }
  return hip_status(sa::launch_read_stream(src, bytes, sink, blocks, as_stream(stream)),
                    "sa_read_stream");
}

int sa_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  return sa_read_stream_grid(src, bytes, sink, sa::kReadStreamBlocks, stream);
}

size_t sa_nm_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m) {
  if (T < 1 || d_in < 1 || m < 1 || n < 1 || n > m) return 0;
  return sa::nm_spmm_workspace_bytes(T, d_in, n, m);
}

int nm_act_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T, int64_t d_in, int n,
                int m, const uint16_t* wt, int64_t d_out, uint16_t* y, void* ws, size_t ws_bytes,
                void* stream) {
  sa::clear_error();
  int st = sa::check_nm_spmm(xval, mask, T, d_in, n, m, wt, d_out, y);
  if (st != SA_OK) return st;
  if (ws != nullptr) {
    const size_t need = T > 0 ? sa::nm_spmm_workspace_bytes(T, d_in, n, m) : 0;
    if (ws_bytes < need) {
      sa::set_error("nm_act_spmm: workspace of %zu bytes, %zu needed", ws_bytes, need);
      return SA_ERR_WORKSPACE;
    }
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) {
      sa::set_error("nm_act_spmm: workspace must be 16-byte aligned");
      return SA_ERR_INVALID_ARG;
    }
  }
  if (T == 0) return SA_OK;
  hipError_t e = sa::launch_nm_spmm(xval, mask, T, d_in, n, m, wt, d_out, y, ws, ws_bytes,
                                    as_stream(stream));
  if (e == hipErrorNotSupported) {
    sa::set_error("nm_act_spmm: shape not supported by the compiled kernels");
    return SA_ERR_UNSUPPORTED;
  }
  return hip_status(e, "nm_act_spmm");
}

size_t sa_nm_shared_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m, int tt) {
  if (T < 1 || d_in < 1 || m < 1 || n < 1 || n > m || tt < 1) return 0;
  return sa::nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt);
}

int nm_shared_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T, int64_t d_in, int n,
                   int m, int tt, const uint16_t* wt, int64_t d_out, uint16_t* y, void* ws,
                   size_t ws_bytes, void* stream) {
  sa::clear_error();
  int st = sa::check_nm_shared_spmm(xval, mask, T, d_in, n, m, tt, wt, d_out, y);
  if (st != SA_OK) return st;
  const size_t need = T > 0 ? sa::nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt) : 0;
  if (need > 0 && (ws == nullptr || ws_bytes < need)) {
    sa::set_error("nm_shared_spmm: this tile size and pattern need a workspace of %zu bytes "
                  "(%zu given)", need, ws == nullptr ? (size_t)0 : ws_bytes);
    return SA_ERR_WORKSPACE;
  }
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) & 15u) != 0) {
    sa::set_error("nm_shared_spmm: workspace must be 16-byte aligned");
    return SA_ERR_INVALID_ARG;
  }
  if (T == 0) return SA_OK;
  hipError_t e = sa::launch_nm_shared_spmm(xval, mask, T, d_in, n, m, tt, wt, d_out, y, ws,
                                           ws_bytes, as_stream(stream));
  if (e == hipErrorNotSupported) {
    sa::set_error("nm_shared_spmm: shape not supported by the compiled kernels");
    return SA_ERR_UNSUPPORTED;
  }
  return hip_status(e, "nm_shared_spmm");
}

int dense_gemm(const uint16_t* x, int64_t T, int64_t d_in, const uint16_t* wt, int64_t d_out,
               uint16_t* y, void* stream) {
  sa::clear_error();
  int st = sa::check_dense_gemm(x, T, d_in, wt, d_out, y);
  if (st != SA_OK) return st;
  if (T == 0) return SA_OK;
  hipError_t e = sa::launch_dense_gemm(x, T, d_in, wt, d_out, y, as_stream(stream));
  if (e == hipErrorNotSupported) {
    sa::set_error("dense_gemm: shape not supported by the compiled kernels");
    return SA_ERR_UNSUPPORTED;
  }
  return hip_status(e, "dense_gemm");
}

int sa_set_gemv_tuning(int tiling, int target_wgs, int handoff) {
  sa::clear_error();
  if (sa::gemv_set_tuning(tiling, target_wgs, handoff) != 0) {
    sa::set_error("sa_set_gemv_tuning: unknown tiling %d, negative target or handoff %d",
                  tiling, handoff);
    return SA_ERR_INVALID_ARG;
  }
  return SA_OK;
}

int sa_set_gemv_test_hooks(int flags) {
  sa::clear_error();
  if (sa::gemv_set_test_hooks(flags) != 0) {
    sa::set_error("sa_set_gemv_test_hooks: flags must be 0 or 1 (got %d)", flags);
    return SA_ERR_INVALID_ARG;
  }
  return SA_OK;
}

int sa_set_gemm_tuning(int tile_rows, int engine, int stages) {
  sa::clear_error();
  if (sa::gemm_set_tuning(tile_rows, engine, stages) != 0) {
    sa::set_error("sa_set_gemm_tuning: tile_rows must be 0, 128 or 256 (got %d; 0 or 256 for "
                  "engine 3), engine 0..3 (got %d) and stages 0 or 3..6 (got %d)", tile_rows,
                  engine, stages);
    return SA_ERR_INVALID_ARG;
  }
  return SA_OK;
}

int sa_gemm_plan(int op, int64_t T, int64_t d_in, int64_t d_out, int n, int m, int cus,
                 int* engine, int* tile_rows, int* tile_cols, int64_t* tiles) {
  sa::clear_error();
  const bool pattern_ok = op == 0 || (m >= 1 && n >= 1 && n <= m && (m == 4 || m == 8 ||
                                                                     m == 16 || m == 32) &&
                                      d_in % m == 0 && d_in % 32 == 0);
  if ((op != 0 && op != 1) || !pattern_ok || T < 1 || d_in < 1 || d_out < 1 || cus < 0 ||
      engine == nullptr || tile_rows == nullptr || tile_cols == nullptr || tiles == nullptr) {
    sa::set_error("sa_gemm_plan: op must be 0 (dense_gemm) or 1 (nm_act_spmm, with a valid "
                  "n:m for d_in), sizes >= 1, cus >= 0 and every output non-NULL");
    return SA_ERR_INVALID_ARG;
  }
  sa::gemm_plan(op, T, d_in, d_out, n, m, cus > 0 ? cus : sa::device_cus(), engine, tile_rows,
                tile_cols, tiles);
  return SA_OK;
}

int sa_gemv_plan(int op, int64_t d_out, int64_t d_in, int64_t batch, int cus, int resident,
                 int* kernel, int* tile_o, int* grid_o, int* slices, int* handoff) {
  sa::clear_error();
  const bool known = op == SA_GEMV_THRESHOLD || op == SA_GEMV_DENSE || op == SA_GEMV_MASKED ||
                     op == SA_GEMV_LIST || op == SA_GEMV_SWIGLU || op == SA_GEMV_SCORED ||
                     op == SA_GEMV_SQUARE || op == SA_GEMV_TOPK;
  if (!known || d_out < 1 || d_in < 1 || batch < 1 || batch > SA_MAX_BATCH || cus < 0 ||
      resident < 0 || kernel == nullptr || tile_o == nullptr || grid_o == nullptr ||
      slices == nullptr || handoff == nullptr) {
    sa::set_error("sa_gemv_plan: unknown op %d, a size out of range (d_out %lld, d_in %lld, "
                  "batch %lld), a negative count or a NULL output", op, (long long)d_out,
                  (long long)d_in, (long long)batch);
    return SA_ERR_INVALID_ARG;
  }
  sa::gemv_plan(op, d_out, d_in, batch, cus, resident, kernel, tile_o, grid_o, slices, handoff);
  return SA_OK;
}

int sa_gemv_tiling_info(int i, int* tile_o, int* threads, int* unroll) {
  sa::clear_error();
  if (sa::gemv_tiling_info(i, tile_o, threads, unroll) != 0) {
    sa::set_error("sa_gemv_tiling_info: no tiling %d", i);
    return SA_ERR_INVALID_ARG;
  }
  return SA_OK;
}

}  // extern "C"
