// Host-side argument checks (see validate.hpp).  No HIP headers here.
#include "validate.hpp"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/sparse_act.h"

namespace sa {
namespace {

thread_local char g_msg[512] = {0};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace

void clear_error() { g_msg[0] = 0; }

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
}

const char* last_error() { return g_msg; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

static int check_rows_d(int64_t rows, int64_t d, const char* fn) {
  REQUIRE(rows >= 0, SA_ERR_INVALID_ARG, "%s: rows must be >= 0 (got %lld)", fn, (long long)rows);
  REQUIRE(d >= 1, SA_ERR_INVALID_ARG, "%s: d must be >= 1 (got %lld)", fn, (long long)d);
  REQUIRE(d <= kMaxD, SA_ERR_UNSUPPORTED, "%s: d = %lld exceeds %lld", fn, (long long)d,
          (long long)kMaxD);
  REQUIRE(rows <= 0x7fffffffLL, SA_ERR_UNSUPPORTED, "%s: rows too large", fn);
  return SA_OK;
}

static int check_list_outputs(const void* x, const void* mask, const void* idx, const void* val,
                              const void* nnz, const char* fn) {
  REQUIRE(x != nullptr, SA_ERR_INVALID_ARG, "%s: x is NULL", fn);
  REQUIRE(idx != nullptr && val != nullptr && nnz != nullptr, SA_ERR_INVALID_ARG,
          "%s: idx, val and nnz must not be NULL", fn);
  REQUIRE(aligned(x, 2) && aligned(val, 2), SA_ERR_INVALID_ARG,
          "%s: x and val must be 2-byte aligned", fn);
  REQUIRE(aligned(idx, 4) && aligned(nnz, 4) && aligned(mask, 4), SA_ERR_INVALID_ARG,
          "%s: idx, nnz and mask must be 4-byte aligned", fn);
  return SA_OK;
}

int check_threshold(const void* x, int64_t rows, int64_t d, float t, const void* mask,
                    const void* idx, const void* val, const void* nnz, int64_t cap) {
  const char* fn = "act_sparsify_threshold";
  int st = check_rows_d(rows, d, fn);
  if (st) return st;
  st = check_list_outputs(x, mask, idx, val, nnz, fn);
  if (st) return st;
  REQUIRE(cap >= d, SA_ERR_INVALID_ARG, "%s: cap (%lld) must be >= d (%lld)", fn,
          (long long)cap, (long long)d);
  REQUIRE(isfinite(t) && t >= 0.f, SA_ERR_INVALID_ARG, "%s: t must be finite and >= 0", fn);
  return SA_OK;
}

int check_scored(const void* x, int64_t rows, int64_t d, const void* mu, const void* colnorm,
                 int n, int m, double t, const void* mask, const void* idx, const void* val,
                 const void* nnz, int64_t cap, const void* alpha) {
  const char* fn = "act_sparsify_scored";
  int st = check_rows_d(rows, d, fn);
  if (st) return st;
  st = check_list_outputs(x, mask, idx, val, nnz, fn);
  if (st) return st;
  REQUIRE(aligned(mu, 2) && aligned(colnorm, 8) && aligned(alpha, 4), SA_ERR_INVALID_ARG,
          "%s: misaligned mu, colnorm or alpha", fn);
  if (m == 0) {
    REQUIRE(isfinite(t) && t >= 0.0, SA_ERR_INVALID_ARG, "%s: t must be finite and >= 0", fn);
    REQUIRE(cap >= d, SA_ERR_INVALID_ARG, "%s: cap (%lld) must be >= d (%lld)", fn,
            (long long)cap, (long long)d);
  } else {
    REQUIRE(m == 4 || m == 8 || m == 16 || m == 32, SA_ERR_INVALID_ARG,
            "%s: m must be 0 (threshold), 4, 8, 16 or 32 (got %d)", fn, m);
    REQUIRE(n >= 1 && n <= m, SA_ERR_INVALID_ARG, "%s: n must be in [1, m] (got %d)", fn, n);
    REQUIRE(d % m == 0, SA_ERR_INVALID_ARG, "%s: d (%lld) must be a multiple of m", fn,
            (long long)d);
    REQUIRE(cap >= d / m * n, SA_ERR_INVALID_ARG, "%s: cap (%lld) must be >= d*n/m", fn,
            (long long)cap);
  }
  return SA_OK;
}

int check_topk(const void* x, int64_t rows, int64_t d, int64_t k, const void* mask,
               const void* idx, const void* val, const void* nnz, int64_t cap) {
  const char* fn = "act_sparsify_topk";
  int st = check_rows_d(rows, d, fn);
  if (st) return st;
  st = check_list_outputs(x, mask, idx, val, nnz, fn);
  if (st) return st;
  REQUIRE(k >= 0 && k <= d, SA_ERR_INVALID_ARG, "%s: k = %lld not in [0, d = %lld]", fn,
          (long long)k, (long long)d);
  REQUIRE(cap >= k && cap >= 1, SA_ERR_INVALID_ARG, "%s: cap (%lld) must be >= max(k, 1)", fn,
          (long long)cap);
  return SA_OK;
}

int check_topk_cutoff(const void* x, int64_t rows, int64_t d, int64_t k, const void* cut,
                      const char* fn) {
  int st = check_rows_d(rows, d, fn);
  if (st) return st;
  REQUIRE(x != nullptr && (cut != nullptr || rows == 0), SA_ERR_INVALID_ARG,
          "%s: x and the cutoff output must not be NULL", fn);
  REQUIRE(aligned(x, 2) && aligned(cut, 8), SA_ERR_INVALID_ARG,
          "%s: x must be 2-byte and cut 8-byte aligned", fn);
  REQUIRE(k >= 0 && k <= d, SA_ERR_INVALID_ARG, "%s: k = %lld not in [0, d = %lld]", fn,
          (long long)k, (long long)d);
  return SA_OK;
}

int check_nm(const void* x, int64_t rows, int64_t d, int n, int m, const void* mask,
             const void* val) {
  const char* fn = "act_sparsify_nm";
  REQUIRE(rows >= 0, SA_ERR_INVALID_ARG, "%s: rows must be >= 0", fn);
  REQUIRE(m == 4 || m == 8 || m == 16 || m == 32, SA_ERR_INVALID_ARG,
          "%s: m must be 4, 8, 16 or 32 (got %d)", fn, m);
  REQUIRE(n >= 1 && n <= m, SA_ERR_INVALID_ARG, "%s: n = %d not in [1, m = %d]", fn, n, m);
  REQUIRE(d >= 32 && d % 32 == 0, SA_ERR_INVALID_ARG,
          "%s: d must be a positive multiple of 32 (got %lld)", fn, (long long)d);
  REQUIRE(x != nullptr && mask != nullptr && val != nullptr, SA_ERR_INVALID_ARG,
          "%s: x, mask and val must not be NULL", fn);
  REQUIRE(aligned(x, 16), SA_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", fn);
  REQUIRE(aligned(mask, 4) && aligned(val, 2), SA_ERR_INVALID_ARG,
          "%s: mask must be 4-byte and val 2-byte aligned", fn);
  REQUIRE(rows * d / 8 <= (int64_t)0x7fffffff * 256, SA_ERR_UNSUPPORTED, "%s: too large", fn);
  return SA_OK;
}

int check_nm_shared(const void* x, int64_t rows, int64_t d, int n, int m, int tt,
                    const void* mask, const void* val) {
  const char* fn = "act_sparsify_nm_shared";
  REQUIRE(rows >= 0, SA_ERR_INVALID_ARG, "%s: rows must be >= 0", fn);
  REQUIRE(m == 4 || m == 8 || m == 16 || m == 32, SA_ERR_INVALID_ARG,
          "%s: m must be 4, 8, 16 or 32 (got %d)", fn, m);
  REQUIRE(n >= 1 && n <= m, SA_ERR_INVALID_ARG, "%s: n = %d not in [1, m = %d]", fn, n, m);
  REQUIRE(tt >= 1 && tt <= 256, SA_ERR_INVALID_ARG, "%s: tt = %d not in [1, 256]", fn, tt);
  REQUIRE(d >= 32 && d % 32 == 0, SA_ERR_INVALID_ARG,
          "%s: d must be a positive multiple of 32 (got %lld)", fn, (long long)d);
  REQUIRE(x != nullptr && mask != nullptr && val != nullptr, SA_ERR_INVALID_ARG,
          "%s: x, mask and val must not be NULL", fn);
  REQUIRE(aligned(x, 16), SA_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", fn);
  REQUIRE(aligned(mask, 4) && aligned(val, 2), SA_ERR_INVALID_ARG,
          "%s: mask must be 4-byte and val 2-byte aligned", fn);
  REQUIRE(d <= (int64_t)65535 * 64, SA_ERR_UNSUPPORTED, "%s: d too large", fn);
  return SA_OK;
}

int check_calibrate(const void* samples, int64_t n, double s, const void* t_out) {
  const char* fn = "act_calibrate_threshold";
  REQUIRE(samples != nullptr && t_out != nullptr, SA_ERR_INVALID_ARG,
          "%s: samples and t_out must not be NULL", fn);
  REQUIRE(n >= 1 && n <= 0x7fffffffLL, SA_ERR_INVALID_ARG, "%s: n = %lld out of range", fn,
          (long long)n);
  REQUIRE(s >= 0.0 && s <= 1.0, SA_ERR_INVALID_ARG, "%s: s must be in [0, 1]", fn);
  REQUIRE(aligned(samples, 2) && aligned(t_out, 4), SA_ERR_INVALID_ARG,
          "%s: misaligned pointer", fn);
  return SA_OK;
}

int check_gemv_common(const void* wt, int64_t d_out, int64_t d_in, int64_t batch,
                      const void* y, const void* ws, size_t ws_bytes, size_t need_ws) {
  REQUIRE(wt != nullptr && y != nullptr, SA_ERR_INVALID_ARG, "gemv: wt and y must not be NULL");
  REQUIRE(d_out >= 8 && d_out % 8 == 0, SA_ERR_INVALID_ARG,
          "gemv: d_out must be a positive multiple of 8 (got %lld)", (long long)d_out);
  REQUIRE(d_out <= kMaxDOut, SA_ERR_UNSUPPORTED, "gemv: d_out = %lld exceeds %lld",
          (long long)d_out, (long long)kMaxDOut);
  REQUIRE(d_in >= 1 && d_in <= kMaxDIn, SA_ERR_INVALID_ARG, "gemv: d_in = %lld out of range",
          (long long)d_in);
  REQUIRE(batch >= 0 && batch <= SA_MAX_BATCH, SA_ERR_INVALID_ARG,
          "gemv: batch = %lld not in [0, %d]", (long long)batch, SA_MAX_BATCH);
  REQUIRE(aligned(wt, 16) && aligned(y, 16), SA_ERR_INVALID_ARG,
          "gemv: wt and y must be 16-byte aligned");
  REQUIRE(ws_bytes >= need_ws && (need_ws == 0 || ws != nullptr), SA_ERR_WORKSPACE,
          "gemv: workspace of %zu bytes needed, %zu given", need_ws, ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), SA_ERR_WORKSPACE, "gemv: workspace must be 256-byte aligned");
  return SA_OK;
}

int check_rows_gemv(const void* w, int64_t d_out, int64_t d_in, int64_t batch, const void* y,
                    const char* fn) {
  REQUIRE(w != nullptr && y != nullptr, SA_ERR_INVALID_ARG, "%s: the weight and its output must not be NULL", fn);
  REQUIRE(d_out >= 1 && d_out <= kMaxDOut, SA_ERR_INVALID_ARG,
          "%s: the row-major weight's row count %lld is not in [1, %lld]", fn, (long long)d_out,
          (long long)kMaxDOut);
  REQUIRE(d_in >= 1 && d_in <= kMaxDIn, SA_ERR_INVALID_ARG, "%s: d_in = %lld out of range", fn,
          (long long)d_in);
  REQUIRE(batch >= 0 && batch <= SA_MAX_BATCH, SA_ERR_INVALID_ARG,
          "%s: batch = %lld not in [0, %d]", fn, (long long)batch, SA_MAX_BATCH);
  REQUIRE(aligned(w, 2) && aligned(y, 2), SA_ERR_INVALID_ARG,
          "%s: the row-major weight and its output must be 2-byte aligned", fn);
  return SA_OK;
}

int check_sparse_gemv(const void* idx, const void* val, const void* nnz, int64_t batch,
                      int64_t cap) {
  (void)batch;
  REQUIRE(idx != nullptr && val != nullptr && nnz != nullptr, SA_ERR_INVALID_ARG,
          "sparse_gemv: idx, val and nnz must not be NULL");
  REQUIRE(cap >= 1, SA_ERR_INVALID_ARG, "sparse_gemv: cap must be >= 1");
  REQUIRE(aligned(idx, 4) && aligned(nnz, 4) && aligned(val, 2), SA_ERR_INVALID_ARG,
          "sparse_gemv: misaligned idx, val or nnz");
  return SA_OK;
}

int check_noalloc_size(size_t need, size_t have) {
  REQUIRE(need <= have, SA_ERR_UNSUPPORTED,
          "sparse_gemv_threshold_noalloc: this shape needs %zu bytes of scratch, more than "
          "the fixed %zu; use sparse_gemv_threshold with a workspace",
          need, have);
  return SA_OK;
}

int check_activation(const void* x, const char* name) {
  REQUIRE(x != nullptr, SA_ERR_INVALID_ARG, "%s must not be NULL", name);
  REQUIRE(aligned(x, 2), SA_ERR_INVALID_ARG, "%s must be 2-byte aligned", name);
  return SA_OK;
}

int check_threshold_value(float t) {
  REQUIRE(isfinite(t) && t >= 0.f, SA_ERR_INVALID_ARG, "t must be finite and >= 0");
  return SA_OK;
}

int check_swiglu(const void* g, const void* u, const void* colnorm, int64_t d_ff, double t,
                 int mode) {
  const char* fn = "masked_swiglu_down";
  REQUIRE(mode == 0 || mode == 1, SA_ERR_INVALID_ARG, "%s: mode must be 0 (CATS) or 1 (RaNA)",
          fn);
  REQUIRE(g != nullptr && u != nullptr, SA_ERR_INVALID_ARG, "%s: g and u must not be NULL", fn);
  REQUIRE(mode == 0 || colnorm != nullptr, SA_ERR_INVALID_ARG,
          "%s: colnorm is required for RaNA (mode 1)", fn);
  REQUIRE(aligned(g, 2) && aligned(u, 2) && aligned(colnorm, 8), SA_ERR_INVALID_ARG,
          "%s: misaligned g, u or colnorm", fn);
  REQUIRE(d_ff >= 1, SA_ERR_INVALID_ARG, "%s: d_ff must be >= 1", fn);
  REQUIRE(isfinite(t) && t >= 0.0, SA_ERR_INVALID_ARG, "%s: t must be finite and >= 0", fn);
  return SA_OK;
}

int check_col_norms(const void* wt, int64_t d_in, int64_t d_out, const void* out) {
  const char* fn = "weight_col_norms";
  REQUIRE(wt != nullptr && out != nullptr, SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  REQUIRE(d_in >= 0 && d_out >= 8 && d_out % 8 == 0, SA_ERR_INVALID_ARG,
          "%s: d_out must be a positive multiple of 8", fn);
  REQUIRE(aligned(wt, 16) && aligned(out, 8), SA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  REQUIRE(d_in <= (int64_t)0x7fffffff * 4, SA_ERR_UNSUPPORTED, "%s: d_in too large", fn);
  return SA_OK;
}

int check_nm_spmm(const void* xval, const void* mask, int64_t T, int64_t d_in, int n, int m,
                  const void* wt, int64_t d_out, const void* y) {
  const char* fn = "nm_act_spmm";
  REQUIRE(T >= 0, SA_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  REQUIRE(m == 4 || m == 8 || m == 16 || m == 32, SA_ERR_INVALID_ARG,
          "%s: m must be 4, 8, 16 or 32", fn);
  REQUIRE(n >= 1 && n <= m, SA_ERR_INVALID_ARG, "%s: n not in [1, m]", fn);
  REQUIRE(d_in >= 32 && d_in % 32 == 0, SA_ERR_INVALID_ARG,
          "%s: d_in must be a positive multiple of 32", fn);
  REQUIRE(d_out >= 8 && d_out % 8 == 0, SA_ERR_INVALID_ARG,
          "%s: d_out must be a positive multiple of 8", fn);
  REQUIRE(xval && mask && wt && y, SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  REQUIRE(aligned(wt, 16) && aligned(y, 16) && aligned(mask, 4) && aligned(xval, 16),
          SA_ERR_INVALID_ARG, "%s: wt, y and xval must be 16-byte aligned, mask 4-byte", fn);
  return SA_OK;
}

int check_nm_shared_spmm(const void* xval, const void* mask, int64_t T, int64_t d_in, int n,
                         int m, int tt, const void* wt, int64_t d_out, const void* y) {
  const char* fn = "nm_shared_spmm";
  REQUIRE(tt >= 1 && tt <= 256, SA_ERR_INVALID_ARG, "%s: tt = %d not in [1, 256]", fn, tt);
  REQUIRE(T >= 0, SA_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  REQUIRE(m == 4 || m == 8 || m == 16 || m == 32, SA_ERR_INVALID_ARG,
          "%s: m must be 4, 8, 16 or 32", fn);
  REQUIRE(n >= 1 && n <= m, SA_ERR_INVALID_ARG, "%s: n not in [1, m]", fn);
  REQUIRE(d_in >= 32 && d_in % 32 == 0, SA_ERR_INVALID_ARG,
          "%s: d_in must be a positive multiple of 32", fn);
  REQUIRE(d_out >= 8 && d_out % 8 == 0, SA_ERR_INVALID_ARG,
          "%s: d_out must be a positive multiple of 8", fn);
  REQUIRE(xval && mask && wt && y, SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  REQUIRE(aligned(wt, 16) && aligned(y, 16) && aligned(mask, 4) && aligned(xval, 16),
          SA_ERR_INVALID_ARG, "%s: wt, y and xval must be 16-byte aligned, mask 4-byte", fn);
  return SA_OK;
}

int check_dense_gemm(const void* x, int64_t T, int64_t d_in, const void* wt, int64_t d_out,
                     const void* y) {
  const char* fn = "dense_gemm";
  REQUIRE(T >= 0, SA_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  REQUIRE(d_in >= 8 && d_in % 8 == 0, SA_ERR_INVALID_ARG,
          "%s: d_in must be a positive multiple of 8", fn);
  REQUIRE(d_out >= 8 && d_out % 8 == 0, SA_ERR_INVALID_ARG,
          "%s: d_out must be a positive multiple of 8", fn);
  REQUIRE(x && wt && y, SA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  REQUIRE(aligned(x, 16) && aligned(wt, 16) && aligned(y, 16), SA_ERR_INVALID_ARG,
          "%s: x, wt and y must be 16-byte aligned", fn);
  return SA_OK;
}

}  // namespace sa
