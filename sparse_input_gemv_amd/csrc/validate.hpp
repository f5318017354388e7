// Host-side argument checks behind every C entry point.  Plain C++ (no HIP),
// so a failing check never touches the runtime.  Each check returns an SA_*
// status and records a message for sa_last_error() on the calling thread.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sa {

void clear_error();
void set_error(const char* fmt, ...);
const char* last_error();

constexpr int64_t kMaxD = 65536;            // sparsifier row length
constexpr int64_t kMaxDOut = 524288;        // GEMV output length (sizes the hand-off counters)
constexpr int64_t kMaxDIn = (int64_t)1 << 30;

int check_threshold(const void* x, int64_t rows, int64_t d, float t, const void* mask,
                    const void* idx, const void* val, const void* nnz, int64_t cap);
int check_scored(const void* x, int64_t rows, int64_t d, const void* mu, const void* colnorm,
                 int n, int m, double t, const void* mask, const void* idx, const void* val,
                 const void* nnz, int64_t cap, const void* alpha);
int check_topk_cutoff(const void* x, int64_t rows, int64_t d, int64_t k, const void* cut,
                      const char* fn);
int check_topk(const void* x, int64_t rows, int64_t d, int64_t k, const void* mask,
               const void* idx, const void* val, const void* nnz, int64_t cap);
int check_nm(const void* x, int64_t rows, int64_t d, int n, int m, const void* mask,
             const void* val);
int check_nm_shared(const void* x, int64_t rows, int64_t d, int n, int m, int tt,
                    const void* mask, const void* val);
int check_calibrate(const void* samples, int64_t n, double s, const void* t_out);

// GEMV family.  `need_ws` is the workspace the call requires.
int check_gemv_common(const void* wt, int64_t d_out, int64_t d_in, int64_t batch,
                      const void* y, const void* ws, size_t ws_bytes, size_t need_ws);
// A dense GEMV on a row-major weight [d_out][d_in] (no workspace).
int check_rows_gemv(const void* w, int64_t d_out, int64_t d_in, int64_t batch, const void* y,
                    const char* fn);
int check_sparse_gemv(const void* idx, const void* val, const void* nnz, int64_t batch,
                      int64_t cap);
int check_activation(const void* x, const char* name);
int check_noalloc_size(size_t need, size_t have);
int check_threshold_value(float t);
int check_swiglu(const void* g, const void* u, const void* colnorm, int64_t d_ff, double t,
                 int mode);
int check_col_norms(const void* wt, int64_t d_in, int64_t d_out, const void* out);
int check_nm_spmm(const void* xval, const void* mask, int64_t T, int64_t d_in, int n, int m,
                  const void* wt, int64_t d_out, const void* y);
int check_nm_shared_spmm(const void* xval, const void* mask, int64_t T, int64_t d_in, int n,
                         int m, int tt, const void* wt, int64_t d_out, const void* y);
int check_dense_gemm(const void* x, int64_t T, int64_t d_in, const void* wt, int64_t d_out,
                     const void* y);

}  // namespace sa
