/*
 * sparse_act.h -- C ABI of libsparse_act.so: activation-sparse linear layers
 * on AMD Instinct MI355X (gfx950).
 *
 * The hot path shared by TEAL, Q-Sparse, CATS/RaNA and N:M activation
 * sparsity: choose the surviving entries of an activation by magnitude, then
 * multiply only the weight columns of those entries.
 *
 * Conventions for every function below
 * ------------------------------------
 * - Pointers are DEVICE pointers owned by the caller unless stated otherwise.
 *   The library allocates nothing; scratch space comes in through `ws`.
 * - fp16 data is passed as uint16_t (IEEE binary16 bit patterns).
 * - Weights are stored transposed: WT[d_in][d_out] row-major, i.e. W
 *   column-major, so the weight column multiplied by activation entry k is
 *   the contiguous run WT + k*d_out of 2*d_out bytes.
 * - Activations are row-major [rows][d].  Bitmasks are uint32 words
 *   [rows][ceil(d/32)], bit j of word w <-> entry 32*w + j, padding bits 0.
 * - Index lists are int32, ascending, rows of length `cap`.
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call enqueues
 *   its work and returns; outputs are valid once the stream has reached the
 *   call.  Nothing blocks the host and nothing is copied to the host.
 * - Accumulation is fp32; fp16 outputs are rounded to nearest even.
 * - Return value is a status code (SA_OK on success).  Argument errors are
 *   detected on the host before any HIP call and leave outputs untouched;
 *   sa_last_error() then describes the first failing check for the calling
 *   thread.  No C++ exception crosses this boundary.
 * - A workspace `ws` (sized by sparse_gemv_workspace_bytes, 256-byte
 *   aligned) holds per-call partial sums and, in its first
 *   SA_WS_TICKET_BYTES (= sa_workspace_zero_bytes()), one arrival counter
 *   per output tile for the one-launch split-K hand-off.  That region must
 *   be all zero before the workspace is first used (allocate it
 *   zero-filled); every call leaves it zero again.  The rest may hold
 *   anything on entry.  Calls that share one workspace must be ordered on
 *   one stream: concurrent calls race.
 * - rows == 0 (or batch == 0, T == 0) is a valid empty call and does nothing.
 *
 * Pages cited (by title; "replies" = the authors' answers to reviewers):
 *   [QS]   Q-Sparse: All Large Language Models can be Fully
 *          Sparsely-Activated (replies)
 *   [TEAL] TEAL: Training-Free Activation Sparsity in Large Language Models
 *          (README)
 *   [RaNA] Adaptive Rank Allocation: Speeding Up Modern Transformers with
 *          RaNA Adapters (replies)
 *   [NM]   Motivating Next-Gen Accelerators with Flexible (N:M) Activation
 *          Sparsity via Benchmarking Lightweight Post-Training
 *          Sparsification Approaches (summary)
 */
#ifndef SPARSE_ACT_H
#define SPARSE_ACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status ------------------------------------------------------------ */
#define SA_OK 0
#define SA_ERR_INVALID_ARG 1 /* a pointer, size, alignment or value check failed */
#define SA_ERR_UNSUPPORTED 2 /* valid but outside what the kernels implement */
#define SA_ERR_WORKSPACE 3   /* ws is NULL or smaller than sa_workspace_bytes() */

/* Leading workspace bytes that must be zero before first use (see above). */
#define SA_WS_TICKET_BYTES ((size_t)1 << 20)
#define SA_ERR_HIP 4         /* the HIP runtime reported an error at launch */

#define SA_MAX_BATCH 8       /* rows per call of the GEMV family */

/* Static string naming a status code. */
const char* sa_status_string(int status);
/* Detail of the last failing call on the calling thread ("" if none). */
const char* sa_last_error(void);
/* ABI version (major*100 + minor). */
int sa_version(void);

/* ---- sparsifiers ---------------------------------------------------------- */

/*
 * act_sparsify_threshold -- per-tensor magnitude threshold.
 * [TEAL] Abstract: hidden-state entries are zeroed by magnitude with a
 * calibrated threshold; the comparator is >=, as in the CATS/RaNA masks
 * ([RaNA] Q3).  keep_i = (|x_i| >= t) && (x_i != 0), so nnz equals the number
 * of nonzeros of the sparsified row and the sparsity is 1 - nnz/d ([QS]
 * answer defining activation sparsity).
 *
 *   x     [rows][d] fp16            t    fp32 threshold, finite, >= 0
 *   mask  [rows][ceil(d/32)] or NULL
 *   idx   [rows][cap] int32: kept indices, ascending (first nnz valid)
 *   val   [rows][cap] fp16:  x at those indices
 *   nnz   [rows] int32
 * Requires d >= 1, cap >= d, d <= 65536.  x must be 2-byte aligned.
 */
int act_sparsify_threshold(const uint16_t* x, int64_t rows, int64_t d, float t,
                           uint32_t* mask, int32_t* idx, uint16_t* val,
                           int32_t* nnz, int64_t cap, void* stream);

/*
 * act_sparsify_topk -- per-token Top-K by magnitude.
 * [QS] answer comparing with MoE: per token, entries of smaller magnitude are
 * pruned.  Exactly k entries survive per row: the k largest |x|, ties to the
 * lower index (fp16 magnitudes compared exactly; -0 == +0).  Outputs as for
 * act_sparsify_threshold with nnz[r] = k.
 * Requires 0 <= k <= d, cap >= max(k,1), 1 <= d <= 65536.
 */
int act_sparsify_topk(const uint16_t* x, int64_t rows, int64_t d, int64_t k,
                      uint32_t* mask, int32_t* idx, uint16_t* val,
                      int32_t* nnz, int64_t cap, void* stream);

/*
 * act_topk_cutoff -- the per-token Top-K selection of act_sparsify_topk as
 * a cutoff instead of lists: per row the pair (tau, i*) such that entry i
 * survives iff its magnitude key (fp16 bits & 0x7fff) is > tau, or == tau
 * and i <= i*.  tau is the k-th largest key and i* the index of the last
 * surviving entry with that key (ties go to the lower index); k = 0 gives
 * tau = 32768, i* = -1 (nothing survives).
 *   cut [rows][2] int32 (device), 8-byte aligned
 * Requires 0 <= k <= d, 1 <= d <= 65536.
 */
int act_topk_cutoff(const uint16_t* x, int64_t rows, int64_t d, int64_t k, int32_t* cut,
                    void* stream);

/*
 * act_sparsify_nm -- N:M activation sparsity.
 * [QS] answer on batched inference (Block Q-Sparse): N:M over M consecutive
 * entries; [NM] section 2 (methodology): N nonzeros kept per block of M,
 * scored by |activation|.  Per aligned group of m entries of each row the n
 * largest |x| survive, ties to the lower position.
 *
 *   x     [rows][d] fp16, 16-byte aligned
 *   mask  [rows][d/32]: exactly n bits set per group
 *   val   [rows][d*n/m] fp16: kept values, group by group, in position order
 * Requires m in {4,8,16,32}, 1 <= n <= m, d % 32 == 0, d >= 32.
 */
int act_sparsify_nm(const uint16_t* x, int64_t rows, int64_t d, int n, int m,
                    uint32_t* mask, uint16_t* val, void* stream);

/*
 * act_sparsify_nm_shared -- tile-shared (vector-wise) N:M sparsity.
 * [QS] answer on batched inference: the batched N:M kernel timed there is
 * nmSPARSE's VW32 form, one N:M pattern shared by a vector of 32.  The page
 * gives no rule for a shared pattern; here, per tile of tt consecutive rows
 * (the last tile holds the rest) and per aligned group of m positions, the
 * n positions with the largest sum of the tile's |x| are kept, ties to the
 * lower position.  The sum is exact (fp64 over at most 256 fp16
 * magnitudes), so the masks are exact.
 *
 *   x     [rows][d] fp16, 16-byte aligned
 *   mask  [ceil(rows/tt)][d/32]: one mask row per tile, n bits per group
 *   val   [rows][d*n/m] fp16: each row's values at its tile's kept
 *         positions, in position order
 * Requires m in {4,8,16,32}, 1 <= n <= m, 1 <= tt <= 256, d % 32 == 0,
 * d >= 32.  Inputs are finite.
 */
int act_sparsify_nm_shared(const uint16_t* x, int64_t rows, int64_t d, int n, int m,
                           int tt, uint32_t* mask, uint16_t* val, void* stream);

/*
 * act_sparsify_scored -- weight-aware selection with a static shift and the
 * variance-correction scale.  [NM] section 2 (methodology): entries scored
 * by the size of the weight they multiply (WT, Amber-Pruner), static
 * per-token shifts that centre activations (S-PTS), a variance correction
 * after sparsification that restores the output scale (VAR); section 3 names
 * S-PTS and VAR the strongest light corrections.  The page gives no
 * formulas; per row and entry this computes
 *   x' = fp16(fp32(x) - fp32(mu))          (mu NULL: x' = x)
 *   score = |x'| * colnorm in fp64        (colnorm NULL: |x'|)
 *   m == 0: keep iff score >= t and x' != 0
 *   m  > 0: keep the n largest scores of every m consecutive entries, ties
 *           to the lower index (exactly n per group)
 *   alpha = sqrt(sum x'^2 / sum_kept x'^2), 1 when nothing is kept
 * and writes the kept x' as lists (ascending, as act_sparsify_threshold).
 * The corrected output is then sparse_gemv_corrected with alpha and the
 * shift's product W mu as the bias.
 *
 *   x       [rows][d] fp16; mu [d] fp16 or NULL; colnorm [d] fp64 or NULL
 *           (weight_col_norms gives ||W[:, i]||)
 *   mask    [rows][ceil(d/32)] uint32 or NULL; idx [rows][cap] int32;
 *           val [rows][cap] fp16 (the shifted values); nnz [rows] int32
 *   alpha   [rows] fp32 or NULL
 * Requires t finite >= 0 and cap >= d when m == 0; m in {4,8,16,32},
 * 1 <= n <= m, d % m == 0 and cap >= d*n/m otherwise.
 * Entries of idx and val past nnz are undefined afterwards: for m == 0 and
 * 4096 <= d <= 65536 the call stages intermediate results at the head of
 * each row's idx and val before writing the lists there.
 */
int act_sparsify_scored(const uint16_t* x, int64_t rows, int64_t d, const uint16_t* mu,
                        const double* colnorm, int n, int m, double t, uint32_t* mask,
                        int32_t* idx, uint16_t* val, int32_t* nnz, int64_t cap, float* alpha,
                        void* stream);

/*
 * act_calibrate_threshold -- threshold for a target sparsity from samples.
 * [TEAL] Inference Usage and Accuracy Usage step 1: thresholds come from
 * per-layer activation histograms.  The histogram here has one bin per fp16
 * magnitude, so the result is the exact linearly interpolated s-quantile of
 * |samples|: with the magnitudes sorted v_0 <= ... <= v_{n-1}, h = (n-1)s,
 * lo = floor(h), t = v_lo + (h - lo)(v_{lo+1} - v_lo) in fp64, rounded to fp32.
 *
 *   samples [n] fp16 (device)    s in [0,1]    t_out: one fp32 (device)
 * Requires 1 <= n <= 2^31 - 1.  NaN samples are outside the contract.
 */
int act_calibrate_threshold(const uint16_t* samples, int64_t n, double s,
                            float* t_out, void* stream);

/* ---- sparse-input GEMV family ------------------------------------------- */

/*
 * Bytes of workspace needed by the GEMV family (sparse_gemv,
 * sparse_gemv_threshold, sparse_gemv_corrected, sparse_gemv_scored,
 * masked_gemv, dense_gemv, masked_swiglu_down, rana_adapter_gemv) for an
 * output length d_out, input length d_in and up to `batch` rows (batch is
 * clamped to 1..SA_MAX_BATCH); 0 for d_out or d_in < 1.  The same size
 * serves every call whose sizes do not exceed these.
 * sparse_gemv_workspace_bytes is the name the hot-path contract uses;
 * sa_workspace_bytes is the same function.
 */
size_t sparse_gemv_workspace_bytes(int64_t d_out, int64_t d_in, int64_t batch);
size_t sa_workspace_bytes(int64_t d_out, int64_t d_in, int64_t batch);
/*
 * Leading bytes of that workspace that must be zero before a call and that
 * every call leaves zero: the hand-off counters, SA_WS_TICKET_BYTES for
 * every size (the arguments are accepted for symmetry).
 */
size_t sa_workspace_zero_bytes(int64_t d_out, int64_t d_in, int64_t batch);

/*
 * sparse_gemv -- y[b] = sum_{j < nnz[b]} W[:, idx[b][j]] * val[b][j].
 * [RaNA] Q5.1: with a sparse activation the products with the weight columns
 * of its zero entries are skipped; [QS] answer A3: the matmul costs
 * 2*d_out*nnz FLOPs.  Only the listed rows of WT are read.
 *
 *   wt  [d_in][d_out] fp16, 16-byte aligned, d_out % 8 == 0
 *   idx [batch][cap] int32 ascending, values in [0, d_in)
 *   val [batch][cap] fp16; nnz [batch] int32 (device), 0 <= nnz <= min(cap,d_in)
 *   y   [batch][d_out] fp16, 16-byte aligned
 * Requires 1 <= batch <= SA_MAX_BATCH.  With batch > 1 every weight row in
 * the union of the lists is read once for all rows.  Out-of-range indices or
 * counts in device memory are clamped/skipped by the kernel, never faulted.
 */
int sparse_gemv(const uint16_t* wt, int64_t d_out, int64_t d_in,
                const int32_t* idx, const uint16_t* val, const int32_t* nnz,
                int64_t batch, int64_t cap, uint16_t* y, void* ws,
                size_t ws_bytes, void* stream);

/*
 * sparse_gemv_threshold -- the threshold sparsifier and the sparse GEMV in
 * one launch: y[b] = W (keep_b .* x[b]) with keep as in
 * act_sparsify_threshold.  Each workgroup thresholds its own slice of x and
 * streams only the kept rows of WT.
 *   x [batch][d_in] fp16 (2-byte aligned); other arguments as sparse_gemv.
 */
int sparse_gemv_threshold(const uint16_t* wt, int64_t d_out, int64_t d_in,
                          const uint16_t* x, int64_t batch, float t,
                          uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * sparse_gemv_topk -- per-token Top-K and the sparse GEMV, without lists:
 * y[b] = W (keep_b .* x[b]) with keep_b the k largest |x[b]| (ties to the
 * lower index), as act_sparsify_topk keeps them ([QS] answer comparing with
 * MoE: per token, the smaller entries are pruned; answer A1: TopK =
 * 60/50/40%).  Each row's cut is the pair (tau, i*) of act_topk_cutoff;
 * the GEMV decides every entry of its own slice from x and that pair (no
 * index list is written or read).  At batch 1, where a GEMV workgroup
 * holds the row (d_in <= 16 x its threads, so at least 4096), one launch:
 * every workgroup finds the pair itself from x, in two radix passes, and
 * the GEMV runs split-K.  Otherwise two launches on `stream`:
 * act_topk_cutoff writes the pairs into the workspace, then the GEMV reads
 * them.  The two forms give the same bits wherever they run the same GEMV
 * plan (the two-launch form takes the full-K kernel for some small
 * weights).
 *   x [batch][d_in] fp16 (2-byte aligned); 0 <= k <= d_in <= 65536; other
 *   arguments as sparse_gemv_threshold.
 */
int sparse_gemv_topk(const uint16_t* wt, int64_t d_out, int64_t d_in, const uint16_t* x,
                     int64_t batch, int64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * sparse_gemv_threshold_noalloc -- sparse_gemv_threshold without a
 * workspace, for callers that cannot allocate device memory around the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments (minus ws), same kernels, same result bit for
 * bit.  Its scratch is a fixed array of SA_NOALLOC_SCRATCH_BYTES in device
 * memory, one copy per GPU the library runs on, held until the process
 * ends; the call itself allocates nothing.  Shapes whose
 * sparse_gemv_workspace_bytes(d_out, d_in, batch) exceeds that size return
 * SA_ERR_UNSUPPORTED before any launch (the Llama-2-7B projections fit at
 * batch 1: 4096 x 11008 and 4096 x 4096 also at batch 2, 11008 x 4096 at
 * batch 1 only).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race; order
 * them on one stream.
 */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int sparse_gemv_threshold_noalloc(const uint16_t* wt, int64_t d_out, int64_t d_in,
                                  const uint16_t* x, int64_t batch, float t, uint16_t* y,
                                  void* stream);

/*
 * sparse_gemv_corrected -- sparse_gemv with an output correction:
 * y[b][o] = fp16(alpha[b] * sum_j W[o][idx[b][j]] * val[b][j] + bias[o]),
 * one fp32 fused multiply-add.  alpha (fp32 [batch], e.g. the variance
 * correction of act_sparsify_scored) and bias (fp16 [d_out], e.g. W mu,
 * the static shift's product, from dense_gemv) may each be NULL.  Other
 * arguments and errors as sparse_gemv.
 */
int sparse_gemv_corrected(const uint16_t* wt, int64_t d_out, int64_t d_in,
                          const int32_t* idx, const uint16_t* val, const int32_t* nnz,
                          int64_t batch, int64_t cap, const float* alpha,
                          const uint16_t* bias, uint16_t* y, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * sparse_gemv_scored -- act_sparsify_scored (threshold kind) and
 * sparse_gemv_corrected in one launch, for one row:
 *   x' = fp16(fp32(x) - fp32(mu)), keep iff |x'| * colnorm >= t (fp64) and
 *   x' != 0, y = fp16(alpha * W (keep .* x') + bias) with alpha the variance
 *   correction sqrt(sum x'^2 / sum_kept x'^2) when var != 0 (else 1).
 * Each workgroup decides its own slice of x; the slices' sums reach the
 * workgroup that finishes each output tile with the partial tiles.
 *   x [d_in] fp16; mu [d_in] fp16 or NULL; colnorm [d_in] fp64 or NULL;
 *   bias [d_out] fp16 or NULL (e.g. W mu from dense_gemv); other arguments
 *   as sparse_gemv_threshold with batch 1.
 */
int sparse_gemv_scored(const uint16_t* wt, int64_t d_out, int64_t d_in,
                       const uint16_t* x, const uint16_t* mu, const double* colnorm,
                       double t, int var, const uint16_t* bias, uint16_t* y,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * sparse_gemv_scored_nm -- act_sparsify_scored (N:M kind) and
 * sparse_gemv_corrected in one launch, for one row (Motivating Next-Gen
 * Accelerators with Flexible (N:M) Activation Sparsity ..., section 2:
 * weight-aware scores choose the n entries of every m consecutive ones):
 *   x' = fp16(fp32(x) - fp32(mu)), score |x'| * colnorm (fp64), keep the n
 *   largest scores of every group of m (ties to the lower index; x' = 0 may
 *   be kept), y = fp16(alpha * W (keep .* x') + bias), alpha as
 *   sparse_gemv_scored.  The kept set is act_sparsify_scored's, bit for bit.
 * Each workgroup decides the groups of its own slice (slices start on
 * multiples of 32 entries, so no group spans two).
 *   m in {4, 8, 16, 32}, 1 <= n <= m, d_in % m == 0; other arguments as
 *   sparse_gemv_scored.
 * Errors: SA_ERR_INVALID_ARG for a bad n, m or d_in % m != 0, and as
 * sparse_gemv_scored otherwise.
 */
int sparse_gemv_scored_nm(const uint16_t* wt, int64_t d_out, int64_t d_in,
                          const uint16_t* x, const uint16_t* mu, const double* colnorm,
                          int n, int m, int var, const uint16_t* bias, uint16_t* y,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * rana_adapter_gemv -- the RaNA linear-layer rank adapter
 * y[b] = A (m_b .* v[b]) with v[b] = B x[b] and m_b,i = (v[b][i]^2 >= t).
 * [RaNA] Q5.1 (Eq. 11): Up, Gate and QKV projections become A (m(x) .* B x),
 * and the columns of A at the mask's zeros are skipped; Q4 (eqn. 9): the
 * masker squares B x element-wise and compares it with a threshold; Q2: one
 * plain GEMV for v = B x, one masked GEMV for A (m .* v).  Two launches on
 * `stream`: a dense GEMV on B in its own row-major layout (one wave per
 * entry of v: each is one contiguous dot product, no workspace), then the
 * masked GEMV on A^T with the mask decided per workgroup from v as stored
 * (fp16; its square is exact in fp32).
 *
 *   b  [r][d_in] fp16: B itself, row-major, 2-byte aligned (16-byte aligned
 *      with d_in % 8 == 0 and x 16-byte aligned for 16-byte loads)
 *   at [r][d_out] fp16: A^T (A is d_out x r), d_out % 8 == 0, 16-byte aligned
 *   x  [batch][d_in] fp16, 2-byte aligned
 *   t  >= 0, finite: keep entry i iff v_i^2 >= t (t = 0 keeps every entry)
 *   v  [batch][r] fp16 out, 2-byte aligned: B x (the first GEMV's output)
 *   y  [batch][d_out] fp16 out, 16-byte aligned
 *   ws workspace of at least sa_workspace_bytes(d_out, r, batch) bytes (the
 *      second GEMV's)
 * v must not overlap x or y.  With batch > 1 the rows of A in the union of
 * the rows' masks are read once for all rows.  Errors as sparse_gemv.
 */
int rana_adapter_gemv(const uint16_t* b, int64_t r, int64_t d_in,
                      const uint16_t* at, int64_t d_out, const uint16_t* x,
                      int64_t batch, float t, uint16_t* v, uint16_t* y,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * masked_gemv -- y[b] = W (mask_b .* x[b]) for a bitmask from any
 * sparsifier (the "masked GEMV" of [RaNA] Q5.1/Q7).  With batch > 1 the
 * union of the masks decides which weight rows are read.
 *   x [batch][d_in] fp16; mask [batch][ceil(d_in/32)].
 */
int masked_gemv(const uint16_t* wt, int64_t d_out, int64_t d_in,
                const uint16_t* x, const uint32_t* mask, int64_t batch,
                uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * masked_swiglu_down -- CATS / RaNA masked down projection of a SwiGLU MLP.
 * [RaNA] Q3 (Eqn. 12 for RaNA), Q5.1: with s = SiLU(g) = g/(1+exp(-g)) and
 * h = s*u,
 *   mode 0 (CATS): keep i iff |s_i| >= t
 *   mode 1 (RaNA): keep i iff |h_i| * colnorm_i >= t, colnorm_i = ||W_down[:,i]||
 * and y = sum_{kept i} W_down[:, i] h_i.  The mask decision is taken in fp64.
 *
 *   g, u    [d_ff] fp16 (gate and up projection outputs)
 *   wdt     [d_ff][d_model] fp16 = W_down transposed, 16-byte aligned
 *   colnorm [d_ff] fp64 (from weight_col_norms); may be NULL for mode 0
 *   t       fp64 threshold, finite, >= 0
 *   y       [d_model] fp16; mask [ceil(d_ff/32)] or NULL; nnz [1] or NULL
 * Requires d_model % 8 == 0.
 */
int masked_swiglu_down(const uint16_t* g, const uint16_t* u,
                       const uint16_t* wdt, const double* colnorm,
                       int64_t d_ff, int64_t d_model, double t, int mode,
                       uint16_t* y, uint32_t* mask, int32_t* nnz, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * weight_col_norms -- out[k] = ||WT[k][:]||_2 in fp64 (the norm of the weight
 * column multiplied by activation entry k; colnorm of [RaNA] Eqn. 12).
 *   wt [d_in][d_out] fp16 16-byte aligned, d_out % 8 == 0; out [d_in] fp64.
 */
int weight_col_norms(const uint16_t* wt, int64_t d_in, int64_t d_out,
                     double* out, void* stream);

/*
 * dense_gemv -- y[b] = W x[b] over every column: the dense baseline, same
 * layout and kernel skeleton as the sparse path.  Arguments as masked_gemv.
 */
int dense_gemv(const uint16_t* wt, int64_t d_out, int64_t d_in,
               const uint16_t* x, int64_t batch, uint16_t* y, void* ws,
               size_t ws_bytes, void* stream);

/* ---- batched N:M matmul ---------------------------------------------------- */

/*
 * nm_act_spmm -- Y[t] = W (mask_t .* x_t) for T tokens whose activations are
 * N:M sparse, given in the compressed form act_sparsify_nm produces.
 * [QS] answer on batched inference: N:M activation sparsity for large
 * batches, measured against a dense matmul.  Runs on MFMA; 2:4 uses the
 * gfx950 sparse MFMA.
 *
 *   xval [T][d_in*n/m] fp16;  mask [T][d_in/32] (exactly n bits per group)
 *   wt   [d_in][d_out] fp16;  y [T][d_out] fp16
 *   ws   NULL, or a device workspace of sa_nm_spmm_workspace_bytes() bytes
 *        (16-byte aligned; its contents on entry do not matter).  With it,
 *        patterns other than 2:4 take two passes -- expand the compressed
 *        values into a zero-filled dense copy in ws, then the dense MFMA
 *        engine -- which is much faster than the single pass without it.
 *        Both give the same result.
 * Requires m in {4,8,16,32}, 1 <= n <= m, d_in % 32 == 0, d_out % 8 == 0,
 * wt, y and xval 16-byte aligned.  SA_ERR_WORKSPACE if ws is too small.  A
 * mask that breaks the N:M contract gives unspecified values but never an
 * out-of-bounds access.
 */
int nm_act_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T,
                int64_t d_in, int n, int m, const uint16_t* wt, int64_t d_out,
                uint16_t* y, void* ws, size_t ws_bytes, void* stream);
/* Workspace bytes for nm_act_spmm's two-pass path (0 for 2:4, which has
 * none; 0 for invalid sizes). */
size_t sa_nm_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m);

/*
 * nm_shared_spmm -- Y[t] = W (mask_{t / tt} .* x_t): the matmul over
 * tile-shared N:M activations in act_sparsify_nm_shared's form.
 * [QS] answer on batched inference (VW32: one pattern per vector of 32, the
 * form that gives N:M savings beyond 2:4).  Three kernels, by tile size:
 *   tt a multiple of 128, n dividing 32, d_in <= 32768 and d_in n / m a
 *     multiple of 32: a whole row tile of the matmul shares one pattern, so
 *     it loads only the kept rows of WT and runs the dense MFMA matmul over
 *     the d_in n / m compressed entries: every byte and FLOP is n/m of dense;
 *   else tt a multiple of 32, n dividing 32 and m / n 2 or 4, d_in a multiple
 *     of 32 m / n: each 32-row MFMA block has one pattern; the kernel stages
 *     whole WT slabs and gathers each block's kept rows on the fly, so only
 *     the MFMA work falls to n/m of dense;
 *   else: the values are expanded into a zero-filled dense copy in ws and
 *     the dense MFMA matmul runs on it.
 * The first two need no workspace.
 *
 *   xval [T][d_in*n/m] fp16; mask [ceil(T/tt)][d_in/32]
 *   wt   [d_in][d_out] fp16;  y [T][d_out] fp16
 *   ws   device workspace of sa_nm_shared_spmm_workspace_bytes() bytes,
 *        16-byte aligned (NULL allowed when that is 0)
 * Requires m in {4,8,16,32}, 1 <= n <= m, 1 <= tt <= 256, d_in % 32 == 0,
 * d_out % 8 == 0, wt, y and xval 16-byte aligned.  SA_ERR_WORKSPACE if a
 * needed workspace is missing or too small.  A mask that breaks the N:M
 * contract gives unspecified values but never an out-of-bounds access.
 */
int nm_shared_spmm(const uint16_t* xval, const uint32_t* mask, int64_t T, int64_t d_in,
                   int n, int m, int tt, const uint16_t* wt, int64_t d_out, uint16_t* y,
                   void* ws, size_t ws_bytes, void* stream);
/* Workspace bytes nm_shared_spmm needs: 0 where one of the gathering kernels
 * applies (see above), T * d_in * 2 otherwise; 0 for invalid sizes. */
size_t sa_nm_shared_spmm_workspace_bytes(int64_t T, int64_t d_in, int n, int m, int tt);

/*
 * dense_gemm -- Y[t][o] = sum_k X[t][k] WT[k][o] (Y = X W^T) on MFMA: the
 * dense baseline of nm_act_spmm.
 *   x [T][d_in] fp16 (d_in % 8 == 0, 16-byte aligned); wt as above;
 *   y [T][d_out] fp16.
 */
int dense_gemm(const uint16_t* x, int64_t T, int64_t d_in, const uint16_t* wt,
               int64_t d_out, uint16_t* y, void* stream);

/* ---- roofline calibration ----------------------------------------------- */

/* Words of `sink` that sa_read_stream writes (one per wave of its grid). */
#define SA_READ_STREAM_SINK_WORDS 8192

/*
 * sa_read_stream -- read every byte of src once with 16-byte loads (a fixed
 * grid of 2048 x 256 threads, grid-stride) and fold it into sink, so that
 * the achievable HBM read rate can be timed beside the nominal peak.  Not
 * part of the method; bench-only.
 *   src  device, 16-byte aligned, `bytes` a positive multiple of 16
 *   sink device, SA_READ_STREAM_SINK_WORDS uint32 (contents meaningless)
 */
int sa_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream);
/*
 * sa_read_stream_grid -- the same read with a grid of `blocks` x 256 threads
 * (1 <= blocks <= 16384), for a curve of read time against bytes and grid
 * size.  sink holds blocks * 4 uint32 words.  Bench-only.
 */
int sa_read_stream_grid(const void* src, size_t bytes, uint32_t* sink, int blocks,
                        void* stream);

/* ---- tuning hook -------------------------------------------------------- */

/*
 * Process-wide launch override for the GEMV family, for tuning sweeps:
 * `tiling` picks one of the compiled tile shapes (-1 = automatic),
 * `target_wgs` the number of workgroups of the split-K stream launch to aim
 * for (0 = automatic) and `handoff` how split-K partials are summed:
 * 0 = automatic, 1 = a second launch, 2 = in the same launch by the last
 * workgroup of each output tile, with partials written through to memory,
 * 3 = the same, but with partials kept in L2 when the tile count lets every
 * slice of an output tile run on one XCD (a multiple of 8 tiles, at most 64
 * input slices; else as 2).  In form 3 the last workgroup checks where the
 * slices ran; if they ran on more than one XCD, it recomputes the other
 * slices' partials itself (same bits, much slower), so the result never
 * depends on where the hardware placed the workgroups.  Automatic takes 3
 * (or 2 where it does not apply) at batch 1; at batch 2, 3 where it applies
 * with at most 24 slices, else 1; from batch 3 on, 1 (one workgroup's final
 * sum grows with slices x rows and then costs more than a second launch).
 * Every tiling computes the same result up to fp32 summation order; the
 * hand-offs give identical bits.
 * Returns SA_ERR_INVALID_ARG for an unknown tiling or handoff.  Not
 * thread-safe.
 */
int sa_set_gemv_tuning(int tiling, int target_wgs, int handoff);
/*
 * Process-wide switches for tests of paths the automatic choices hide.
 * flags bit 0: the first input slice of every output tile reports a
 * different XCD to the L2-local hand-off's (form 3) placement check, as if
 * it had run on another XCD.  The last workgroup of every tile then takes
 * the recompute path; results are unchanged, bit for bit.
 * flags bit 1: sparse_gemv_topk always takes its two-launch form (the
 * select kernel writes the cutoff pairs, then the GEMV reads them), also
 * where its workgroups would select the cutoff themselves.
 * 0 (the default) turns both off.  Returns SA_ERR_INVALID_ARG for other
 * flags.  Not thread-safe.
 */
int sa_set_gemv_test_hooks(int flags);
/*
 * Process-wide matmul choices of dense_gemm / nm_act_spmm / nm_shared_spmm,
 * for tuning sweeps and cross-checks.
 *   tile_rows: 0 = automatic (dense: 256 x 256 tiles where their rounds
 *     over the CUs beat 256 x 128 tiles, else 256-row tiles when they give
 *     at least one workgroup per CU, else 128; 2:4: 256 x 256 tiles where
 *     their rounds stay within 1.5x their tiles per CU, else 128 x 128), or
 *     128 / 256 (128-column tiles of that height; for nm_shared_spmm with
 *     tt a multiple of 32 but not of 128, the per-32-row-block gather at that
 *     height instead of 32-row tiles).
 *   engine: 0 = automatic, 1 = the staged-register engine, 2 = the
 *     pipelined engine with 128-column tiles, 3 = the pipelined engine with
 *     256 x 256 tiles (dense, 2:4 and the expanded N:M patterns; tile_rows
 *     0 or 256; for nm_shared_spmm on 32-row tiles: 256 columns).  The
 *     pipelined engines apply when d_in is a multiple of their K step, 32
 *     for dense and the expanded N:M patterns, 64 for 2:4, with 16-byte
 *     aligned rows; other calls take the staged-register engine.
 *   stages: the pipelined engine's LDS stage count, 0 = automatic (3 for
 *     128-column tiles, 5 for dense 256 x 256, 3 for 2:4 256 x 256 and for
 *     32-row tiles), or 3..6 (loads run stages - 1 K steps ahead); a count
 *     whose stages exceed the 160 KB of LDS for the tile is lowered to the
 *     most that fit (2:4 256 x 256: always 3; 32-row tiles: 3, or 4 for any
 *     count above 3).
 * Every choice issues the same MFMA sequence per output element: identical
 * results.  Returns SA_ERR_INVALID_ARG for other values.  Not thread-safe.
 */
int sa_set_gemm_tuning(int tile_rows, int engine, int stages);
/* Describe tiling `i` (tile_o, threads, unroll); tile_o is negative for a
 * full-K tiling (one launch, no split of d_in).  Returns SA_ERR_INVALID_ARG
 * past the last one.  Output pointers are HOST pointers (may be NULL). */
int sa_gemv_tiling_info(int i, int* tile_o, int* threads, int* unroll);

/* GEMV entry points, as named by sa_gemv_plan. */
enum {
  SA_GEMV_THRESHOLD = 0, /* sparse_gemv_threshold */
  SA_GEMV_DENSE = 1,     /* dense_gemv */
  SA_GEMV_MASKED = 2,    /* masked_gemv */
  SA_GEMV_LIST = 3,      /* sparse_gemv, sparse_gemv_corrected */
  SA_GEMV_SWIGLU = 4,    /* masked_swiglu_down */
  SA_GEMV_SCORED = 6,    /* sparse_gemv_scored */
  SA_GEMV_SQUARE = 7,    /* the second GEMV of rana_adapter_gemv */
  SA_GEMV_TOPK = 8       /* the GEMV of sparse_gemv_topk */
};
/*
 * The decomposition a GEMV entry point would use for a call shape, under the
 * current sa_set_gemv_tuning choices, for inspection and performance work.
 * It computes nothing on the GPU.
 *   op: SA_GEMV_*; d_out, d_in >= 1; batch 1..SA_MAX_BATCH.
 *   cus: compute units of the device to plan for (0: the current device's).
 *   resident: workgroups of the split-K kernel that fit on one CU (0: ask
 *     the current device, which needs one).
 * Outputs (HOST pointers, none NULL):
 *   kernel: 0 split-K (k_gemv), 1 full-K (k_gemv_fk);
 *   tile_o: outputs per workgroup;
 *   grid_o: output tiles;
 *   slices: input slices per output tile (1 for full-K);
 *   handoff: 0 none (one slice or full-K), 1 a second launch sums the
 *     partials, 2 the last workgroup of a tile sums them in the same launch,
 *     3 the same with the partials kept in L2 (every slice of a tile on one
 *     XCD: grid_o a multiple of 8, or at batch 1 a grid padded up to the
 *     next multiple of 8 whose padding workgroups exit at once).
 * Returns SA_ERR_INVALID_ARG for an unknown op, a size out of range, a
 * negative count or a NULL output.
 */
int sa_gemv_plan(int op, int64_t d_out, int64_t d_in, int64_t batch, int cus, int resident,
                 int* kernel, int* tile_o, int* grid_o, int* slices, int* handoff);
/*
 * The engine and output tile a matmul call would take, under the current
 * sa_set_gemm_tuning choices, for inspection and performance work.  It
 * computes nothing on the GPU and assumes 16-byte aligned operands.
 *   op: 0 dense_gemm; 1 nm_act_spmm with pattern n:m (valid for d_in as
 *     act_sparsify_nm requires), patterns other than 2:4 given a workspace.
 *   T, d_in, d_out >= 1; cus: compute units to plan for (0: the current
 *     device's).
 * Outputs (HOST pointers, none NULL): engine 1 staged-register, 2
 * pipelined (128-column tiles), 3 pipelined 256 x 256; tile_rows x
 * tile_cols outputs per workgroup; tiles in the grid.
 * Returns SA_ERR_INVALID_ARG for an unknown op or pattern, a size out of
 * range or a NULL output.
 */
int sa_gemm_plan(int op, int64_t T, int64_t d_in, int64_t d_out, int n, int m, int cus,
                 int* engine, int* tile_rows, int* tile_cols, int64_t* tiles);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ACT_H */
