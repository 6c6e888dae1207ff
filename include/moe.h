/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts layer library.
 *
 * One MoE layer on one device's share of T tokens: router logits, softmax
 * top-k expert selection, per-expert token counting and index generation,
 * token permutation into expert-contiguous order, a grouped GEMM over all
 * experts with a SwiGLU activation between the two expert projections, the
 * weighted un-permute (combine), and the backward pass of every step.
 *
 * Sources, cited by page title and section:
 *   [Brief]   llm-wiki paper brief of arXiv 2604.00785 ("在 Aurora 超级计算机上
 *             实现大规模 MoE 语言模型的可扩展预训练").
 *   [Summary] shd-paper.top summary "Scalable Pretraining of Large Mixture of
 *             Experts Language Models on Aurora Super Computer".
 * The pages name the steps (expert selection; GPU kernels for token counting
 * and index generation; one grouped GEMM merging every expert's products;
 * optimised matmul and activation; forward plus backward) without formal
 * definitions.  The definitions used here: softmax gate over all E experts,
 * selection of the k largest logits (ties to the lower expert index), combine
 * weights = the selected probabilities (optionally renormalised), dropless
 * routing, stable token-major order inside each expert's group, expert FFN
 * SwiGLU with the gate in the first F columns of W1 and the up projection in
 * the last F.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as tensors are DEVICE pointers owned by the caller.  The
 *   library never allocates, frees or synchronises; every call enqueues work
 *   on `stream` (a hipStream_t; NULL = the null stream) and returns.
 * - Tensors are dense row-major.  Index type is int32 (T*k < 2^31).
 * - moe_dtype selects the storage of activations and weights: MOE_F32 or
 *   MOE_BF16.  Router logits, probabilities, gate weights and their
 *   gradients are always float32 unless a dtype argument says otherwise.
 *   All products accumulate in float32.
 * - Errors: every call returns moe_status.  Validation is host-side only and
 *   never reads device memory; on error nothing is enqueued and
 *   moe_last_error() returns a message (thread-local, valid until the next
 *   call on the same thread).  MOE_ERR_HIP reports a failed kernel launch.
 *   Out-of-range indices inside device buffers (expert ids, row maps, group
 *   offsets) are caller bugs.  Every kernel that reads one checks its range:
 *   an expert id is clamped into [0, E), a row outside its array is not
 *   read (zeros stand in) or not written, a group whose offsets are
 *   reversed or leave [0, M] is treated as empty.  The results for those
 *   entries are meaningless, but no access leaves its buffer, and the kernel
 *   records the event for moe_index_errors().  Row maps (dest, src) should
 *   come from moe_count_index.
 * - Weight layouts: router wr[d, E]; expert W1[E, d, 2F] (columns [0, F) gate,
 *   [F, 2F) up); expert W2[E, F, d].
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, k > E, ...  */
  MOE_ERR_UNSUPPORTED = 2, /* dtype or shape outside what the kernels take  */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
  MOE_ERR_HIP = 4          /* a HIP launch failed                           */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef void* moe_stream_t; /* hipStream_t */

/* Maximum sizes accepted by the routing kernels. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/*
 * moe_index_errors -- which range checks on device-side indices have failed
 * since the record was last cleared.  The pages define no error handling;
 * this is the debugging aid for the index-range convention above.
 * *mask receives an OR of:
 *   MOE_IDXERR_EXPERT  an expert id outside [0, E): forced ids
 *                      (moe_route_topk), topk_idx (moe_route_topk_bwd,
 *                      moe_count_index and its no-alloc variant).
 *   MOE_IDXERR_ROW     a dest entry outside [0, T*k): moe_permute,
 *                      moe_unpermute, moe_unpermute_bwd; a src entry
 *                      outside [0, n): moe_gather_scale.
 *   MOE_IDXERR_GROUP   a group with offsets[e] > offsets[e+1], or outside
 *                      [0, M]: every grouped-GEMM entry point.
 *   MOE_IDXERR_GATHER  a row-map entry outside [0, phys * div): the
 *                      *_gather GEMM entry points.
 * The record lives on the device (one per GPU, the current device is read)
 * and every kernel of the library ORs into it.  The call enqueues a copy of
 * it on `stream` and WAITS for that stream -- the one call of the library
 * that synchronises; use it in tests and debugging, not in a hot loop.  With
 * clear != 0 the record is then reset to 0.  Kernels still running on other
 * streams may add bits at any time.
 */
#define MOE_IDXERR_EXPERT 1u
#define MOE_IDXERR_ROW 2u
#define MOE_IDXERR_GROUP 4u
#define MOE_IDXERR_GATHER 8u
moe_status moe_index_errors(unsigned int* mask, int clear, moe_stream_t stream);

/*
 * moe_route_topk -- expert selection [Summary, Method details / technical
 * framework: the forward pass selects experts, then computes them].
 *
 * Per token t: z[t, e] = logits[t, e] + bias[e] (float32 add; bias may be
 * NULL), p = softmax(z[t, :]) over all E experts.  Without forced_idx, slot j
 * receives the expert with the j-th largest z (equal values: lower expert
 * index first).  With forced_idx ([T, k] int32, k distinct ids in [0, E) per
 * token) the ids are copied as given (forced uniform routing, [Brief,
 * Limitations]).  topk_w[t, j] = p[t, topk_idx[t, j]], divided by
 * sum_j p[t, topk_idx[t, j]] when renorm != 0.
 *   logits   [T, E] float32, in.        bias [E] float32 or NULL, in.
 *   topk_idx [T, k] int32, out.         topk_w [T, k] float32, out.
 *   probs    [T, E] float32 or NULL, out (p, kept for the backward pass).
 * Requires 1 <= k <= min(E, 32), 1 <= E <= 1024, T >= 1.
 * NaN scores rank below every number (-inf included) and among themselves by
 * expert index, so every token gets k distinct ids in [0, E) even when its
 * logits hold NaNs (the order of a stable descending sort with NaNs last);
 * the weights of such a token are then NaN.
 */
moe_status moe_route_topk(const float* logits, const float* bias, int T, int E,
                          int k, int renorm, const int32_t* forced_idx,
                          int32_t* topk_idx, float* topk_w, float* probs,
                          moe_stream_t stream);

/*
 * moe_route_topk_bwd -- gradient of the routing weights with respect to the
 * logits [Brief, Key results: the sped-up unit is forward plus backward].
 *
 * dp[t, e] = dw[t, j] if e == topk_idx[t, j] else 0 (with renorm:
 * dp_j = (dw_j - sum_l dw_l w_l) / S, S = sum_j p_j);
 * dlogits[t, e] = p[t, e] * (dp[t, e] - sum_e' p[t, e'] dp[t, e']).
 *   probs [T, E] float32, in (from moe_route_topk).
 *   topk_idx [T, k] int32, in.          dtopk_w [T, k] float32, in.
 *   dlogits [T, E] out, stored as dlogits_dtype (float32 or bf16).
 */
moe_status moe_route_topk_bwd(const float* probs, const int32_t* topk_idx,
                              const float* dtopk_w, int T, int E, int k,
                              int renorm, void* dlogits, moe_dtype dlogits_dtype,
                              moe_stream_t stream);

/*
 * moe_count_index -- token counting and index generation [Brief, Core
 * method: GPU kernels count the tokens of each expert and generate the
 * indices that feed the grouped GEMM].
 *
 * Flat slot s = t*k + j has expert topk_idx[s].
 *   counts[e]   = number of slots with expert e                 (int32 [E])
 *   offsets[e]  = sum_{e' < e} counts[e'], offsets[E] = T*k      (int32 [E+1])
 *   src[p]      = slot held by row p of the expert-sorted order; inside an
 *                 expert's rows [offsets[e], offsets[e+1]) slots increase
 *                 (stable order)                                  (int32 [T*k])
 *   dest[s]     = row of slot s (inverse of src)                 (int32 [T*k])
 * Deterministic: built from scans, not from atomically claimed slots.
 * ws: device workspace of at least moe_count_index_workspace_size(T, k, E)
 * bytes, 16-byte aligned.
 */
size_t moe_count_index_workspace_size(int T, int k, int E);
moe_status moe_count_index(const int32_t* topk_idx, int T, int k, int E,
                           int32_t* counts, int32_t* offsets, int32_t* dest,
                           int32_t* src, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/*
 * moe_count_index_noalloc -- moe_count_index for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and the same results,
 * with the block tables in a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * per GPU (held from the first call on a device until the process ends)
 * instead of a caller workspace.  It calls no allocating routine.
 * Limit: moe_count_index_workspace_size(T, k, E) <= MOE_NOALLOC_SCRATCH_BYTES
 * (e.g. T*k <= 1 Mi slots at E = 256, 256 Ki slots at E = 1024); larger
 * shapes return MOE_ERR_UNSUPPORTED.  Every word of the array is written
 * before it is read, so nothing is cleared between calls.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results; calls ordered on
 * one stream are safe.  Other arguments and errors as moe_count_index.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_count_index_noalloc(const int32_t* topk_idx, int T, int k, int E,
                                   int32_t* counts, int32_t* offsets,
                                   int32_t* dest, int32_t* src,
                                   moe_stream_t stream);

/*
 * moe_permute -- copy token rows into expert-contiguous order:
 * xp[dest[t*k + j], :] = x[t, :] for every slot (t, j), i.e.
 * xp[p, :] = x[src[p] / k, :].  The expert computation on the pages runs on
 * tokens grouped per expert [Brief, Core method].
 *   x [T, d], xp [T*k, d], both `dtype`.   dest [T*k] int32 from
 *   moe_count_index (a permutation of [0, T*k)).  Requires d % 8 == 0.
 *   Bitwise copy.
 */
moe_status moe_permute(const void* x, const int32_t* dest, int T, int k, int d,
                       moe_dtype dtype, void* xp, moe_stream_t stream);

/*
 * moe_unpermute -- weighted combine back to token order [Summary, Method
 * details / technical framework: experts are selected, then computed, and
 * their outputs form the layer's output for each token; Brief, Core method:
 * the expert computation runs on tokens grouped per expert, so the results
 * return to token order].  No passage defines the combination; the reading
 * used is the gate-weighted sum of the token's k expert outputs:
 * y[t, :] = sum_{j<k} w[t, j] * yp[dest[t*k + j], :], summed in float32 in
 * increasing j, rounded once to `dtype`.  With w == NULL every weight is 1
 * (this is also the backward pass of moe_permute).
 *   yp [T*k, d], y [T, d], both `dtype`.  w [T, k] float32 or NULL.
 *   Requires d % 8 == 0.
 */
moe_status moe_unpermute(const void* yp, const int32_t* dest, const float* w,
                         int T, int k, int d, moe_dtype dtype, void* y,
                         moe_stream_t stream);

/*
 * moe_unpermute_bwd -- backward of moe_unpermute [Brief, Key results: the
 * sped-up unit is the forward plus the backward pass]:
 * dyp[dest[t*k+j], :] = w[t, j] * dy[t, :]   (rounded to dtype) and
 * dw[t, j] = sum_i dy[t, i] * yp[dest[t*k+j], i]   (float32).
 *   dy [T, d], yp [T*k, d], dyp [T*k, d]: `dtype`.  w [T, k] float32, in.
 *   dw [T, k] float32, out.  Requires d % 8 == 0.
 *   dyp may be NULL: only dw is computed (the path in which GEMM 2's
 *   backward reads dy through the row map instead, see
 *   moe_grouped_gemm_bwd_scaled_gather).
 */
moe_status moe_unpermute_bwd(const void* dy, const void* yp,
                             const int32_t* dest, const float* w, int T, int k,
                             int d, moe_dtype dtype, void* dyp, float* dw,
                             moe_stream_t stream);

/*
 * Grouped GEMM -- one launch computes every expert's product [Brief, Core
 * method: the experts' matrix products are merged into a grouped GEMM;
 * Summary, Method details / key design: optimised matrix multiplication].
 *
 * Rows [offsets[e], offsets[e+1]) of the row-major operands belong to group
 * e; `offsets` (int32 [E+1], offsets[0] = 0, non-decreasing,
 * offsets[E] <= M) is read ON THE DEVICE, so no host synchronisation is
 * needed between counting and the GEMM.  M is the host-known row count.
 * A group whose range is reversed or leaves [0, M] is skipped (no rows
 * computed; zero weight gradient) and recorded (MOE_IDXERR_GROUP).
 *
 * moe_grouped_gemm_fwd:  c[rows e] = a[rows e] @ b[e]
 *   a [M, K] ab_dtype, b [E, K, N] ab_dtype, c [M, N] c_dtype.
 *   With ab_dtype == MOE_BF16, c_dtype may be MOE_BF16 or MOE_F32;
 *   with MOE_F32 inputs c_dtype must be MOE_F32.
 *   Rows outside every group are left untouched.
 *
 * moe_grouped_gemm_bwd: given dc = dL/dc,
 *   da[rows e] = dc[rows e] @ b[e]^T (+ da_add[rows e])   [M, K], dtype
 *   db[e]      = a[rows e]^T @ dc[rows e]                  [E, K, N] float32
 *   (db[e] = 0 for an empty group).  a, b, dc, da, da_add share `dtype`;
 *   da or db may be NULL to skip that product; da_add may be NULL.
 *
 * The bf16 path runs on MFMA tiles when K % 8 == 0 and N % 8 == 0; other
 * shapes and float32 run on an LDS-tiled 64x64 kernel on the float32 matrix
 * cores.  On the MFMA path every operand and result pointer must be 16-byte
 * aligned (MOE_ERR_INVALID_ARG otherwise).  ws/ws_bytes: device workspace
 * of at least moe_grouped_gemm_workspace_size() bytes, 16-byte aligned, used by
 * moe_grouped_gemm_bwd for db when the weight gradient is reduced in row
 * slices (shapes with few output tiles); MOE_ERR_WORKSPACE if it is needed
 * and missing or too small.  The size is 0 (NULL allowed) when no slicing is
 * planned; moe_grouped_gemm_fwd ignores it.
 */
size_t moe_grouped_gemm_workspace_size(int M, int K, int N, int E,
                                       moe_dtype dtype);
/*
 * moe_grouped_gemm_plan -- the kernel configuration the grouped GEMM entry
 * points choose for a shape (host-only query, enqueues nothing).
 * product: 0 = forward c (moe_grouped_gemm_fwd), 1 = da, 2 = db
 * (moe_grouped_gemm_bwd), 3 = h of moe_grouped_gemm_swiglu_fwd (N = 2F).
 * Writes the row/column tile sizes, the wavefront grid of a workgroup
 * (waves_m x waves_n), and the number of reduction slices; *mfma = 1 for
 * the bf16 MFMA kernel, 0 for the float32-MFMA kernel.  Any output pointer
 * may be NULL.
 */
moe_status moe_grouped_gemm_plan(int product, int M, int K, int N, int E,
                                 moe_dtype dtype, int* tile_m, int* tile_n,
                                 int* waves_m, int* waves_n, int* split,
                                 int* mfma);
moe_status moe_grouped_gemm_fwd(const void* a, const void* b,
                                const int32_t* offsets, int M, int K, int N,
                                int E, moe_dtype ab_dtype, void* c,
                                moe_dtype c_dtype, void* ws, size_t ws_bytes,
                                moe_stream_t stream);
moe_status moe_grouped_gemm_bwd(const void* a, const void* b, const void* dc,
                                const int32_t* offsets, int M, int K, int N,
                                int E, moe_dtype dtype, void* da,
                                const void* da_add, float* db, void* ws,
                                size_t ws_bytes, moe_stream_t stream);

/*
 * moe_grouped_gemm_swiglu_fwd -- GEMM 1 with the SwiGLU activation in its
 * epilogue [Summary, Method details / key design: optimised matrix
 * multiplication and activation function].  For the rows of every group e:
 *   h[rows e]  = a[rows e] @ b[e]                 [M, 2F], dtype
 *   act[m, f]  = silu(h[m, f]) * h[m, F + f]      [M, F],  dtype
 * a [M, K], b [E, K, 2F] with the gate columns [0, F) and the up columns
 * [F, 2F); offsets as above.  act is computed from the stored h values
 * (rounded to dtype first), so the result is the one moe_grouped_gemm_fwd
 * followed by moe_act_fwd gives -- which is also what this call runs for
 * shapes and dtypes that the bf16 MFMA path does not take.  h is still
 * written because the backward pass reads it.  F must be a multiple of 8
 * (MOE_ERR_UNSUPPORTED); on the MFMA path every pointer must be 16-byte
 * aligned (MOE_ERR_INVALID_ARG).  Rows outside every group are left
 * untouched.
 */
moe_status moe_grouped_gemm_swiglu_fwd(const void* a, const void* b,
                                       const int32_t* offsets, int M, int K,
                                       int F, int E, moe_dtype dtype, void* h,
                                       void* act, moe_stream_t stream);

/*
 * Gathered-operand variants: the permutation fused into the operand loads
 * of the GEMMs that read the permuted activations [Brief, Core method: the
 * index generation feeds the grouped GEMM].  Instead of a permuted copy
 * a [M, K], they take the unpermuted array x [x_phys, K] and a row map:
 * logical row p of a is row x_rows[p] / x_div of x.  With the outputs of
 * moe_count_index, x_rows = src and x_div = k give a = xp without writing
 * it (xp[p] = x[src[p] / k]).  Results equal, bit for bit, the plain call on
 * the permuted copy.
 *
 * moe_grouped_gemm_swiglu_fwd_gather: moe_grouped_gemm_swiglu_fwd with a
 *   gathered.
 * moe_grouped_gemm_bwd_gather: moe_grouped_gemm_bwd with a gathered (only db
 *   reads a).
 *   x_rows int32 [M] device; every x_rows[p] / x_div (for the rows the
 *   groups cover) must lie in [0, x_phys) (an entry outside [0, x_phys *
 *   x_div) reads as a zero row and is recorded, MOE_IDXERR_GATHER).
 *   Requires the bf16 MFMA path
 *   (K and F, or K and N, multiples of 8) and x_phys * K < 2^30;
 *   MOE_ERR_UNSUPPORTED otherwise.  Other arguments, alignment, workspace
 *   and errors as in the plain calls.
 */
moe_status moe_grouped_gemm_swiglu_fwd_gather(const void* x, const int32_t* x_rows,
                                              int x_div, int x_phys, const void* b,
                                              const int32_t* offsets, int M, int K,
                                              int F, int E, moe_dtype dtype, void* h,
                                              void* act, moe_stream_t stream);
moe_status moe_grouped_gemm_bwd_gather(const void* a, const int32_t* a_rows,
                                       int a_div, int a_phys, const void* b,
                                       const void* dc, const int32_t* offsets,
                                       int M, int K, int N, int E, moe_dtype dtype,
                                       void* da, const void* da_add, float* db,
                                       void* ws, size_t ws_bytes,
                                       moe_stream_t stream);

/*
 * moe_gather_scale -- the gate weights in expert-sorted row order:
 * out[p] = w[src[p]] for p < n (w and src as from moe_route_topk and
 * moe_count_index, n = T*k; w read as [T*k]).  A src entry outside [0, n)
 * gives 0 and is recorded (MOE_IDXERR_ROW).  The row scale of
 * moe_grouped_gemm_bwd_scaled_gather and moe_act_bwd_scaled.
 */
moe_status moe_gather_scale(const float* w, const int32_t* src, int n, float* out,
                            moe_stream_t stream);

/*
 * moe_grouped_gemm_bwd_scaled_gather -- GEMM 2's backward without the
 * combine's gradient in memory [Brief, Core method: the grouped GEMM and
 * its index generation; Summary, Method details / key design: optimised
 * matrix multiplication].  The combine's backward would write
 * dc[p, :] = row_scale[p] * dy[dc_rows[p] / dc_div, :] (row_scale: the gate
 * weight of the slot held by row p, moe_gather_scale; dc_rows = src,
 * dc_div = k); this call reads dy through the row map instead:
 *   da[rows e] = diag(row_scale) (dy_g[rows e] @ b[e]^T)   [M, K] dtype
 *   db[e]      = a_scaled[rows e]^T @ dy_g[rows e]          [E, K, N] float32
 * with dy_g[p] = dy[dc_rows[p] / dc_div].  The scale of db sits on the
 * activation operand: the caller passes a_scaled = diag(row_scale) a
 * (moe_act_bwd_scaled writes it), which gives the same product
 * a^T diag(row_scale) dy_g.  da is the float32 product times the scale,
 * rounded once; db is float32 (zero for an empty group).
 *   a_scaled [M, K], b [E, K, N], dy [dc_phys, N], da [M, K]: `dtype`
 *   (bf16 only: the MFMA path, K and N multiples of 8, every pointer
 *   16-byte aligned).  dc_rows int32 [M]; every dc_rows[p] / dc_div for the
 *   rows the groups cover must lie in [0, dc_phys) (otherwise a zero row
 *   stands in and MOE_IDXERR_GATHER is recorded).  row_scale float32 [M].
 *   da or db may be NULL to skip that product.  Offsets, workspace and
 *   errors as in moe_grouped_gemm_bwd.
 */
moe_status moe_grouped_gemm_bwd_scaled_gather(
    const void* a_scaled, const void* b, const void* dy, const int32_t* dc_rows,
    int dc_div, int dc_phys, const float* row_scale, const int32_t* offsets,
    int M, int K, int N, int E, moe_dtype dtype, void* da, float* db, void* ws,
    size_t ws_bytes, moe_stream_t stream);

/*
 * moe_act_fwd -- SwiGLU activation [Summary, Method details / key design:
 * optimised activation]: a[m, f] = silu(h[m, f]) * h[m, F + f],
 * silu(z) = z / (1 + exp(-z)).   h [M, 2F], a [M, F], both `dtype`.
 * Requires F % 8 == 0.
 *
 * moe_act_bwd -- its gradient: with g = h[m, f], u = h[m, F+f],
 * s = sigmoid(g):  dh[m, f] = da * u * s * (1 + g (1 - s)),
 * dh[m, F+f] = da * g * s.   h, dh [M, 2F], da [M, F], all `dtype`.
 */
moe_status moe_act_fwd(const void* h, int M, int F, moe_dtype dtype, void* a,
                       moe_stream_t stream);
moe_status moe_act_bwd(const void* h, const void* da, int M, int F,
                       moe_dtype dtype, void* dh, moe_stream_t stream);

/*
 * moe_act_bwd_scaled -- moe_act_bwd, plus the activation recomputed from h
 * and scaled per row, for moe_grouped_gemm_bwd_scaled_gather:
 * a_scaled[m, f] = row_scale[m] * silu(h[m, f]) * h[m, F + f], rounded once
 * to dtype.  dh is bit for bit the result of moe_act_bwd.
 *   h, dh [M, 2F], da, a_scaled [M, F]: `dtype`.  row_scale float32 [M].
 */
moe_status moe_act_bwd_scaled(const void* h, const void* da,
                              const float* row_scale, int M, int F,
                              moe_dtype dtype, void* dh, void* a_scaled,
                              moe_stream_t stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MOE_MI355X_H */
