/*
 * sd.h -- C ABI of the MI355X (gfx950) sparse decode-step library.
 *
 * One single-sequence LLM decode step with two sparsity branches, as
 * described in "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
 * Decoding" (below: [Cross]):
 *
 *   - KV branch ([Cross] §4.1): once after prefill, score the cache with the
 *     attention of an observation window of queries, keep sinks, the window
 *     and the best-scoring entries of each KV head, and gather them into one
 *     contiguous buffer; every later step reads that buffer with the same
 *     split-K attention kernel that dense mode uses and appends its own key
 *     and value to it.
 *   - Projection branch: CATS-style activation sparsity as kept by
 *     "Sensitivity-Aware Thresholding and Token Routing for Activation
 *     Sparsification in Large Language Models" (below: [SATS]): the SiLU gate
 *     output is thresholded per layer and only the kept channels' up rows and
 *     down columns are read.
 *   - Byte account ([Cross] §3): bytes per step, savings, speedup bounds and
 *     crossover lengths from model dimensions and keep ratios.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Pointers are device pointers unless marked [host].  The caller
 *   owns every buffer; the library never allocates device memory and keeps no
 *   pointer after the call returns.  Device buffers must stay valid until the
 *   work enqueued on `stream` has finished.  Host structs are read (and, where
 *   stated, updated) only during the call.
 * Layouts.  Row-major, densely packed.  Caches are [n_kv_heads, cap, head_dim]
 *   (row j of KV head h at element (h*cap + j)*head_dim).  Weights are
 *   [out_features, in_features] (nn.Linear order) except the down projection,
 *   stored transposed as w_down_t [d_ff, d_model] so that one kept channel's
 *   down column is one contiguous row.  Activations are float32.
 * Element types.  sd_dims.w_dtype applies to all projection weights and
 *   sd_dims.kv_dtype to all cache buffers: SD_F32 or SD_BF16.  Norm vectors
 *   are float32.  Arithmetic is float32 throughout (bf16 inputs are widened).
 * Alignment.  Every device pointer must be 16-byte aligned.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  All work
 *   is asynchronous; there is no implicit synchronization.
 * Workspace.  Entry points that take (ws, ws_bytes) use it for intermediate
 *   state; size it with sd_workspace_bytes().  Its contents need no
 *   initialisation and are undefined after a call.  Calls that share one
 *   workspace must be ordered on one stream.
 * Errors.  Every argument check runs on the host before anything is enqueued;
 *   a failing call enqueues nothing and returns:
 *     SD_EINVAL        null or misaligned pointer, inconsistent sizes;
 *     SD_ENOSPC        workspace or buffer capacity too small;
 *     SD_EUNSUPPORTED  head_dim not 64 or 128, d_model or input widths not a
 *                      multiple of 8 or above 8192, unknown dtype;
 *     SD_EHIP          a HIP launch or query failed (work may be partial).
 *   sd_last_error() gives a message for the calling thread's last failure.
 *   No exception crosses the ABI and the library never aborts.
 * Threads.  Every compute entry point is reentrant and keeps no state between
 *   calls (beyond per-device launch-shape caches, filled once under a lock),
 *   with two exceptions: the opt-in kernel profiler (sd_profile_start /
 *   sd_profile_stop) keeps one process-wide recording that is not safe to
 *   drive from several threads at once, and sd_decode_step_noalloc runs on
 *   one scratch buffer per GPU, so its calls on one GPU must not overlap.
 */
#ifndef SD_H
#define SD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SD_OK = 0,
  SD_EINVAL = 1,
  SD_ENOSPC = 2,
  SD_EUNSUPPORTED = 3,
  SD_EHIP = 4
} sd_status;

enum { SD_F32 = 0, SD_BF16 = 1 };

/* flags */
enum {
  SD_SCORES_IN = 1u,  /* sd_select_kv: rank caller-given scores, skip scoring */
  SD_GATE_IN = 2u,    /* sd_sparse_mlp: mask caller-given activations, skip gate */
  SD_KV_SPARSE = 4u,  /* sd_decode_step: attend over the gathered buffer */
  SD_MLP_SPARSE = 8u, /* sd_decode_step: CATS-threshold the MLP */
  SD_KV_WINDOW = 16u, /* sd_decode_step: attend over sinks + recent rows of the full cache */
  SD_ATTN_MASKED = 32u, /* sd_decode_step: dense attention by the masked comparison path */
  SD_ATTN_FUSED = 64u,  /* sd_decode_step: dense attention by the fused (no split-K) path */
  SD_PROJ_TEAL = 128u,  /* sd_decode_step: TEAL-threshold the inputs of all seven projections */
  SD_ACCUMULATE = 256u, /* sd_teal_gemv: y += result instead of y = result */
  SD_MATRIX_CORES = 512u /* sd_decode_step_batch: projections on the matrix cores (tile weights) */
};

/* output columns per block of the TEAL weight layout (sd_teal_gemv) */
#define SD_TEAL_BLOCK 128

/* projection sets of the byte account */
enum { SD_PROJ_ALL7 = 0, SD_PROJ_FFN = 1, SD_PROJ_CATS = 2 };

typedef struct {
  int32_t d_model;     /* hidden width d */
  int32_t n_q_heads;   /* query heads h_q */
  int32_t n_kv_heads;  /* KV heads h_kv; h_q % h_kv == 0, query head h reads KV head h / (h_q/h_kv) */
  int32_t head_dim;    /* d_h: 64 or 128 */
  int32_t d_ff;        /* feed-forward width */
  int32_t w_dtype;     /* SD_F32 or SD_BF16 */
  int32_t kv_dtype;    /* SD_F32 or SD_BF16 */
  float rms_eps;       /* RMSNorm epsilon (Llama: 1e-5) */
  float rope_theta;    /* RoPE base (Llama-3: 500000); <= 0 disables RoPE */
} sd_dims;

/* Bytes of workspace that every call below needs for these dims, for caches
 * of up to max_rows rows and observation windows of up to max_window queries
 * (max_rows also sizes the score rows of the masked comparison path).
 * [host]; returns 0 on invalid dims. */
size_t sd_workspace_bytes(const sd_dims* dims, int32_t max_rows, int32_t max_window);

/*
 * sd_select_kv -- one-time attention-scored KV selection and gather
 * ([Cross] §4.1, SnapKV-style).
 *
 * k_full, v_full  [h_kv, cap_full, d_h] kv_dtype: rows 0..n-1 valid.
 * q_window        [h_q, w, d_h] float32: queries of the last w prompt tokens
 *                 (already rotated); query i sits at position n - w + i and
 *                 attends causally to rows 0..n-w+i.
 * Score of row j for KV head kv: sum over the window queries and over the
 * query heads of group kv of the softmax weight on row j (logits scaled by
 * 1/sqrt(d_h)).  Rows [0, n_sink) and [n-w, n) are always kept; the other
 * k_keep - n_sink - w kept rows are the highest scores of [n_sink, n-w), equal
 * scores ordered by lower position.
 * scores          [h_kv, n] float32: written, or read with SD_SCORES_IN (then
 *                 q_window may be NULL; scores are compared as float32,
 *                 NaN not allowed).
 * idx             [h_kv, k_eff] int32 out, ascending, k_eff = min(k_keep, n);
 *                 k_keep >= n keeps every row (keep ratio 1 disables the branch).
 * k_sel, v_sel    [h_kv, cap_sel, d_h] kv_dtype out: rows 0..k_eff-1 = the kept
 *                 rows in idx order; cap_sel >= k_eff, and later steps append
 *                 at row k_eff onwards.
 * Errors: EINVAL unless 1 <= w <= n, 0 <= n_sink, n_sink + w <= k_keep
 *         (when k_keep < n), n <= cap_full; ENOSPC if cap_sel < k_eff.
 */
sd_status sd_select_kv(const sd_dims* dims, const void* k_full, const void* v_full,
                       int32_t cap_full, int32_t n, const float* q_window, int32_t w,
                       int32_t n_sink, int32_t k_keep, float* scores, int32_t* idx,
                       void* k_sel, void* v_sel, int32_t cap_sel, uint32_t flags,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * sd_decode_attn -- split-K (flash-decoding style) GQA decode attention over
 * rows 0..n_ctx-1 of one cache, full or gathered ([Cross] §1, §4.1, §4.4:
 * one kernel serves dense and sparse modes).
 *
 * q      [h_q, d_h] float32 (already rotated).
 * k, v   [h_kv, cap, d_h] kv_dtype; n_ctx >= 1 rows read.
 * out    [h_q, d_h] float32: softmax(scale * q.K^T) V per query head.
 * lse    [h_q] float32 log-sum-exp of the scaled logits, or NULL.
 * n_splits  chunks of the row range per KV head (at most 256), 0 = chosen by
 *           the library; the result depends on it only through float32
 *           rounding.  A second launch merges the chunks in chunk order.
 * Errors: EINVAL unless 1 <= n_ctx <= cap; ENOSPC for a short workspace or
 *         n_splits above 256.
 */
sd_status sd_decode_attn(const sd_dims* dims, const float* q, const void* k, const void* v,
                         int32_t cap, int32_t n_ctx, float scale, int32_t n_splits,
                         float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * sd_select_kv_ragged -- sd_select_kv with a budget per KV head
 * ("CateKV: On Sequential Consistency for Long-Context LLM Inference
 * Acceleration", §3 "CateKV Cache Policy": consistent heads keep a small
 * fixed number of critical entries, adaptive heads a large share of theirs).
 *
 * k_keep_heads    [h_kv] int32 [host]: KV head kv keeps k_eff[kv] =
 *                 min(k_keep_heads[kv], n) rows by the rule of sd_select_kv.
 * idx             [h_kv, idx_stride] int32 out: head kv's kept rows ascending
 *                 in idx[kv*idx_stride .. kv*idx_stride + k_eff[kv] - 1]; the
 *                 rest of each row is left untouched.
 * k_sel, v_sel    [h_kv, cap_sel, d_h] out: rows 0..k_eff[kv]-1 of head kv
 *                 are its kept rows; later steps append at row k_eff[kv].
 * Everything else as sd_select_kv (same kernels, same scores, same ranking).
 * Errors: EINVAL unless each k_keep_heads[kv] >= n_sink + w (or >= n) and
 *         idx_stride >= max k_eff; ENOSPC if cap_sel < max k_eff;
 *         EUNSUPPORTED for more than 32 KV heads.
 */
sd_status sd_select_kv_ragged(const sd_dims* dims, const void* k_full, const void* v_full,
                              int32_t cap_full, int32_t n, const float* q_window, int32_t w,
                              int32_t n_sink, const int32_t* k_keep_heads, float* scores,
                              int32_t* idx, int32_t idx_stride, void* k_sel, void* v_sel,
                              int32_t cap_sel, uint32_t flags, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * sd_decode_attn_ragged -- sd_decode_attn where KV head kv reads its own
 * n_ctx_heads[kv] rows (the gathered buffers of sd_select_kv_ragged; same
 * CateKV passage).  Query heads of group kv attend over rows
 * 0..n_ctx_heads[kv]-1 of KV head kv.
 * n_ctx_heads  [h_kv] int32 [host].
 * n_splits     chunks of the longest head (at most 256); a shorter head leaves
 *              its trailing chunks empty.  0 = chosen by the library so that the
 *              rows of all heads together spread over the whole GPU.
 * Errors: EINVAL unless 1 <= n_ctx_heads[kv] <= cap for every head; ENOSPC as
 *         sd_decode_attn; EUNSUPPORTED for more than 32 KV heads.
 */
sd_status sd_decode_attn_ragged(const sd_dims* dims, const float* q, const void* k, const void* v,
                                int32_t cap, const int32_t* n_ctx_heads, float scale,
                                int32_t n_splits, float* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * sd_decode_attn_window -- attention over a sink-plus-recent window read in
 * place from one cache ([Cross] §4.1: the StreamingLLM-style policy that reads
 * as many entries as the selection keeps; §4.4 times it): of the n_rows valid
 * rows, rows [0, n_sink) and the most recent n_keep - n_sink rows, for every
 * KV head; all rows when n_keep >= n_rows.  Same kernel, outputs and n_splits
 * rule as sd_decode_attn over those rows.
 * Errors: EINVAL unless 1 <= n_rows <= cap and 0 <= n_sink <= n_keep, n_keep >= 1.
 */
sd_status sd_decode_attn_window(const sd_dims* dims, const float* q, const void* k, const void* v,
                                int32_t cap, int32_t n_rows, int32_t n_sink, int32_t n_keep,
                                float scale, int32_t n_splits, float* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * sd_decode_attn_baseline -- dense decode attention by one of the two
 * comparison paths of [Cross] §4.4, with the outputs of sd_decode_attn:
 *   SD_ATTN_MASKED  scores of every query head over every allocated row
 *                   (rows >= n_ctx masked to -inf), a row softmax, then P.V --
 *                   each query head reads its KV head's rows itself; needs the
 *                   workspace of sd_workspace_bytes(dims, cap, 0);
 *   SD_ATTN_FUSED   one pass per query head in one workgroup (online softmax,
 *                   no split-K).
 * Errors: EINVAL unless 1 <= n_ctx <= cap and path is one of the two.
 */
sd_status sd_decode_attn_baseline(const sd_dims* dims, const float* q, const void* k,
                                  const void* v, int32_t cap, int32_t n_ctx, float scale,
                                  int32_t path, float* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * sd_sparse_mlp -- CATS sparse SwiGLU MLP ([SATS], CATS runtime masking).
 *
 * x        [d] float32 input; if norm_w is not NULL it is first normalised,
 *          x_hat = x / sqrt(mean(x^2) + rms_eps) * norm_w, else x_hat = x.
 * w_gate, w_up [d_ff, d]; w_down_t [d_ff, d] (down projection transposed).
 * act      [d_ff] float32: a = SiLU(w_gate x_hat), written; with SD_GATE_IN it is
 *          read instead and the gate projection is skipped.
 * Channel i is kept iff threshold < 0 or |a_i| > threshold (strict).
 * y        [d] float32 out: sum over kept i of a_i (w_up[i] . x_hat) w_down_t[i].
 * idx      [d_ff] int32 out: the kept channels ascending in idx[0..n_kept-1].
 * n_kept   [1] int32 out (device).
 * Errors: EINVAL for bad pointers; EUNSUPPORTED for widths (see above).
 */
sd_status sd_sparse_mlp(const sd_dims* dims, const float* x, const float* norm_w,
                        const void* w_gate, const void* w_up, const void* w_down_t,
                        float threshold, float* y, float* act, int32_t* idx,
                        int32_t* n_kept, uint32_t flags, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * sd_teal_gemv -- one TEAL-sparse projection ([Cross] §3.2 "Sparse Branches",
 * §4.1 "Setup": the projection keeps only the input activation channels whose
 * magnitude clears a calibrated threshold and loads only their weights).
 *
 * x        [d_in] float32 input; if norm_w is not NULL it is first normalised,
 *          x_hat = x / sqrt(mean(x^2) + rms_eps) * norm_w, else x_hat = x.
 * Input channel j is kept iff threshold < 0 or |x_hat_j| > threshold (strict,
 * decided in float32).
 * w_t      the projection's weight W [d_out, d_in] in dims->w_dtype, stored in
 *          column blocks of SD_TEAL_BLOCK (128) outputs: element (c, j) of W at
 *          ((c / 128) d_in + j) 128 + c % 128, [ceil(d_out / 128)][d_in][128]
 *          elements (columns past d_out are padding, never written out).  A
 *          kept channel's piece of a block is one contiguous 128-element row;
 *          only kept channels' pieces are read.
 * w2_t     optional second matrix in the same layout with the same input
 *          (gate and up), its result in y2; NULL for one projection.
 * y        [d_out] float32 out: sum over kept j of x_hat_j W[:, j]; with
 *          SD_ACCUMULATE it is added to y.  Fixed summation order.  y, y2 must
 *          not overlap x.
 * idx      [d_in] int32 out or NULL: the kept channels ascending in
 *          idx[0..n_kept-1].  n_kept [1] int32 out (device) or NULL.
 * Sizes:   d_in, d_out multiples of 8; d_in <= 32768; the workspace of
 *          sd_workspace_bytes(dims, ...) covers any d_in, d_out up to the
 *          widths of dims (d_model, d_ff, n_q_heads d_h, (n_q + 2 n_kv) d_h),
 *          else ENOSPC.
 * Errors: EINVAL for bad pointers or sizes.
 */
sd_status sd_teal_gemv(const sd_dims* dims, const float* x, int32_t d_in, const float* norm_w,
                       float threshold, const void* w_t, const void* w2_t, int32_t d_out,
                       float* y, float* y2, uint32_t flags, int32_t* idx, int32_t* n_kept,
                       void* ws, size_t ws_bytes, void* stream);

/* One decoder layer's state for sd_decode_step. */
typedef struct {
  const float* attn_norm;  /* [d] */
  const void* w_qkv;       /* [(h_q + 2 h_kv) d_h, d]: q rows, then k rows, then v rows */
  const void* w_o;         /* [d, h_q d_h] */
  const float* mlp_norm;   /* [d] */
  const void* w_gate;      /* [d_ff, d] */
  const void* w_up;        /* [d_ff, d] */
  const void* w_down_t;    /* [d_ff, d] */
  float cats_threshold;    /* per-layer t; < 0 means dense even in sparse mode */
  int32_t pad0;
  void* k_full;            /* [h_kv, cap_full, d_h] */
  void* v_full;
  int32_t cap_full;
  int32_t n_full;          /* valid rows before the step; advanced by one [host] */
  void* k_sel;             /* gathered buffer [h_kv, cap_sel, d_h], or NULL */
  void* v_sel;
  int32_t cap_sel;
  int32_t n_sel;           /* valid gathered rows; advanced by one when k_sel != NULL */
  uint8_t* mask_out;       /* optional [d_ff], 16-byte aligned: receives 1 for kept channels, else 0 */
  int32_t window_keep;     /* SD_KV_WINDOW: entries read (sinks included) */
  int32_t window_sink;     /* SD_KV_WINDOW: sink entries among them */
  /* SD_PROJ_TEAL: the projections in the column-block layout of sd_teal_gemv
   * ([ceil(d_out / 128)][d_in][128]) and the four input thresholds, attention
   * input, O input, MLP input, down input (w_down_t above, or w_down_b below,
   * serves every mode) */
  const void* w_qkv_t;     /* W_qkv in column blocks: d_in = d, d_out = (h_q + 2 h_kv) d_h */
  const void* w_o_t;       /* W_o: d_in = h_q d_h, d_out = d */
  const void* w_gate_t;    /* W_gate: d_in = d, d_out = d_ff */
  const void* w_up_t;      /* W_up: d_in = d, d_out = d_ff */
  float teal_t[4];
  uint8_t* teal_masks_out; /* optional, 16-byte aligned: the four keep masks (1 kept, 0 dropped),
                              [d | h_q d_h | d | d_ff] bytes in that order */
  int32_t* n_sel_heads;    /* optional [h_kv] [host]: per-KV-head valid gathered rows (ragged
                              budgets of sd_select_kv_ragged); replaces n_sel when not NULL,
                              each entry advanced by one; excludes SD_KV_WINDOW */
  /* sd_decode_step_batch with SD_MATRIX_CORES: bf16 weights in the tile layout
   * of sd_pack_tiles (the other modes and entry points do not read them) */
  const void* w_qkv_m;     /* W_qkv [(h_q + 2 h_kv) d_h, d] */
  const void* w_o_m;       /* W_o [d, h_q d_h] */
  const void* w_gate_m;    /* W_gate [d_ff, d] */
  const void* w_up_m;      /* W_up [d_ff, d] */
  const void* w_down_m;    /* W_down [d, d_ff] (the down projection itself, not w_down_t) */
  /* optional, sd_decode_step, any mode: W_down [d, d_ff] in the column-block
   * layout of sd_teal_gemv (w_t with d_out = d, d_in = d_ff), 16-byte
   * aligned, d at most 131072.  When set, the down projection reads only the
   * kept channels' pieces of it (every channel when dense), with the partial
   * sums added inside the launch, instead of w_down_t's rows and a separate
   * reduce launch; same results up to float32 summation order.  NULL:
   * w_down_t.  The caller owns it; the library only reads it. */
  const void* w_down_b;
} sd_layer;

/*
 * sd_decode_step -- one decode step through n_layers pre-norm Llama layers:
 *   x = RMSNorm(h) attn_norm; [q;k;v] = w_qkv x; RoPE(q, k) at position pos
 *   (rotate-half pairs (i, i + d_h/2)); k, v rounded to kv_dtype (nearest, ties
 *   to even) are appended at row n_full of the full cache and, if the layer has
 *   a gathered buffer, at row n_sel of it, in every mode ([Cross] §3.2: nothing
 *   is discarded and modes may switch per step); attention over rows
 *   0..n_full (dense) or 0..n_sel of the gathered buffer (SD_KV_SPARSE), scale
 *   1/sqrt(d_h); h += w_o attn; x = RMSNorm(h) mlp_norm; h += CATS-MLP(x) with
 *   the layer threshold under SD_MLP_SPARSE, dense otherwise.
 *   SD_PROJ_TEAL makes all seven projections TEAL-sparse instead (sd_teal_gemv
 *   semantics, w_*_t weights, thresholds teal_t): the attention input feeds
 *   W_q, W_k, W_v under one mask, the attention output W_o, the MLP input
 *   W_gate and W_up under one mask, and SiLU(gate) * up the down projection;
 *   it excludes SD_MLP_SPARSE.
 *   SD_KV_WINDOW attends instead over rows [0, window_sink) and the most recent
 *   window_keep - window_sink rows of the full cache (after the append), read
 *   in place ([Cross] §4.1, §4.4).  SD_ATTN_MASKED / SD_ATTN_FUSED run dense
 *   attention by the comparison paths of sd_decode_attn_baseline (the masked
 *   path needs the workspace of sd_workspace_bytes(dims, largest cap_full, 0)).
 *   At most one of SD_KV_SPARSE, SD_KV_WINDOW, SD_ATTN_MASKED, SD_ATTN_FUSED.
 * hidden  [d] float32, updated in place.
 * layers  [host] array; n_full and n_sel are advanced on success.
 * Errors: EINVAL for a missing gathered buffer under SD_KV_SPARSE or bad
 *         pointers; ENOSPC when a cache is full (n_full == cap_full, or
 *         n_sel == cap_sel) or the workspace is short.
 */
sd_status sd_decode_step(const sd_dims* dims, int32_t n_layers, sd_layer* layers, int32_t pos,
                         float* hidden, uint32_t mode, void* ws, size_t ws_bytes, void* stream);

/*
 * sd_decode_step_noalloc -- sd_decode_step without a caller workspace, for
 * callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, semantics and kernels as sd_decode_step; the intermediate
 * state lives in a buffer of SD_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (set up on the first call on a
 * device).  It runs on the current device; `stream` must belong to it.  Every
 * call on one GPU shares that buffer: calls that overlap on one GPU (other
 * streams, other threads) race, so order them on one stream.  The buffer keeps
 * the last call's contents; the step needs none of them.
 * Errors: as sd_decode_step; ENOSPC when the step's workspace
 *         (sd_workspace_bytes(dims, 0, 0), or with SD_ATTN_MASKED
 *         sd_workspace_bytes(dims, largest cap_full, 0)) exceeds the buffer;
 *         EHIP if the buffer's device address cannot be obtained.
 */
#define SD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sd_status sd_decode_step_noalloc(const sd_dims* dims, int32_t n_layers, sd_layer* layers,
                                 int32_t pos, float* hidden, uint32_t mode, void* stream);

/* One sequence's caches in one layer, for sd_decode_step_batch (the fields of
 * sd_layer with the same names, same meaning). */
typedef struct {
  void* k_full;            /* [h_kv, cap_full, d_h] */
  void* v_full;
  int32_t cap_full;
  int32_t n_full;          /* valid rows before the step; advanced by one [host] */
  void* k_sel;             /* gathered buffer [h_kv, cap_sel, d_h], or NULL */
  void* v_sel;
  int32_t cap_sel;
  int32_t n_sel;           /* advanced by one when k_sel != NULL */
} sd_seq_kv;

/*
 * sd_batch_workspace_bytes -- workspace of sd_decode_step_batch for `batch`
 * sequences [host]; 0 on invalid dims or batch.
 */
size_t sd_batch_workspace_bytes(const sd_dims* dims, int32_t batch);

/*
 * sd_decode_step_batch -- one decode step of `batch` sequences (2..8) that
 * share every weight read ([Cross] §3.3 "Dispatch and batching", §4.4
 * "Batching"): each sequence computes exactly its own sd_decode_step (its own
 * hidden state, position, caches and CATS mask, the layer threshold shared),
 * but each weight row is read once for the whole batch.  Under SD_MLP_SPARSE
 * the up rows and down columns read are those of the union of the batch's
 * masks (a channel kept by at least one sequence); a sequence that dropped a
 * channel gets no contribution from it.
 * SD_MATRIX_CORES runs the five projections as matrix products on the
 * matrix cores instead (bf16 weights in the tile layout, w_*_m of sd_layer;
 * float32 inputs split exactly into three bf16 parts, float32 sums): same
 * results to float32 rounding, same masks and union.  That path reads up and
 * down whole rather than the union's rows: at the batch sizes it is for, the
 * union keeps nearly every channel.
 * layers  [host] [n_layers]: weights, norms and cats_threshold as in
 *         sd_decode_step (its cache fields are not used); mask_out, when not
 *         NULL, receives the union mask [d_ff] (1 kept by some sequence).
 * kv      [host] [batch * n_layers], sequence-major (kv[b * n_layers + l]):
 *         each sequence's caches; n_full and n_sel advanced on success.
 * pos     [host] [batch] positions; hidden [batch, d] float32, in place.
 * mode    0, SD_KV_SPARSE, SD_MLP_SPARSE or both, optionally | SD_MATRIX_CORES.
 * Sizes:  d_model and n_q_heads * d_h at most 4096.
 * Errors: EINVAL for batch outside 2..8, other mode bits, bad pointers or a
 *         missing gathered buffer under SD_KV_SPARSE, or SD_MATRIX_CORES
 *         without all five tile weights; ENOSPC for a full cache or a short
 *         workspace (sd_batch_workspace_bytes); EUNSUPPORTED for widths, or
 *         SD_MATRIX_CORES with float32 weights.
 */
sd_status sd_decode_step_batch(const sd_dims* dims, int32_t n_layers, const sd_layer* layers,
                               int32_t batch, sd_seq_kv* kv, const int32_t* pos, float* hidden,
                               uint32_t mode, void* ws, size_t ws_bytes, void* stream);

/*
 * sd_pack_tiles -- a bf16 weight W [rows, d_in] (row-major, d_in a multiple of
 * 8, 16-byte aligned) rewritten into the tile layout that SD_MATRIX_CORES
 * reads: tiles of 16 rows by steps of 32 input channels, each (tile, step)
 * 1 KB in the A-operand order of the gfx950 matrix core, step-major: element
 * (r, c) at index ((c / 32) T + r / 16) 512 + ((r % 16) + 16 ((c % 32) / 8)) 8
 * + c % 8, T = ceil(rows / 16), padding rows and channels zero ([Cross] §3.3
 * "Dispatch and batching": a batch shares one read of every weight).
 * out     device, SD_TILE_BYTES(rows, d_in) bytes, 16-byte aligned, not
 *         overlapping w; enqueued on `stream`.
 * Errors: EINVAL for bad pointers or sizes.
 */
#define SD_TILE_BYTES(rows, d_in) \
  ((((size_t)(rows) + 15) / 16) * (((size_t)(d_in) + 31) / 32) * (size_t)1024)
sd_status sd_pack_tiles(const void* w, int32_t rows, int32_t d_in, void* out, void* stream);

/*
 * sd_stream_read -- one plain read of a device buffer with the access pattern
 * of the library's weight streams (16-byte non-temporal loads, eight per wave
 * in flight, the waves in flight reading one contiguous window), for the
 * read-bandwidth ceiling that the decode kernels are measured against
 * ([Cross] §4.1 "Timing and quality": achieved bandwidth is the measure).
 * buf    device, bytes a positive multiple of 8192, 16-byte aligned.
 * out    [SD_STREAM_BLOCKS] uint32 device out: the XOR of every 32-bit word
 *        each workgroup read; the XOR of all entries is the XOR of the buffer.
 * Errors: EINVAL for bad pointers or sizes.
 */
#define SD_STREAM_BLOCKS 2048
sd_status sd_stream_read(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* Byte account record ([Cross] §3). Bytes as doubles (exact below 2^53). */
typedef struct {
  double b_attn;        /* bytes of W_q, W_k, W_v, W_o per layer */
  double b_mlp;         /* bytes of W_gate, W_up, W_down per layer */
  double b_kv;          /* bytes of the keys and values of n tokens per layer */
  double b_total;       /* L (b_attn + b_mlp + b_kv) + fixed_bytes */
  double delta_p;       /* bytes the projection branch skips per step */
  double delta_kv;      /* bytes the KV branch skips per step */
  double bound_p;       /* b_total / (b_total - delta_p) */
  double bound_kv;
  double bound_both;
  double n_star;        /* crossover context in tokens (inf when r_kv == 1) */
  double n_star_budget; /* crossover of a KV method that keeps a fixed budget b = r_kv n
                           tokens whatever the context: b + P s_w (1 - r_p) / (2 h_kv d_h s_kv)
                           ([Cross] §3.3) */
  double gap_per_k;     /* s: seconds by which the byte-time gap between the branches grows
                           per 1K more tokens, the KV bytes the KV branch skips in 1024
                           tokens over bw_eff ([Cross] §4.3); NaN without a latency model */
  double n_lat;         /* latency crossing n* - (c_p - c_kv) / s * 1024 tokens ([Cross] §4.3);
                           inf when r_kv == 1; NaN without a latency model */
} sd_byte_record;

/* Kernel costs beyond byte time, for the latency crossing ([Cross] §4.3). */
typedef struct {
  double bw_eff;  /* effective bandwidth in bytes/s (> 0) */
  double c_p;     /* projection branch: seconds per step beyond its byte time */
  double c_kv;    /* KV branch: seconds per step beyond its byte time */
} sd_latency_model;

/*
 * sd_byte_account -- [Cross] §3.2-§3.3 from model dimensions: projection set
 * SD_PROJ_ALL7 (all seven projections), SD_PROJ_FFN (gate, up, down) or
 * SD_PROJ_CATS (up and down; the CATS gate is always read).  s_w, s_kv are
 * bytes per weight and cache element; r_p, r_kv keep ratios in [0, 1].
 * lat [host] or NULL: kernel costs for gap_per_k and n_lat (NaN when NULL).
 * out [host].  Errors: EINVAL for out-of-range arguments (bw_eff <= 0 among them).
 */
sd_status sd_byte_account(const sd_dims* dims, int32_t n_layers, double n, double r_p,
                          double r_kv, double s_w, double s_kv, int32_t proj_set,
                          double fixed_bytes, const sd_latency_model* lat, sd_byte_record* out);

/*
 * sd_latency_fit -- the latency model of a measured context sweep ([Cross]
 * §4.3, the kernel costs its predictions use): a bandwidth-bound step takes
 * its bytes / bw_eff plus a fixed kernel cost.
 *   bw_eff    = inverse slope of the least-squares line of the dense step's time
 *               t_dense[i] (seconds) against its bytes bytes_dense[i];
 *   c_modes[m] = mean over i of t_modes[m][i] - bytes_modes[m][i] / bw_eff.
 * bytes_modes, t_modes [host] [n_modes, n_points] row-major; bw_eff [host] out,
 * c_modes [host] [n_modes] out.
 * Errors: EINVAL for n_points < 2, non-finite values, or a dense time that
 *         does not grow with its bytes.
 */
sd_status sd_latency_fit(int32_t n_points, const double* bytes_dense, const double* t_dense,
                         int32_t n_modes, const double* bytes_modes, const double* t_modes,
                         double* bw_eff, double* c_modes);

/*
 * sd_latency_crossing -- measured crossing of two latency curves sampled at
 * the same ascending contexts ([Cross] §4.3 "Locating the Crossing"): linear
 * interpolation of t_a - t_b between the first neighbouring contexts whose
 * differences change sign; a zero difference is itself the crossing.
 * n_cross [host] out: the context in tokens, NaN when the curves do not cross
 * inside the sweep.  Errors: EINVAL for n_points < 1 or contexts that do not
 * ascend.
 */
sd_status sd_latency_crossing(int32_t n_points, const double* ctx, const double* t_a,
                              const double* t_b, double* n_cross);

/*
 * sd_latency_gate -- the latency gate of [Cross] §3.3 "Dispatch and batching":
 * among the admissible configurations, the one with the least total time over
 * a decode of `horizon` steps, horizon * t_step[i] + t_once[i] (t_once: the
 * one-time KV selection, 0 for configurations without one); equal totals go to
 * the lower index.  admissible [host] [n_configs] bytes (0 = excluded by a
 * quality test) or NULL for all.  best [host] out: the index, -1 when none is
 * admissible.  Errors: EINVAL for n_configs < 1, negative or non-finite times.
 */
sd_status sd_latency_gate(int32_t n_configs, const double* t_step, const double* t_once,
                          const uint8_t* admissible, double horizon, int32_t* best);

/*
 * sd_byte_crossover_batch -- the per-sequence crossover of a batch ([Cross]
 * §3.3 "Dispatch and batching"): B sequences share each weight read and the
 * union of their kept channels covers a fraction u_b of the projection set,
 * so n_B* = P s_w (1 - u_b) / (2 B h_kv d_h s_kv (1 - r_kv)) tokens (infinite
 * at r_kv = 1).  n_star [host] out.  Errors: EINVAL for out-of-range
 * arguments.
 */
sd_status sd_byte_crossover_batch(const sd_dims* dims, int32_t batch, double u_b, double r_kv,
                                  double s_w, double s_kv, int32_t proj_set, double* n_star);

/*
 * sd_cats_calibrate -- per-layer CATS threshold from calibration states, the
 * percentile rule CATS uses ([SATS]): a = SiLU(w_gate RMSNorm(x) norm_w) for
 * each of the n_states rows of `states` [n_states, d]; with v the float32 |a|
 * values sorted ascending (N = n_states * d_ff of them) and
 * k = round(sparsity N), threshold = v[k-1] (or -1 when k == 0).
 * threshold [1] float32 out (device).  Errors: EINVAL for sparsity outside
 * [0, 1] or n_states < 1; ENOSPC for a short workspace
 * (needs sd_calibrate_workspace_bytes).
 */
size_t sd_calibrate_workspace_bytes(const sd_dims* dims, int32_t n_states);
sd_status sd_cats_calibrate(const sd_dims* dims, const float* states, int32_t n_states,
                            const float* norm_w, const void* w_gate, float sparsity,
                            float* threshold, void* ws, size_t ws_bytes, void* stream);

/*
 * Opt-in per-kernel timing.  Between sd_profile_start() and sd_profile_stop(),
 * every kernel the library launches is bracketed by two HIP events on its
 * stream.  sd_profile_stop() waits for the recorded work, writes up to
 * max_stats entries (one per kernel kind that ran: launch count and summed
 * event-to-event milliseconds) to out [host], and returns the number of kinds
 * (-1 if an event query failed).  The state is process-wide; profiling adds
 * two event records per launch, so time the step itself with it off.
 */
typedef struct {
  char name[32];
  int32_t launches;
  int32_t pad0;
  double total_ms;
} sd_kernel_stat;

sd_status sd_profile_start(void);
int32_t sd_profile_stop(sd_kernel_stat* out, int32_t max_stats);

const char* sd_status_string(sd_status status);
const char* sd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SD_H */
