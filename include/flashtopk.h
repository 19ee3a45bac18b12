/*
 * flashtopk.h -- C ABI of the MI355X (gfx950) fused indexer top-k library.
 *
 * One call scores every key of each query row's window with the lightning
 * indexer and returns the row's exact top-k keys:
 *
 *     I[t,s] = sigma[s] * sum_{h<32} w[t,h] * ReLU( q[t,h,:] . kv[s,:] )
 *
 * for s in the half-open window [ks[t], ke[t])  (FlashTopK README, section
 * "Quick start": the indexer-score equation, the window, the causal-chunk
 * example and its shapes).  Selection is exact and deterministic: row t lists
 * min(topk, ke[t]-ks[t]) absolute key indices ordered by score descending, and
 * among equal scores the smaller key index comes first (README, "What you can
 * do": "Exact" and "Deterministic").  Slots beyond the window length are padded
 * with index -1 and value -inf (DeepSelect README, "Variable-length rows": rows
 * shorter than topk are padded with fill values; -1 / -inf are this library's
 * fill values).  +0 and -0 scores compare equal and are returned as +0.
 *
 * Operand layouts (all row-major, contiguous, device memory):
 *   q          [num_q, 32, 128]  FP8 E4M3FN (OCP, finite-only) or BF16
 *   kv         [num_kv, 128]     same dtype as q; one key per token, shared by
 *                                all 32 heads
 *   kv_scales  [num_kv] float32  per-key scale sigma >= 0, or NULL for all ones
 *   weights    [num_q, 32] float32 per-head weights (any sign)
 *   ks, ke     [num_q] int32     window bounds, 0 <= ks[t] <= ke[t] <= num_kv
 *   out_idx    [num_q, topk] int32, or int64 with FLASHTOPK_OUT_INT64
 *   out_val    [num_q, topk] float32 (the score of out_idx), or NULL to skip
 *
 * Ownership: the caller allocates and owns every operand and output.  The
 * library owns only scratch memory: a grow-only workspace per (device,
 * stream) that it keeps between calls and frees in flashtopk_release().
 * Operands must stay unmodified until the stream has finished the call.
 *
 * Synchronisation: work is enqueued on `stream` (a hipStream_t; NULL is the
 * device's null stream) and is stream-ordered: out_idx / out_val are complete
 * once the stream has reached the end of the call's work (synchronise the
 * stream, or wait on an event recorded after the call).  A call does not
 * block the calling thread: every decision (which rows need dense
 * rescoring, whether a tile prunes) stays on the device, and the rescoring
 * is launched up front in batches sized for the worst case, whose work
 * items exit at once when no row needs them.  Exceptions: a call that grows
 * the workspace first drains the stream (flashtopk_reserve avoids this), and
 * options.validate / options.profile wait for the GPU.  Calls on one stream
 * from several host threads are serialised by a lock on the stream's
 * workspace; calls on different streams run concurrently.
 *
 * Precision: scores are binary32, and a (row, key) pair's score has the same
 * bits on every path and in every batch (the selection is exact with respect
 * to these scores).  BF16 dot products round like binary32 sums.  The FP8
 * matrix cores' dot products err by up to about 2^-16 of sum_d |q_d kv_d|;
 * FP8 rows whose window holds more than 4096 keys also evaluate the head sum
 * through (sum_h w|x_h| + qbar . kv) / 2 with the query sum qbar carried to
 * 12 significant bits, which adds at most 2^-12 * sigma * max_d |kv_d| *
 * sum_h |w_h| ||q_h||_1; shorter rows use the plain ReLU form.
 *
 * Errors: every entry point returns 0 (FLASHTOPK_OK) or a positive status;
 * nothing is thrown across the ABI and nothing is printed.  Preconditions
 * that cost a device read (window bounds inside [0, num_kv], finite operands)
 * are not checked; violating them is undefined behaviour.
 */
#ifndef FLASHTOPK_H
#define FLASHTOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Operand dtypes (README, "Support": FP8 or BF16 operands). */
#define FLASHTOPK_FP8_E4M3 0
#define FLASHTOPK_BF16 1

/* Fixed indexer geometry (README, "Support": indexers of 32 heads x 128). */
#define FLASHTOPK_HEADS 32
#define FLASHTOPK_DIM 128
/* Largest supported topk (README, "Support": topk up to 4096). */
#define FLASHTOPK_MAX_TOPK 4096

/* Status codes. */
#define FLASHTOPK_OK 0
#define FLASHTOPK_ERR_INVALID_ARGUMENT 1 /* null required pointer, bad size, topk outside [1, 4096],
                                            unknown output flag */
#define FLASHTOPK_ERR_UNSUPPORTED 2      /* dtype other than FP8 E4M3 / BF16 */
#define FLASHTOPK_ERR_OUT_OF_MEMORY 3    /* workspace allocation failed */
#define FLASHTOPK_ERR_HIP 4              /* a HIP runtime or launch error */
#define FLASHTOPK_ERR_WORKSPACE_LIMIT 5  /* flashtopk_select_noalloc: the call needs more
                                            scratch than its fixed array holds */

/* Execution paths.  Every path returns bit-identical results; they differ only
 * in speed.  Used by tests and benchmarks to force a path.
 *   AUTO     calls of at most 8M (row, key) pairs (num_q * num_kv) take the
 *            dense path, larger ones the fused path with the per-tile prune
 *            decision
 *   SCAN     fused: sampled threshold + full filtering scan, no pruning
 *   PRUNE    fused: sampled threshold + score-bound key pruning everywhere
 *   RECOVER  dense: every row's window scores are materialised in the
 *            workspace and selected exactly (the rescoring that the fused
 *            path applies to rows its threshold misjudged)
 *   FUSED    fused with the per-tile prune decision, whatever the size */
#define FLASHTOPK_PATH_AUTO 0
#define FLASHTOPK_PATH_SCAN 1
#define FLASHTOPK_PATH_PRUNE 2
#define FLASHTOPK_PATH_RECOVER 3
#define FLASHTOPK_PATH_FUSED 4

/* Output options (DeepSelect README, "Usage": sorted_index and indices_type;
 * "Recommendations": index order costs time).  Bit flags.
 *   FLASHTOPK_OUT_INDEX_ORDER  the same topk keys, listed by ascending index
 *                              (values follow their indices); padding still
 *                              at the end
 *   FLASHTOPK_OUT_INT64        out_idx holds int64 entries (-1 padding) */
#define FLASHTOPK_OUT_INDEX_ORDER 1
#define FLASHTOPK_OUT_INT64 2

/* Knobs for flashtopk_select_ex.  Zero-initialise for defaults. */
typedef struct flashtopk_options {
    int path;                 /* FLASHTOPK_PATH_* */
    int cand_capacity;        /* candidates kept per row before a row is
                                 rescored densely; 0 = default min(16384, 4*topk),
                                 otherwise clamped to [topk, 16384] */
    float sample_rank_scale;  /* multiplies the rank of the sampled threshold;
                                 0 = 1.  Below 1 raises the threshold (fewer
                                 candidates), above 1 lowers it */
    int sample_target;        /* most keys sampled per row for the
                                 threshold; 0 = 2048, at most 2048 (the
                                 lattice stride is also at least topk / 32) */
    int64_t recover_budget_bytes; /* scratch for dense scores; 0 = 2 GiB.  The
                                 fused path reserves it for the rescoring it
                                 launches up front; rows are rescored in
                                 batches of budget / (4 * num_kv) rows (at
                                 least 16), so a smaller budget means more
                                 batches */
    int profile;              /* nonzero: time each kernel phase with HIP
                                 events on the call's stream (ms_* of
                                 flashtopk_info); adds a few microseconds */
    int out_flags;            /* FLASHTOPK_OUT_* bits; 0 = score order, int32 */
    int heads;                /* indexer heads: 0 or 32, or 64 (README
                                 "Roadmap": head counts besides 32, with 64
                                 as the named case); q is [num_q, heads, 128]
                                 and weights [num_q, heads].  64-head calls
                                 take the scan path (no score-bound pruning) */
    int validate;             /* nonzero: check the data preconditions on the
                                 device first and wait for the result (a debug
                                 aid, it synchronises the stream): windows in
                                 [0, num_kv] with ks <= ke, no NaN / infinity
                                 codes in q and (contiguous) kv, finite
                                 weights, finite non-negative kv_scales, page
                                 ids inside the pool.  Violations are reported
                                 in flashtopk_info.invalid (FLASHTOPK_INVALID_*
                                 bits) and any violation makes the call return
                                 FLASHTOPK_ERR_INVALID_ARGUMENT before a
                                 scoring kernel runs: the outputs are not
                                 written.  Paged calls check q, weights,
                                 windows and page ids, not the pool's keys */
} flashtopk_options;

/* Bits of flashtopk_info.invalid (calls made with options.validate). */
#define FLASHTOPK_INVALID_WINDOW 1   /* a window outside [0, num_kv] or with ks > ke */
#define FLASHTOPK_INVALID_Q 2        /* a NaN / infinity code in q */
#define FLASHTOPK_INVALID_KV 4       /* a NaN / infinity code in kv */
#define FLASHTOPK_INVALID_WEIGHT 8   /* a non-finite weight */
#define FLASHTOPK_INVALID_SCALE 16   /* a negative or non-finite kv_scale */
#define FLASHTOPK_INVALID_PAGE 32    /* a block_table entry outside [0, num_pages) */

/* What the last call on a stream did (README, "Usage": last_info). */
typedef struct flashtopk_info {
    int32_t status;             /* status of that call */
    int32_t path;               /* FLASHTOPK_PATH_SCAN / _PRUNE (fused path, pruned
                                   somewhere or not) or _RECOVER (dense path) */
    int64_t rows;               /* num_q */
    int64_t rows_empty;         /* ks == ke */
    int64_t rows_take_all;      /* fused path: window no longer than the candidate
                                   capacity, every key is a candidate */
    int64_t rows_sampled;       /* fused path: rows filtered by a sampled threshold */
    int64_t rows_underflow;     /* fused path: rows left with fewer than min(topk,
                                   window) candidates */
    int64_t rows_overflow;      /* fused path: rows with more candidates than capacity */
    int64_t rows_recovered;     /* rows rescored densely (fused path: underflow +
                                   overflow; dense path: every non-empty row) */
    int64_t max_candidates;     /* largest candidate count of a sampled row */
    int64_t window_keys;        /* sum of window lengths */
    int64_t pruned_keys;        /* (row, key) pairs skipped by the score bound */
    int32_t cand_capacity;      /* capacity used */
    int32_t sample_target;      /* sample size used */
    /* Device time of each phase in milliseconds when the call ran with
     * options.profile set, else 0: strided-sample scoring (with the per-key
     * and per-row preparation passes), per-row threshold, fused score +
     * filter (with the score bound), triage (0: done inside the selection),
     * candidate selection with triage, dense recovery (the dense path: the
     * whole call). */
    float ms_sample, ms_tau, ms_filter, ms_triage, ms_select, ms_recover;
    int32_t invalid;            /* FLASHTOPK_INVALID_* bits found by options.validate, else 0 */
    int64_t candidates;         /* fused path: candidates of the sampled rows, summed (the
                                   threshold aims at 2 * topk per row) */
} flashtopk_info;

/* Exact top-k of the indexer score for every query row (see the file comment
 * for operand layouts and semantics).  num_q >= 0, 0 <= num_kv < 2^31,
 * 1 <= topk <= 4096, dtype FLASHTOPK_FP8_E4M3 or FLASHTOPK_BF16.  num_q == 0
 * is a no-op. */
int flashtopk_select(const void *q, const void *kv, const float *kv_scales,
                     const float *weights, const int32_t *ks, const int32_t *ke,
                     int64_t num_q, int64_t num_kv, int dtype, int topk,
                     void *out_idx, float *out_val, void *stream);

/* flashtopk_select with options (opt may be NULL = defaults). */
int flashtopk_select_ex(const void *q, const void *kv, const float *kv_scales,
                        const float *weights, const int32_t *ks, const int32_t *ke,
                        int64_t num_q, int64_t num_kv, int dtype, int topk,
                        void *out_idx, float *out_val, void *stream,
                        const flashtopk_options *opt);

/* Score-row dtypes of flashtopk_topk_rows (DeepSelect README, "Supported
 * Cases": BF16 rows for the indexer scenario, float32 for sampling). */
#define FLASHTOPK_SCORES_F32 0
#define FLASHTOPK_SCORES_BF16 1

/* Exact top-k of every row of an already materialized score matrix
 * (DeepSelect README, "Usage" and "Variable-length rows").
 *
 *   x         [rows, row_stride] float32 or BF16 (score_dtype), device memory;
 *             the first `cols` entries of each row are its scores.  x must be
 *             16-byte aligned; when rows > 1, row_stride >= cols and
 *             row_stride * element size is a multiple of 16 bytes (the
 *             README's stride requirement; pad rows otherwise).
 *   ends      [rows] int32, or NULL: row r keeps only its first ends[r]
 *             entries (exclusive bound, clamped to [0, cols]); NULL = cols.
 *   out_idx   [rows, topk] int32 (int64 with FLASHTOPK_OUT_INT64), out_val
 *             [rows, topk] float32 or NULL.
 *   out_flags FLASHTOPK_OUT_* bits (0: score order, int32 indices).
 *   nan_flag  one int32 in device memory, or NULL: the call sets it to 1 when
 *             an entry inside some row's bound is NaN (the caller clears it;
 *             the README's kernel aborts instead).  Rows holding NaN get an
 *             unspecified selection, but every write stays in bounds.
 *
 * Row r lists min(topk, its length) column indices by value descending,
 * smaller index first among equal values, padded with -1 / -inf; +0 and -0
 * compare equal and values come back as float32 (BF16 widened exactly), +0
 * for a zero.  0 <= rows, cols < 2^31, 1 <= topk <= 4096.  rows == 0 is a
 * no-op.  Enqueued on `stream` without blocking the host.  Calls of few rows
 * (fewer than the GPU has compute units) split each row over several
 * workgroups and keep per-row state in the stream's workspace (a few bytes
 * per row plus 64 KiB per row of candidates); others use no workspace.
 * Ownership, synchronisation and errors as for flashtopk_select. */
int flashtopk_topk_rows(const void *x, int score_dtype, int64_t rows, int64_t cols, int64_t row_stride,
                        const int32_t *ends, int topk, void *out_idx, float *out_val, int32_t *nan_flag,
                        int out_flags, void *stream);

/* flashtopk_select_ex over keys held in a paged cache (README, "Roadmap":
 * paged KV cache).  Logical key s (0 <= s < num_kv; windows, outputs and the
 * tie rule use logical positions) is row s % page_size of page
 * block_table[s / page_size] of the pool
 *   kv_pages     [num_pages, page_size, 128] FP8 / BF16 (16-byte aligned)
 *   scale_pages  [num_pages, page_size] float32, or NULL for all ones
 *   block_table  [ceil(num_kv / page_size)] int32 page ids in [0, num_pages)
 * shared by every query row of the call.  The call gathers its keys into the
 * workspace (one streaming pass over num_kv keys) and then runs as
 * flashtopk_select_ex; results are bit-identical to a call on the gathered
 * contiguous keys.  A page id outside [0, num_pages) is a precondition
 * violation: its keys read as zero with zero scale.  page_size >= 1. */
int flashtopk_select_paged(const void *q, const void *kv_pages, const float *scale_pages, const int32_t *block_table,
                           int page_size, int64_t num_pages, const float *weights, const int32_t *ks,
                           const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype, int topk, void *out_idx,
                           float *out_val, void *stream, const flashtopk_options *opt);

/* Pre-allocate the workspace of (current device, stream) for calls up to the
 * given sizes (README, "Usage": the Selector's plan() owns the workspace and
 * prepares up front), so that later calls of at most max_q rows, max_kv keys
 * and max_topk, of this dtype, with 32 or 64 heads, on either path, with the
 * default candidate capacity, sample size and recovery budget, and row top-k
 * calls of at most max_q rows of max_kv entries, allocate nothing and never
 * drain the stream.  Calls whose options raise the capacity, the sample size
 * or the budget may still grow it.  The workspace holds about
 * max_q * (8 * min(16384, 4 * max_topk) + 8 KiB) bytes plus the recovery
 * scratch (up to 2 GiB by default). */
int flashtopk_reserve(int64_t max_q, int64_t max_kv, int max_topk, int dtype, void *stream);

/* Record of the last call issued on `stream` from this process.  Synchronises
 * the stream, then counts the row classes from the workspace's arrays (so it
 * must be read before the next call on the stream overwrites them).  Returns
 * FLASHTOPK_ERR_INVALID_ARGUMENT if the stream has had no call. */
int flashtopk_get_last_info(void *stream, flashtopk_info *out);

/* Rows that the last call on `stream` scored densely (README, "Highlights":
 * rows whose sampled threshold misjudged them are rescored; on the dense
 * path, every row with a non-empty window), as a diagnostic: synchronises
 * the stream, writes the first min(count, max_rows) row indices, in no
 * particular order, to the host array `rows`, and their number to *count.
 * Like flashtopk_get_last_info it must be read before the next call on the
 * stream.  rows may be NULL when max_rows is 0. */
int flashtopk_get_last_recovered(void *stream, int32_t *rows, int64_t max_rows, int64_t *count);

/* flashtopk_select for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results bit-identical to
 * flashtopk_select's, and no hipMalloc, hipFree or other allocating call.
 * Its scratch is one fixed array of FLASHTOPK_NOALLOC_SCRATCH_BYTES in the
 * library's device code object: every GPU the library is loaded on holds
 * its own copy until the process ends.  A call whose workspace does not fit
 * (roughly: num_q * (min(16384, 4 * topk) * 8 + 8192) bytes for calls above
 * 8M (row, key) pairs, num_q * num_kv * 4 bytes of window scores below;
 * dense rescoring takes at most 32 MiB of it) returns
 * FLASHTOPK_ERR_WORKSPACE_LIMIT before any work is enqueued.  Default
 * options only.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (from several host threads, or on several streams whose
 * work runs concurrently) race on it and must be serialised by the caller;
 * successive calls on one stream are safe.  It keeps no record for
 * flashtopk_get_last_info. */
#define FLASHTOPK_NOALLOC_SCRATCH_BYTES (128ll << 20)
int flashtopk_select_noalloc(const void *q, const void *kv, const float *kv_scales,
                             const float *weights, const int32_t *ks, const int32_t *ke,
                             int64_t num_q, int64_t num_kv, int dtype, int topk,
                             void *out_idx, float *out_val, void *stream);

/* Diagnostic: the attainable throughput of the scan's matrix-core
 * instruction on the stream's device under sustained load, in TFLOP/s
 * (dense, 2 FLOPs per multiply-add), written to *tflops.  dtype picks the
 * instruction: FLASHTOPK_FP8_E4M3, v_mfma_f32_16x16x128_f8f6f4 on E4M3
 * operands; FLASHTOPK_BF16, v_mfma_f32_32x32x16_bf16.  Four workgroups of
 * four waves per compute unit each issue iters rounds of four independent
 * accumulation chains on register operands (fixed per-lane pseudo-random
 * finite codes), with no memory traffic; one warm-up launch of iters / 8
 * rounds precedes the timed launch, which is timed with HIP events on
 * `stream`.  Synchronises the stream; allocates no device memory.
 * FLASHTOPK_ERR_INVALID_ARGUMENT for a NULL tflops, iters <= 0 or another
 * dtype. */
int flashtopk_probe_mfma(int dtype, int iters, void *stream, double *tflops);

/* Frees every cached workspace.  No call may be in flight. */
void flashtopk_release(void);

/* Human-readable name of a status code (static storage). */
const char *flashtopk_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int flashtopk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHTOPK_H */
