/*
 * tria.h -- C ABI of the MI355X (gfx950) TriAttention KV-cache eviction pass.
 *
 * The pass, for every (layer, KV head) of a cache (one "unit"):
 *   1. scores every cached key by calibrated RoPE-direction importance,
 *   2. z-normalises each query head's scores and takes the max over the query
 *      heads that share the KV head,
 *   3. keeps the top-budget rows while always keeping the sink prefix and the
 *      recent window,
 *   4. compacts K, V and positions in place, in order, with no gaps.
 *
 * Sources (web pages, cited by title and section):
 *   [WL] "TriAttention Native C++ Worklog" (TensorRT-Model-Connect).
 *   [LC] llama.cpp docs "TriAttention KV-Cache Eviction (--triattention)".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Device pointers are HIP device memory owned by the caller; host pointers
 *   are ordinary host memory, read during the call only.  The library keeps no
 *   pointer to caller memory after a call returns.
 * - Every call only enqueues work on `stream` (0 = the null stream) and never
 *   synchronises it.  Kept counts are computed on the host from the sizes, so
 *   they are returned without waiting for the GPU.
 * - A context is not thread-safe: use one context per stream.  Calls on one
 *   context must be stream-ordered (they share the context's scratch).
 * - Errors: a negative TRIA_E_* code.  Argument and eligibility errors are
 *   detected before anything is enqueued, so caller buffers are untouched.  A
 *   HIP failure during a pass (TRIA_E_HIP) can leave a cache partly compacted;
 *   treat it as invalid.  No C++ exception crosses this interface.
 * - Key rows are stored already rotated (RoPE applied, rotate-half layout:
 *   pair f is (x[f], x[f + head_dim/2])).  Row n-1 of every unit must hold the
 *   newest token when a pass starts (its position is the phase reference).
 * - A tria_evict, tria_evict_noalloc or tria_evict_paged_batch pass may be
 *   captured in a HIP graph and the graph replayed any number of times on one
 *   stream: the pass enqueues kernels only (no copy, memset or host wait), and
 *   the state one launch hands the next (task counter, compaction epoch) lives
 *   on the device.  Capture tria_evict or tria_evict_paged_batch after an eager
 *   call of the same or a larger shape on the context, so that it does not
 *   allocate while capturing; tria_evict_noalloc never allocates.  Replays use
 *   the shapes, budgets and pointers of the capture.
 *
 * Layouts
 * -------
 *   contiguous cache  k, v : [L][Hkv][cap] rows of tria_row_bytes(type, hd)
 *                     pos  : [L][Hkv][cap] int32 absolute positions
 *   paged cache       k, v : [L][n_blocks][Hkv][16] rows (16-token blocks)
 *                     pos  : [L][n_blocks][Hkv][16] int32
 *                     block_table : [n_seq][max_blocks] int32 physical block
 *                     ids; logical row r of a sequence lives in block
 *                     block_table[seq][r / 16], slot r % 16, for every
 *                     (layer, KV head).
 *   statistics        [L][Hq][hd/2] fp32; query head h = g*G + j (j < G,
 *                     G = Hq/Hkv) belongs to KV head g.
 *   raw scores        [L][Hkv][n][G] fp32
 *   agg               [L][Hkv][n] fp32
 *   keep_idx          [L][Hkv][kept] int32, ascending row indices
 */
#ifndef TRIA_H
#define TRIA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define TRIA_OK 0
#define TRIA_E_INVAL (-1)       /* null or misaligned pointer, size out of range, negative budget/sink/window,
                                   offsets not strictly ascending and positive */
#define TRIA_E_UNSUPPORTED (-2) /* shape outside the GPU scorer's eligibility gate */
#define TRIA_E_HIP (-3)         /* a HIP runtime call failed; see tria_last_hip_error */
#define TRIA_E_NOMEM (-4)       /* device or host allocation failed */
#define TRIA_E_DEVICE (-5)      /* a compaction workgroup gave up a bounded wait (reported by
                                   tria_device_status; the cache is then not trustworthy) */

/* Storage types of a cached row. */
#define TRIA_KV_F16 0  /* head_dim IEEE fp16 values, 2*head_dim bytes */
#define TRIA_KV_Q8_0 1 /* head_dim/32 blocks of {fp16 scale d, 32 x int8 q}; value = d*q;
                          34*head_dim/32 bytes ([LC] section 4: the GPU scorers read q8_0 K) */

/* Largest number of sequences in one tria_evict_paged_batch call. */
#define TRIA_MAX_SEQ 64
/* Largest number of rows (n_tokens) of one unit that any entry point takes;
 * more gives TRIA_E_UNSUPPORTED before anything is enqueued. */
#define TRIA_MAX_ROWS 262144
/* Rows per block of a paged cache. */
#define TRIA_BLOCK 16

typedef struct tria_ctx tria_ctx;

/* Model shape and scoring constants, fixed for the life of a context. */
typedef struct tria_model_desc {
    int32_t n_layers;      /* L >= 1 */
    int32_t n_kv_heads;    /* Hkv >= 1 */
    int32_t n_q_heads;     /* Hq, a multiple of Hkv, Hq/Hkv <= 64 */
    int32_t head_dim;      /* hd, a multiple of 32, <= 256 ([LC] section 4 gate) */
    int32_t k_type;        /* TRIA_KV_F16 or TRIA_KV_Q8_0 */
    int32_t v_type;        /* TRIA_KV_F16 or TRIA_KV_Q8_0 (V is only moved) */
    double rope_theta;     /* RoPE base: omega_f = theta^(-2f/hd), > 1 */
    int32_t n_offsets;     /* |D| >= 1 */
    const int64_t *offsets;/* host: future query offsets, strictly ascending, > 0 */
} tria_model_desc;

/* Contiguous cache (device pointers, caller-owned).  k and v start on a
 * 16-byte boundary, pos on a 4-byte one (TRIA_E_INVAL otherwise): the kernels
 * move rows in pieces of up to 16 bytes. */
typedef struct tria_cache {
    void *k;
    void *v;
    int32_t *pos;
    int64_t cap; /* rows per unit */
} tria_cache;

/* Paged cache (device pointers, caller-owned).  k_pool and v_pool start on a
 * 16-byte boundary, pos_pool and block_table on a 4-byte one. */
typedef struct tria_paged_cache {
    void *k_pool;
    void *v_pool;
    int32_t *pos_pool;
    int64_t n_blocks;           /* physical blocks per layer */
    const int32_t *block_table; /* device [n_seq][max_blocks] */
    int32_t max_blocks;         /* row stride of block_table */
} tria_paged_cache;

/* Create a context: copies the calibration statistics to the device.
 * The score is ([WL], "Phase 9: final root cause - native scorer used the
 * wrong formulation"; [LC] section 5, "Phase C"):
 *   s_h(r) = sum_f Re(qbar_{h,f} A_f conj(K_f(r))) + sum_f w_{h,f} |K_f(r)|,
 *   A_f = mean over delta in offsets of exp(i omega_f (p + delta)),
 * with p the absolute position of the newest cached row ([WL], "2026-04-18:
 * later-compaction absolute-position bug isolated and fixed").
 *   q_re, q_im : host [L][Hq][hd/2], the complex mean pre-RoPE query qbar.
 *   norm_w     : host [L][Hq][hd/2], the weight of the |K_f| term.
 * On success *out owns device memory until tria_free. */
int tria_load_stats(tria_ctx **out, const tria_model_desc *desc, const float *q_re,
                    const float *q_im, const float *norm_w, hipStream_t stream);

/* Release a context (waits for nothing; the caller must have synchronised the
 * stream the context was used on).  NULL is ignored. */
void tria_free(tria_ctx *ctx);

/* Static description of an error code. */
const char *tria_strerror(int code);

/* hipError_t of the last failed HIP call made for this context (0 if none). */
int tria_last_hip_error(const tria_ctx *ctx);

/* Bytes of one stored row, or a negative code for an unknown type/shape. */
int64_t tria_row_bytes(int32_t kv_type, int32_t head_dim);

/* Rows one pass keeps: n if budget >= n, else max(budget, |protected|), where
 * the protected rows are the first `sink` and the last `window` rows ([LC]
 * section 5, "Phase B"; kept rows equal the budget in [WL]'s compaction
 * logs).  Negative arguments give TRIA_E_INVAL. */
int64_t tria_kept_count(int64_t n_tokens, int64_t budget, int64_t sink, int64_t window);

/* Raw per-query-head scores of the first n_tokens rows of every unit.
 *   raw_scores : device [L][Hkv][n_tokens][G] fp32, written; 16-byte aligned.
 * 0 <= n_tokens <= cache->cap, n_tokens <= TRIA_MAX_ROWS.  Returns TRIA_OK or
 * an error code. */
int tria_score(tria_ctx *ctx, const tria_cache *cache, int64_t n_tokens, float *raw_scores,
               hipStream_t stream);

/* Aggregate and select ([LC] section 5, "Phase B" steps 2-3 and "Phase C"):
 * per query head, z = (s - mu)/sigma over the unit's rows with a finite score
 * (sigma = 0 gives z = 0); agg = max over the group, or -inf if any of the
 * row's scores is not finite; keep the protected rows plus the highest-agg
 * candidates (ties to the lower row index) up to tria_kept_count.
 *   raw_scores : device [L][Hkv][n_tokens][G], read; 16-byte aligned.
 *   keep_idx   : device [L][Hkv][kept], written (ascending rows); 4-byte aligned.
 *   agg_out    : device [L][Hkv][n_tokens] fp32, written if not NULL; 4-byte aligned.
 * n_tokens <= TRIA_MAX_ROWS.  Returns the kept count (>= 0) or an error code. */
int64_t tria_select(tria_ctx *ctx, const float *raw_scores, int64_t n_tokens, int64_t budget,
                    int64_t sink, int64_t window, int32_t *keep_idx, float *agg_out,
                    hipStream_t stream);

/* In-place, order-preserving compaction of K, V and pos ([LC] section 5,
 * "Phase B" step 4; [WL], "What was implemented": GPU gather/repack):
 *   row d <- row keep_idx[d] for d < kept, in every unit.  Bytes are copied
 *   exactly; rows >= kept are left unspecified.
 * keep_idx (4-byte aligned) must be strictly ascending per unit (as
 * tria_select writes it).  An entry outside [d, n_tokens) is skipped (row d is left as it was).
 * Indices that are not ascending never cause an access out of bounds, but the
 * result is then unspecified. */
int tria_compact(tria_ctx *ctx, const tria_cache *cache, int64_t n_tokens,
                 const int32_t *keep_idx, int64_t kept, hipStream_t stream);

/* One whole eviction pass: tria_score, tria_select, tria_compact with the
 * context's own scratch for the scores and kept indices, all on `stream`.
 * Returns the kept count.  budget >= n_tokens enqueues nothing and returns
 * n_tokens.  The context's scratch grows (hipMalloc) when a pass needs more
 * than an earlier one; tria_evict_noalloc is the variant that never
 * allocates. */
int64_t tria_evict(tria_ctx *ctx, const tria_cache *cache, int64_t n_tokens, int64_t budget,
                   int64_t sink, int64_t window, hipStream_t stream);

/* tria_evict for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same pass with the
 * same results, whose scratch (coefficient tables, raw scores, moment
 * partials, kept indices, chunk prefix counts, compaction flags and task
 * counter) lives in one fixed array of TRIA_NOALLOC_SCRATCH_BYTES per GPU in
 * the library's code object, held until the process ends.  The call makes no
 * hipMalloc, hipFree or hipMemset; its address is looked up once per device
 * (in tria_load_stats, or on the first call on a device).  Layers are processed
 * in as few groups as the array holds (one layer of a 36 x 8 x 32K q8_0 cache
 * needs about 4.5 MiB).  Returns the kept count, or TRIA_E_UNSUPPORTED before
 * anything is enqueued if one layer does not fit, or if a shared keep mode is
 * set (tria_set_keep_mode); otherwise the errors of tria_evict.  Every call on
 * a GPU uses that GPU's one array: calls that overlap on one GPU (concurrent
 * streams, several threads) race and give wrong results; a call must finish on
 * the GPU before the next one starts, which calls on one stream do. */
#define TRIA_NOALLOC_SCRATCH_BYTES 67108864 /* 64 MiB */
int64_t tria_evict_noalloc(tria_ctx *ctx, const tria_cache *cache, int64_t n_tokens,
                           int64_t budget, int64_t sink, int64_t window, hipStream_t stream);

/* The same pass over n_seq sequences of a paged cache, one launch per kernel
 * for all sequences.  n_tokens, budget: host [n_seq]; kept_out: host [n_seq],
 * written with each sequence's kept count.  Each sequence's rows beyond its
 * kept count are left unspecified; the caller may return those blocks.
 * 1 <= n_seq <= TRIA_MAX_SEQ; every n_tokens[i] <= TRIA_MAX_ROWS. */
int tria_evict_paged_batch(tria_ctx *ctx, const tria_paged_cache *cache, int32_t n_seq,
                           const int64_t *n_tokens, const int64_t *budget, int64_t sink,
                           int64_t window, int64_t *kept_out, hipStream_t stream);

/* Who shares a keep set in tria_select / tria_evict / tria_evict_paged_batch.
 *   TRIA_KEEP_PER_UNIT (default): every (layer, KV head) unit selects on its
 *     own scores (tria_select's rule).
 *   TRIA_KEEP_PER_KV_HEAD: one keep set per KV head g, used by every layer:
 *     the worklog ("TriAttention Native C++ Worklog", section "Later
 *     correction: selector and compaction are now cleared on the aggressive
 *     sample7 path") checks one keep-index list per KV head and gathers it in
 *     all layers, after a cross-layer aggregation step.
 *   TRIA_KEEP_GLOBAL: one keep set for the whole cache: the llama.cpp page
 *     ("TriAttention KV-Cache Eviction (--triattention)", section 5, "Phase
 *     C") ships a global z-normalisation shader for its cells, which hold
 *     every layer and head.
 * Neither page spells out the cross-unit reduction; it is taken as the GQA
 * group's rule over the larger group: each member query head is z-normalised
 * over its own unit's rows, the group score of a row is the max of those
 * z-scores over every member head (-inf if any member score is not finite),
 * and the group keeps the protected rows plus its highest-scoring candidates.
 * The raw scores, kept counts and compaction are those of the per-unit pass;
 * keep_idx (and agg_out) are written for every unit, equal within a group.
 * Returns TRIA_OK, or TRIA_E_INVAL for another mode. */
#define TRIA_KEEP_PER_UNIT 0
#define TRIA_KEEP_PER_KV_HEAD 1
#define TRIA_KEEP_GLOBAL 2
int tria_set_keep_mode(tria_ctx *ctx, int32_t mode);

/* How tria_compact / tria_evict / tria_evict_paged_batch pack the kept rows.
 *   TRIA_COMPACT_ORDERED (default): the order-preserving gather documented at
 *     tria_compact.
 *   TRIA_COMPACT_HOLE_FILL: a variant that moves far fewer rows once a cache
 *     is in steady state.  The llama.cpp page ("TriAttention KV-Cache Eviction
 *     (--triattention)", section 5, "Phase B" step 4) asks only that the kept
 *     rows end up packed in place with no gaps (cells carry their positions).
 *     With K kept rows of n: let the run be the kept rows n-r .. n-1 (the
 *     longest run of kept rows ending at row n-1; it holds the window).  The
 *     rows below K-r that are not kept (holes) receive, in ascending order,
 *     the kept rows at or above K-r outside the run (tails, ascending); then
 *     the run moves to rows K-r .. K-1 in order.  Kept rows below K-r (the
 *     sinks among them) do not move.  Rows [0, K) then hold exactly the kept
 *     rows, the sinks first and the newest rows last, so later passes protect
 *     the same tokens and keep the same ones as with the ordered gather,
 *     except where candidates tie exactly at the cutoff (a tie goes to the
 *     lower row, and rows are no longer in position order).  Positions move
 *     with their rows.  keep_idx must be ascending as for tria_compact; an
 *     entry that would move a row outside [0, n) is skipped.
 * Returns TRIA_OK, or TRIA_E_INVAL for another mode. */
#define TRIA_COMPACT_ORDERED 0
#define TRIA_COMPACT_HOLE_FILL 1

/* Cap on the workgroups of the order-preserving compaction (tria_compact,
 * tria_evict and its variants).  0 (the default): as many as the GPU holds at
 * once.  1: one workgroup takes every chunk task in order, so no task ever
 * waits for another: the serial reference against which the parallel in-place
 * rule is compared bit for bit.  Results do not depend on the cap.  Returns
 * TRIA_OK or TRIA_E_INVAL for a negative value. */
int tria_set_compaction_workgroups(tria_ctx *ctx, int32_t max_workgroups);
int tria_set_compaction(tria_ctx *ctx, int32_t mode);

/* ------------------------------------------------------------------------
 * Decode-loop policy: when a pass runs, and with which arguments.
 *   TRIA_TRIGGER_THRESHOLD ("TriAttention Native C++ Worklog", sections
 *     "4. Separate physical cache limit from logical TriAttention budget" and
 *     the compaction-trigger notes): a pass runs once the counted rows reach
 *     budget + divide_length and keeps `budget` counted rows (the logged
 *     schedule: 3200 rows -> 3072 every 128 decode steps at budget 3072,
 *     divide length 128).  With protect_prefill the prompt rows are neither
 *     counted nor evicted (decode-only accounting; prompt state is never
 *     compacted while it is being built).
 *   TRIA_TRIGGER_INTERVAL (llama.cpp page, section 1 --tri-interval; section 5
 *     "Phase B": the evictor fires in decode only): a pass runs every
 *     `interval` decode steps once the counted rows exceed the budget.
 * Passes never run during prefill: the caller sets n_prompt after prefill and
 * calls tria_decode_step once per decode step.
 * ------------------------------------------------------------------------ */
#define TRIA_TRIGGER_THRESHOLD 0
#define TRIA_TRIGGER_INTERVAL 1

typedef struct {
    int32_t trigger;         /* TRIA_TRIGGER_* */
    int32_t protect_prefill; /* 1: the prompt rows are kept and not counted */
    int64_t budget;          /* counted rows a pass keeps (>= 1) */
    int64_t divide_length;   /* THRESHOLD: slack before a pass runs (>= 1) */
    int64_t interval;        /* INTERVAL: decode steps between passes (>= 1) */
    int64_t sink, window;    /* as for tria_evict (>= 0) */
} tria_policy;

typedef struct {
    int64_t n_rows;   /* rows in the cache, the newest last */
    int64_t n_prompt; /* prompt rows at the front (0 if none) */
    int64_t steps;    /* decode steps since the last pass (or since the prompt) */
    int64_t passes;   /* passes run so far */
} tria_decode_state;

/* Host-only decision for the current state: returns 1 and the arguments of
 * the pass (for tria_evict) if one is due, 0 if not, TRIA_E_INVAL on a bad
 * policy or state.  With protect_prefill the pass keeps budget + n_prompt
 * rows with sink max(sink, n_prompt). */
int tria_policy_due(const tria_policy *p, const tria_decode_state *st, int64_t *budget_rows,
                    int64_t *sink_rows, int64_t *window_rows);

/* Physical rows a cache must hold so that appending one row per decode step
 * never overflows before the policy's pass runs (the worklog's fix for
 * prompt-time overflow: physical capacity above the logical budget).  Returns
 * the row count or TRIA_E_INVAL. */
int64_t tria_policy_peak_rows(const tria_policy *p, int64_t n_prompt);

/* One decode step, after the caller appended this step's row (st->n_rows
 * counts it): counts the step, runs tria_evict if the policy says so (on
 * `stream`), and updates the state.  Returns the rows now in the cache, or an
 * error code (TRIA_E_INVAL also when n_rows exceeds the cache's capacity). */
int64_t tria_decode_step(tria_ctx *ctx, const tria_cache *cache, const tria_policy *p,
                         tria_decode_state *st, hipStream_t stream);

/* One decode step's attention over the cache -- the cost an eviction pass
 * cuts ("TriAttention Native C++ Worklog", "What was implemented": decode
 * continues on the compacted cache).  For every layer and query head h =
 * g*G + j (KV head g):
 *   out_h = sum_r softmax_r(scale * q_h . k_r) v_r   over the unit's n rows.
 * Row order does not matter (ordered or hole-filled caches alike).
 *   q, out : device fp32 [L][Hq][head_dim], 4-byte aligned (q already rotated
 *            for its position; the keys are stored rotated); n_tokens = 0 gives
 *            zeros.
 * fp32 arithmetic; every K and V row is read once.  Scratch (per-range
 * partial results) is owned by the context. */
int tria_decode_attention(tria_ctx *ctx, const tria_cache *cache, int64_t n_tokens,
                          const float *q, float scale, float *out, hipStream_t stream);

/* The same over n_seq sequences of a paged cache: q, out [n_seq][L][Hq][hd]. */
int tria_decode_attention_paged_batch(tria_ctx *ctx, const tria_paged_cache *cache,
                                      int32_t n_seq, const int64_t *n_tokens, const float *q,
                                      float scale, float *out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Calibration statistics (the stats tria_load_stats takes), accumulated on
 * the GPU from pre-RoPE query vectors: the llama.cpp page ("TriAttention
 * KV-Cache Eviction (--triattention)", section 2, "Generating a .tria file")
 * hooks each layer's pre-RoPE query tensor during forward passes over a
 * corpus and accumulates per-head statistics; section 5, "Phase C", names the
 * per-head q_mean / q_abs arrays.  Per layer l, query head h and pair f, with
 * q_f = q[f] + i q[f + head_dim/2] over the T tokens added for that layer:
 *   q_re + i q_im = (1/T) sum q_f,   q_abs = (1/T) sum |q_f|,
 *   norm_w = q_abs - |q_re + i q_im|   (zero when every token's pair points the
 *   same way; q_abs when the directions cancel).
 * Sums are fp64 and their order is fixed by the calls, so a sequence of calls
 * gives the same result every time.
 * ------------------------------------------------------------------------ */
#define TRIA_Q_F32 0
#define TRIA_Q_F16 1
#define TRIA_Q_BF16 2
typedef struct tria_calib tria_calib;

/* Zeroed accumulators for n_layers x n_q_heads x head_dim/2 pairs (device
 * memory owned by the object).  head_dim even, <= 1024.  Synchronous. */
int tria_calib_create(tria_calib **out, int32_t n_layers, int32_t n_q_heads, int32_t head_dim);

/* Adds n_tokens query rows of one layer: q (device) holds row t at element
 * t * row_stride, head h's head_dim values at + h * head_dim (row_stride >=
 * n_q_heads * head_dim, e.g. the query slice of a fused projection), type
 * TRIA_Q_*, q aligned to its element size.  Rows whose base and stride allow
 * it are read in 16-byte (fp32) or 8-byte pieces.  Stream-ordered; q must stay
 * valid until the work has run.  One
 * kernel launch, no allocation.  Calls on one object must use one stream (or
 * be ordered by the caller): they add into the same accumulators. */
int tria_calib_add(tria_calib *c, int32_t layer, const void *q, int32_t q_type, int64_t n_tokens,
                   int64_t row_stride, hipStream_t stream);

/* tria_calib_add for n_layers consecutive layers layer0 .. layer0 + n_layers - 1
 * at once (one kernel launch for all of them; per-layer launches of a few tens
 * of MB are dominated by their start and tail): layer layer0 + i's rows start
 * at element i * layer_stride of q (layer_stride >= n_tokens * row_stride when
 * n_layers > 1, so that layers do not overlap).  A call over many layers
 * spreads each layer's tokens over fewer accumulator slots than one-layer calls
 * do (so that one launch holds a few thousand workgroups), so its sums may
 * differ from those of per-layer calls in fp64 rounding; for a given sequence
 * of calls every sum is formed in a fixed order.
 * 1 <= n_layers <= n_layers of the object - layer0. */
int tria_calib_add_layers(tria_calib *c, int32_t layer0, int32_t n_layers, const void *q,
                          int32_t q_type, int64_t n_tokens, int64_t row_stride,
                          int64_t layer_stride, hipStream_t stream);

/* Tokens added so far to a layer (host count), or an error code. */
int64_t tria_calib_tokens(const tria_calib *c, int32_t layer);

/* Writes the statistics of every layer to device arrays [n_layers][n_q_heads]
 * [head_dim/2] fp32 (q_abs may be NULL); a layer with no tokens gives zeros.
 * Stream-ordered; the accumulators keep their sums (more adds may follow). */
int tria_calib_finish(tria_calib *c, float *q_re, float *q_im, float *q_abs, float *norm_w,
                      hipStream_t stream);

void tria_calib_free(tria_calib *c);

/* Waits for the whole device, then reports and clears the context's device
 * error word: TRIA_OK, or TRIA_E_DEVICE if a compaction launched through this
 * context gave up one of its bounded waits since the last call (its output
 * is then not trustworthy).  A diagnostic call: it synchronises. */
int tria_device_status(tria_ctx *ctx);

/* Per-kernel timing of the passes run through a context (a trace facility,
 * off by default).  While enabled, every score, select and compaction launch
 * made by the entry points above is bracketed by HIP events recorded on the
 * caller's stream, which every kernel of a pass runs on.  At most
 * TRIA_TIMED_MAX launches are recorded between two
 * reads; later ones are counted in the read's return value and not timed.
 * enable: 1 turns timing on, 0 off (pending records are discarded). */
#define TRIA_TIMED_MAX 256
#define TRIA_STAGE_SCORE 0
#define TRIA_STAGE_SELECT 1
#define TRIA_STAGE_COMPACT 2
int tria_timing_enable(tria_ctx *ctx, int32_t enable);

/* Wait for the recorded launches, add their durations (ms) and counts per
 * stage into ms[3] and launches[3] (indexed by TRIA_STAGE_*; both host,
 * written), and clear the record.  Returns the number of launches that were
 * not timed (>= 0) or an error code. */
int tria_timing_read(tria_ctx *ctx, double *ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* TRIA_H */
