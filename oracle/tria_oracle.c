/*
 * tria_oracle.c -- plain CPU reference of the TriAttention KV-cache eviction
 * pass (score -> aggregate -> select -> compact).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library) never calls it and shares no code with it.
 *
 * Everything is computed in fp64, one (layer, KV head) unit at a time, in the
 * order the sources describe it, with no blocking or fusion.  The only
 * parallelism is an OpenMP loop over independent units.
 *
 * Sources (web pages; cited by title and section):
 *   [WL]  "TriAttention Native C++ Worklog" (TensorRT-Model-Connect).
 *   [LC]  llama.cpp docs page "TriAttention KV-Cache Eviction (--triattention)".
 *
 * Notation: L layers, Hkv KV heads, Hq query heads, G = Hq/Hkv, hd head dim,
 * F = hd/2 RoPE frequency pairs, n cached rows of one unit, B budget, S sink,
 * W window, D offset set, p reference position.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_KV_F16 0
#define ORC_KV_Q8_0 1

/* ------------------------------------------------------------------------ */
/* Key-row decoding.                                                          */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 -> double, written out from the format definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits). Exact. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal (or zero): m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Size in bytes of one stored row of head_dim values.
 * f16: 2 bytes per value.  q8_0: blocks of 32 values, each block stored as an
 * fp16 scale followed by 32 signed 8-bit integers (34 bytes) -- the K cache
 * type the HIP/Vulkan scorers of [LC] read (section 4, "GPU scoring
 * requirements"; section 5, "Phase C"). */
int64_t orc_row_bytes(int kv_type, int hd)
{
    if (kv_type == ORC_KV_F16) return 2 * (int64_t)hd;
    if (kv_type == ORC_KV_Q8_0) return 34 * (int64_t)(hd / 32);
    return -1;
}

/* Decode one stored key row into hd doubles.  q8_0 value = scale * q. */
int orc_decode_row(int kv_type, const uint8_t *row, int hd, double *out)
{
    if (kv_type == ORC_KV_F16) {
        for (int d = 0; d < hd; d++) {
            uint16_t h = (uint16_t)(row[2 * d] | (row[2 * d + 1] << 8));
            out[d] = orc_half_to_double(h);
        }
        return 0;
    }
    if (kv_type == ORC_KV_Q8_0) {
        for (int b = 0; b < hd / 32; b++) {
            const uint8_t *blk = row + 34 * b;
            double scale = orc_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int i = 0; i < 32; i++) out[32 * b + i] = scale * (double)(int8_t)blk[2 + i];
        }
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------ */
/* Query-side trigonometric term.                                             */
/* ------------------------------------------------------------------------ */

/* RoPE frequency of pair f: theta^(-2f/hd). */
double orc_omega(double theta, int hd, int f)
{
    return pow(theta, -2.0 * (double)f / (double)hd);
}

/* Mean over the offset set D of the future-query phase, per pair:
 *   A_f = (1/|D|) * sum_{delta in D} exp(i * omega_f * (p + delta)).
 * p is the absolute position of the newest cached token, never the cached
 * row count ([WL], "2026-04-18: later-compaction absolute-position bug
 * isolated and fixed").  The phase is applied to the query side only
 * ([WL], "Phase 9: final root cause - native scorer used the wrong
 * formulation"). */
void orc_offset_mean(double theta, int hd, int64_t p, const int64_t *offsets, int n_off,
                     double *a_re, double *a_im)
{
    int F = hd / 2;
    for (int f = 0; f < F; f++) {
        double w = orc_omega(theta, hd, f);
        double sr = 0.0, si = 0.0;
        for (int t = 0; t < n_off; t++) {
            double ang = w * (double)(p + offsets[t]);
            sr += cos(ang);
            si += sin(ang);
        }
        a_re[f] = sr / (double)n_off;
        a_im[f] = si / (double)n_off;
    }
}

/* ------------------------------------------------------------------------ */
/* Raw per-query-head score of one unit.                                      */
/* ------------------------------------------------------------------------ */

/* For the G query heads that share one KV head, and every cached row r:
 *
 *   s_j(r) = sum_f Re( qbar_{j,f} * A_f * conj(K_f(r)) ) + sum_f w_{j,f} |K_f(r)|
 *
 * with K_f = k[f] + i*k[f+F] (rotate-half / NEOX pairing of the stored,
 * already-rotated key).  The first sum scores the stored rotated key directly
 * against the phase-shifted mean query; the second is the additive term on
 * |K_rot| ([WL], "Phase 9 ..."; [LC] section 5, "Phase C": per-head q_mean
 * and q_abs statistics).
 *
 * k_rows: n rows of row_stride bytes; q_re/q_im/w: [G][F] statistics of the
 * unit's query heads; raw: output [n][G]. */
int orc_raw_scores_unit(int kv_type, const uint8_t *k_rows, int64_t row_stride, int64_t n,
                        int hd, int G, const float *q_re, const float *q_im, const float *w,
                        double theta, int64_t p, const int64_t *offsets, int n_off, double *raw)
{
    int F = hd / 2;
    double *a_re = (double *)malloc(sizeof(double) * F);
    double *a_im = (double *)malloc(sizeof(double) * F);
    double *c_re = (double *)malloc(sizeof(double) * F * G);
    double *c_im = (double *)malloc(sizeof(double) * F * G);
    double *k = (double *)malloc(sizeof(double) * hd);
    if (!a_re || !a_im || !c_re || !c_im || !k) {
        free(a_re); free(a_im); free(c_re); free(c_im); free(k);
        return -1;
    }
    orc_offset_mean(theta, hd, p, offsets, n_off, a_re, a_im);
    /* C_{j,f} = qbar_{j,f} * A_f (complex product). */
    for (int j = 0; j < G; j++) {
        for (int f = 0; f < F; f++) {
            double qr = q_re[j * F + f], qi = q_im[j * F + f];
            c_re[j * F + f] = qr * a_re[f] - qi * a_im[f];
            c_im[j * F + f] = qr * a_im[f] + qi * a_re[f];
        }
    }
    for (int64_t r = 0; r < n; r++) {
        orc_decode_row(kv_type, k_rows + r * row_stride, hd, k);
        for (int j = 0; j < G; j++) {
            double trig = 0.0, norm = 0.0;
            for (int f = 0; f < F; f++) {
                double kre = k[f], kim = k[f + F];
                /* Re(C * conj(K)) = Cre*Kre + Cim*Kim */
                trig += c_re[j * F + f] * kre + c_im[j * F + f] * kim;
                norm += (double)w[j * F + f] * sqrt(kre * kre + kim * kim);
            }
            raw[r * G + j] = trig + norm;
        }
    }
    free(a_re); free(a_im); free(c_re); free(c_im); free(k);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* GQA aggregation: per-head z-normalisation, then max over the group.        */
/* ------------------------------------------------------------------------ */

/* [LC] section 5, "Phase C": each query head's scores are z-normalised on
 * their own, then the KV head's score is the max over its query heads.
 * Population statistics over every cached row of the unit whose score is
 * finite; sigma = 0 gives z = 0.  A row with any non-finite head score gets
 * agg = -inf (evicted unless protected).  mu/sigma: optional [G] outputs. */
void orc_aggregate_unit(const double *raw, int64_t n, int G, double *agg, double *mu_out,
                        double *sigma_out)
{
    double *mu = (double *)malloc(sizeof(double) * (G > 0 ? G : 1));
    double *sg = (double *)malloc(sizeof(double) * (G > 0 ? G : 1));
    for (int j = 0; j < G; j++) {
        double sum = 0.0, lo = INFINITY, hi = -INFINITY;
        int64_t cnt = 0;
        for (int64_t r = 0; r < n; r++) {
            double s = raw[r * G + j];
            if (isfinite(s)) {
                sum += s;
                cnt++;
                lo = s < lo ? s : lo;
                hi = s > hi ? s : hi;
            }
        }
        double m = cnt ? sum / (double)cnt : 0.0;
        double ss = 0.0;
        for (int64_t r = 0; r < n; r++) {
            double s = raw[r * G + j];
            if (isfinite(s)) ss += (s - m) * (s - m);
        }
        /* Equal scores have sigma = 0 exactly; the rounding of the mean must not
         * turn them into a tiny sigma (which would give z = +-1). */
        if (cnt && lo == hi) {
            m = lo;
            ss = 0.0;
        }
        mu[j] = m;
        sg[j] = cnt ? sqrt(ss / (double)cnt) : 0.0;
        if (mu_out) mu_out[j] = mu[j];
        if (sigma_out) sigma_out[j] = sg[j];
    }
    for (int64_t r = 0; r < n; r++) {
        double best = -INFINITY;
        int bad = 0;
        for (int j = 0; j < G; j++) {
            double s = raw[r * G + j];
            if (!isfinite(s)) { bad = 1; break; }
            double z = sg[j] > 0.0 ? (s - mu[j]) / sg[j] : 0.0;
            if (j == 0 || z > best) best = z;
        }
        agg[r] = bad ? -INFINITY : best;
    }
    free(mu);
    free(sg);
}

/* ------------------------------------------------------------------------ */
/* Selection.                                                                 */
/* ------------------------------------------------------------------------ */

/* Protected rows: the first S rows (attention sinks) and the last W rows
 * (recent window) ([LC] section 5, "Phase B", step 2; section 1 flag table).
 * Returns the number of protected rows and the candidate range
 * [*cand_lo, *cand_hi). */
int64_t orc_protected(int64_t n, int64_t sink, int64_t window, int64_t *cand_lo, int64_t *cand_hi)
{
    int64_t s_end = sink < n ? sink : n;
    int64_t w_start = n - window;
    if (w_start < s_end) w_start = s_end;
    *cand_lo = s_end;
    *cand_hi = w_start;
    return s_end + (n - w_start);
}

/* Rows kept by one pass.  Budget >= n keeps everything.  Otherwise the budget
 * counts the protected rows, so kept = budget ([WL], "Compaction schedule"
 * logs: kept rows equal the KV budget), but never fewer than the protected
 * rows.  Returns -1 on negative arguments. */
int64_t orc_kept_count(int64_t n, int64_t budget, int64_t sink, int64_t window)
{
    if (n < 0 || budget < 0 || sink < 0 || window < 0) return -1;
    if (budget >= n) return n;
    int64_t lo, hi;
    int64_t np = orc_protected(n, sink, window, &lo, &hi);
    return budget > np ? budget : np;
}

typedef struct {
    double key;
    int64_t idx;
} orc_cand;

/* Sort order: score descending, then row index ascending (lower row wins a
 * tie). */
static int orc_cand_cmp(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    if (x->idx < y->idx) return -1;
    if (x->idx > y->idx) return 1;
    return 0;
}

/* [LC] section 5, "Phase B", steps 2-3: protect sink and window, sort the
 * remaining rows by score and evict the lowest down to the budget.
 * keep_idx: output, ascending row indices; returns the kept count. */
int64_t orc_select_unit(const double *agg, int64_t n, int64_t budget, int64_t sink,
                        int64_t window, int32_t *keep_idx)
{
    int64_t K = orc_kept_count(n, budget, sink, window);
    if (K < 0) return -1;
    if (K == n) {
        for (int64_t r = 0; r < n; r++) keep_idx[r] = (int32_t)r;
        return n;
    }
    int64_t lo, hi;
    int64_t np = orc_protected(n, sink, window, &lo, &hi);
    int64_t k = K - np; /* candidates to keep */
    int64_t nc = hi - lo;
    unsigned char *keep = (unsigned char *)calloc((size_t)(n > 0 ? n : 1), 1);
    orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(nc > 0 ? nc : 1));
    if (!keep || !c) { free(keep); free(c); return -1; }
    for (int64_t r = 0; r < lo; r++) keep[r] = 1;
    for (int64_t r = hi; r < n; r++) keep[r] = 1;
    for (int64_t i = 0; i < nc; i++) {
        c[i].key = agg[lo + i];
        c[i].idx = lo + i;
    }
    qsort(c, (size_t)nc, sizeof(orc_cand), orc_cand_cmp);
    for (int64_t i = 0; i < k; i++) keep[c[i].idx] = 1;
    int64_t out = 0;
    for (int64_t r = 0; r < n; r++)
        if (keep[r]) keep_idx[out++] = (int32_t)r;
    free(keep);
    free(c);
    return out;
}

/* ------------------------------------------------------------------------ */
/* Compaction.                                                                */
/* ------------------------------------------------------------------------ */

/* Order-preserving gather of the kept rows to the front of the unit's
 * storage, no gaps ([LC] section 5, "Phase B", step 4; [WL], "What was
 * implemented": GPU gather/repack, and the exact-gather checks).  Done
 * through a temporary copy: dst[d] = src[keep_idx[d]]. */
int orc_compact_rows(uint8_t *rows, int64_t row_bytes, const int32_t *keep_idx, int64_t K)
{
    uint8_t *tmp = (uint8_t *)malloc((size_t)(K * row_bytes > 0 ? K * row_bytes : 1));
    if (!tmp) return -1;
    for (int64_t d = 0; d < K; d++)
        memcpy(tmp + d * row_bytes, rows + (int64_t)keep_idx[d] * row_bytes, (size_t)row_bytes);
    memcpy(rows, tmp, (size_t)(K * row_bytes));
    free(tmp);
    return 0;
}

/* Hole-filling compaction (a variant; the order-preserving gather above is
 * the pages' rule).  [LC] section 5, "Phase B" step 4 asks only that the kept
 * rows end up packed in place with no gaps; the cache's cells carry their
 * positions.  The variant keeps the layout the selection relies on -- the
 * sink rows stay first, the newest rows stay last and in order -- and moves
 * as few rows as that allows:
 *   R = the trailing run: the kept rows n-|R| .. n-1 (the longest run of
 *       kept rows that ends at row n-1; it holds the protected window);
 *   holes = the rows below K-|R| that are not kept, ascending;
 *   tails = the kept rows at or above K-|R| that are not in R, ascending
 *           (as many as there are holes);
 *   hole i <- tail i, then the run moves to rows K-|R| .. K-1, in order.
 * Rows kept below K-|R| (the sinks among them) do not move.  Positions move
 * with their rows, so rows [0, K) hold exactly the kept rows.
 * keep_idx: ascending kept rows (K of them) of a unit of n rows.
 * Returns the number of rows written (moves), or -1. */
int64_t orc_compact_holefill(uint8_t *rows, int64_t row_bytes, const int32_t *keep_idx,
                             int64_t K, int64_t n)
{
    if (K >= n || K <= 0) return 0;
    int64_t run = 0;
    while (run < K && keep_idx[K - 1 - run] == n - 1 - run) run++;
    int64_t lim = K - run; /* rows [0, lim) hold the kept rows outside the run */
    unsigned char *kept = (unsigned char *)calloc((size_t)n, 1);
    if (!kept) return -1;
    for (int64_t e = 0; e < K; e++) kept[keep_idx[e]] = 1;
    int64_t moves = 0;
    int64_t h = 0;                                     /* next hole candidate */
    for (int64_t e = 0; e < K - run; e++) {            /* kept rows outside the run */
        int64_t src = keep_idx[e];
        if (src < lim) continue;                       /* already in place */
        while (kept[h]) h++;                           /* next hole below lim */
        memcpy(rows + h * row_bytes, rows + src * row_bytes, (size_t)row_bytes);
        h++;
        moves++;
    }
    /* the run moves down by n - K rows, in ascending order (an overlapping
     * move towards lower rows is safe in this order) */
    for (int64_t j = 0; j < run; j++) {
        int64_t src = n - run + j, dst = lim + j;
        if (src != dst) {
            memmove(rows + dst * row_bytes, rows + src * row_bytes, (size_t)row_bytes);
            moves++;
        }
    }
    free(kept);
    return moves;
}

/* ------------------------------------------------------------------------ */
/* Whole pass over a contiguous cache [L][Hkv][cap][row].                     */
/* ------------------------------------------------------------------------ */

/* Keep-set sharing.  ORC_KEEP_UNIT: every (layer, KV head) unit selects on its
 * own.  ORC_KEEP_KV_HEAD: one keep set per KV head, shared by all layers ([WL]
 * "Later correction: selector and compaction are now cleared ...": keep sets
 * compared per head, 8 of 8, and one per-head index list gathered in all 36
 * layers; the worklog names a cross-layer aggregation step).  ORC_KEEP_GLOBAL:
 * one keep set for the whole cache ([LC] section 5, "Phase C", the global
 * z-normalisation shader; the cache's cells hold every layer and head).
 * Neither page writes out the cross-unit reduction; it is read as the same
 * rule as the GQA group's: every member query head is z-normalised over its
 * own unit's rows, and the group score of a row is the max of those z-scores
 * over all member heads (-inf if any member score is not finite). */
#define ORC_COMPACT_ORDERED 0
#define ORC_COMPACT_HOLEFILL 1
#define ORC_KEEP_UNIT 0
#define ORC_KEEP_KV_HEAD 1
#define ORC_KEEP_GLOBAL 2

/* Group of unit (l, g) and number of groups under a keep mode. */
/* Wall-clock seconds of the stages of the last orc_evict_ex call (benchmark
 * reporting only): [0] raw scores and per-unit z-normalised maxima, [1] group
 * scores and selection, [2] compaction. */
static double orc_stage_s[3];

static double orc_now(void)
{
#ifdef _OPENMP
    extern double omp_get_wtime(void);
    return omp_get_wtime();
#else
    return 0.0;
#endif
}

void orc_last_stage_seconds(double *out)
{
    for (int i = 0; i < 3; i++) out[i] = orc_stage_s[i];
}

static int orc_n_groups(int mode, int L, int Hkv)
{
    return mode == ORC_KEEP_UNIT ? L * Hkv : (mode == ORC_KEEP_KV_HEAD ? Hkv : 1);
}
static int orc_group_of(int mode, int Hkv, int u)
{
    return mode == ORC_KEEP_UNIT ? u : (mode == ORC_KEEP_KV_HEAD ? u % Hkv : 0);
}

/* One eviction pass over every (layer, KV head) unit.
 *   keep_mode : ORC_KEEP_UNIT, ORC_KEEP_KV_HEAD or ORC_KEEP_GLOBAL.
 *   compact_mode : ORC_COMPACT_ORDERED (the gather) or ORC_COMPACT_HOLEFILL.
 *   k, v, pos : host copies, [L][Hkv][cap] rows; compacted in place.
 *   q_re, q_im, w : statistics [L][Hq][F]; query head h = g*G + j belongs to
 *                   KV head g (contiguous GQA grouping).
 *   keep_idx  : output [L][Hkv][K] (may be NULL); a shared keep set is written
 *               for every member unit.
 *   raw       : output [L][Hkv][n][G] (may be NULL)
 *   agg       : output [L][Hkv][n] (may be NULL): the score the unit's keep set
 *               was selected on (its group's score under a shared mode).
 * Returns the kept count K, or -1. */
int64_t orc_evict_ex(int keep_mode, int compact_mode, int k_type, int v_type, int L, int Hkv,
                     int Hq, int hd, double theta, const int64_t *offsets, int n_off, uint8_t *k,
                     uint8_t *v, int32_t *pos, int64_t cap, int64_t n, int64_t budget,
                     int64_t sink, int64_t window, const float *q_re, const float *q_im,
                     const float *w, int32_t *keep_idx, double *raw, double *agg, int do_compact)
{
    int G = Hq / Hkv;
    int F = hd / 2;
    int U = L * Hkv;
    int64_t kb = orc_row_bytes(k_type, hd), vb = orc_row_bytes(v_type, hd);
    int64_t K = orc_kept_count(n, budget, sink, window);
    if (K < 0 || kb < 0 || vb < 0 || n > cap) return -1;
    if (keep_mode < ORC_KEEP_UNIT || keep_mode > ORC_KEEP_GLOBAL) return -1;
    if (compact_mode != ORC_COMPACT_ORDERED && compact_mode != ORC_COMPACT_HOLEFILL) return -1;
    int NG = orc_n_groups(keep_mode, L, Hkv);
    int64_t nn = n > 0 ? n : 1;
    double *rs = raw ? raw : (double *)malloc(sizeof(double) * (size_t)(U * nn * G));
    double *ua = (double *)malloc(sizeof(double) * (size_t)(U * nn)); /* per-unit GQA max */
    double *ga = (double *)malloc(sizeof(double) * (size_t)(NG * nn)); /* group score */
    int32_t *gk = (int32_t *)malloc(sizeof(int32_t) * (size_t)(NG * nn));
    int failed = !rs || !ua || !ga || !gk;
    double t0 = orc_now(), t1 = t0, t2 = t0;
    if (!failed && n > 0) {
        /* 1. raw scores and the unit's z-normalised GQA max */
#pragma omp parallel for schedule(dynamic, 1)
        for (int u = 0; u < U; u++) {
            int l = u / Hkv, g = u % Hkv;
            uint8_t *ku = k + (int64_t)u * cap * kb;
            int32_t *pu = pos + (int64_t)u * cap;
            int64_t stat = ((int64_t)l * Hq + (int64_t)g * G) * F;
            int64_t p = pu[n - 1];
            int bad = orc_raw_scores_unit(k_type, ku, kb, n, hd, G, q_re + stat, q_im + stat,
                                          w + stat, theta, p, offsets, n_off,
                                          rs + (int64_t)u * n * G);
            orc_aggregate_unit(rs + (int64_t)u * n * G, n, G, ua + (int64_t)u * n, NULL, NULL);
            if (bad) {
#pragma omp atomic write
                failed = 1;
            }
        }
        t1 = orc_now();
        /* 2. group score: max over the member units' z-maxima (a unit's value is
         *    -inf exactly when one of its head scores is not finite, and then the
         *    group's is -inf too) */
        for (int64_t i = 0; i < (int64_t)NG * n; i++) ga[i] = 0.0;
        for (int gr = 0; gr < NG; gr++) {
            double *gs = ga + (int64_t)gr * n;
            int first = 1;
            for (int u = 0; u < U; u++) {
                if (orc_group_of(keep_mode, Hkv, u) != gr) continue;
                const double *us = ua + (int64_t)u * n;
                for (int64_t r = 0; r < n; r++) {
                    if (us[r] == -INFINITY || (!first && gs[r] == -INFINITY)) gs[r] = -INFINITY;
                    else if (first || us[r] > gs[r]) gs[r] = us[r];
                }
                first = 0;
            }
        }
        /* 3. one selection per group */
#pragma omp parallel for schedule(dynamic, 1)
        for (int gr = 0; gr < NG; gr++) {
            if (orc_select_unit(ga + (int64_t)gr * n, n, budget, sink, window,
                                gk + (int64_t)gr * nn) != K) {
#pragma omp atomic write
                failed = 1;
            }
        }
        t2 = orc_now();
        /* 4. every unit gathers its rows with its group's keep set */
#pragma omp parallel for schedule(dynamic, 1)
        for (int u = 0; u < U; u++) {
            int gr = orc_group_of(keep_mode, Hkv, u);
            const int32_t *ki = gk + (int64_t)gr * nn;
            int bad = 0;
            if (keep_idx) memcpy(keep_idx + (int64_t)u * K, ki, sizeof(int32_t) * (size_t)K);
            if (agg) memcpy(agg + (int64_t)u * n, ga + (int64_t)gr * n, sizeof(double) * (size_t)n);
            if (do_compact && !failed && compact_mode == ORC_COMPACT_HOLEFILL) {
                bad |= orc_compact_holefill(k + (int64_t)u * cap * kb, kb, ki, K, n) < 0;
                bad |= orc_compact_holefill(v + (int64_t)u * cap * vb, vb, ki, K, n) < 0;
                bad |= orc_compact_holefill((uint8_t *)(pos + (int64_t)u * cap), 4, ki, K, n) < 0;
            } else if (do_compact && !failed) {
                bad |= orc_compact_rows(k + (int64_t)u * cap * kb, kb, ki, K);
                bad |= orc_compact_rows(v + (int64_t)u * cap * vb, vb, ki, K);
                bad |= orc_compact_rows((uint8_t *)(pos + (int64_t)u * cap), 4, ki, K);
            }
            if (bad) {
#pragma omp atomic write
                failed = 1;
            }
        }
    }
    orc_stage_s[0] = t1 - t0;
    orc_stage_s[1] = t2 - t1;
    orc_stage_s[2] = orc_now() - t2;
    if (!raw) free(rs);
    free(ua);
    free(ga);
    free(gk);
    return failed ? -1 : K;
}

/* Order-preserving compaction (the pages' rule). */
int64_t orc_evict_mode(int keep_mode, int k_type, int v_type, int L, int Hkv, int Hq, int hd,
                       double theta, const int64_t *offsets, int n_off, uint8_t *k, uint8_t *v,
                       int32_t *pos, int64_t cap, int64_t n, int64_t budget, int64_t sink,
                       int64_t window, const float *q_re, const float *q_im, const float *w,
                       int32_t *keep_idx, double *raw, double *agg, int do_compact)
{
    return orc_evict_ex(keep_mode, ORC_COMPACT_ORDERED, k_type, v_type, L, Hkv, Hq, hd, theta,
                        offsets, n_off, k, v, pos, cap, n, budget, sink, window, q_re, q_im, w,
                        keep_idx, raw, agg, do_compact);
}

/* The per-unit pass (each unit selects on its own). */
int64_t orc_evict(int k_type, int v_type, int L, int Hkv, int Hq, int hd, double theta,
                  const int64_t *offsets, int n_off, uint8_t *k, uint8_t *v, int32_t *pos,
                  int64_t cap, int64_t n, int64_t budget, int64_t sink, int64_t window,
                  const float *q_re, const float *q_im, const float *w, int32_t *keep_idx,
                  double *raw, double *agg, int do_compact)
{
    return orc_evict_mode(ORC_KEEP_UNIT, k_type, v_type, L, Hkv, Hq, hd, theta, offsets, n_off,
                          k, v, pos, cap, n, budget, sink, window, q_re, q_im, w, keep_idx, raw,
                          agg, do_compact);
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the cache.                                          */
/* ------------------------------------------------------------------------ */

/* One decode step's attention for one (layer, KV head) unit: the G query
 * heads of the KV head ([LC] section 4's GQA grouping, query head g*G + j)
 * attend to the unit's n cached rows -- the rows an eviction pass leaves,
 * whatever their order ([WL] "What was implemented": decode continues on the
 * compacted cache; attention weights do not depend on the row order):
 *   s_j(r) = scale * q_j . k_r,   p_j(r) = exp(s_j(r)) / sum_r' exp(s_j(r')),
 *   out_j  = sum_r p_j(r) v_r.
 * q: [G][hd]; k_rows / v_rows: n stored rows (decoded exactly); out: [G][hd].
 * Returns 0, or -1 on a bad row type. */
int orc_decode_attention_unit(int k_type, int v_type, const uint8_t *k_rows,
                              const uint8_t *v_rows, int64_t n, int hd, int G, const double *q,
                              double scale, double *out)
{
    int64_t kb = orc_row_bytes(k_type, hd), vb = orc_row_bytes(v_type, hd);
    if (kb < 0 || vb < 0) return -1;
    double *kd = (double *)malloc(sizeof(double) * (size_t)hd);
    double *vd = (double *)malloc(sizeof(double) * (size_t)hd);
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)G);
    if (!kd || !vd || !s) { free(kd); free(vd); free(s); return -1; }
    for (int64_t r = 0; r < n; r++) {
        orc_decode_row(k_type, k_rows + r * kb, hd, kd);
        for (int j = 0; j < G; j++) {
            double d = 0.0;
            for (int e = 0; e < hd; e++) d += q[j * hd + e] * kd[e];
            s[r * G + j] = scale * d;
        }
    }
    for (int j = 0; j < G; j++) {
        double mx = -INFINITY;
        for (int64_t r = 0; r < n; r++) mx = s[r * G + j] > mx ? s[r * G + j] : mx;
        double den = 0.0;
        for (int64_t r = 0; r < n; r++) den += exp(s[r * G + j] - mx);
        for (int e = 0; e < hd; e++) out[j * hd + e] = 0.0;
        for (int64_t r = 0; r < n; r++) {
            double pr = exp(s[r * G + j] - mx) / den;
            orc_decode_row(v_type, v_rows + r * vb, hd, vd);
            for (int e = 0; e < hd; e++) out[j * hd + e] += pr * vd[e];
        }
    }
    free(kd);
    free(vd);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Calibration statistics.                                                    */
/* ------------------------------------------------------------------------ */

/* [LC] section 2, "Generating a .tria file": the generator hooks each layer's
 * pre-RoPE query tensor during forward passes and accumulates, per query head
 * and frequency pair, the mean query direction and a per-frequency weight
 * ([LC] section 5, "Phase C": per-head q_mean / q_abs arrays).  With the
 * query pair q_f = q[f] + i q[f + hd/2] (NEOX halves) of every token t:
 *   q_mean_f = (1/T) sum_t q_f(t)        (complex)
 *   q_abs_f  = (1/T) sum_t |q_f(t)|
 *   w_f      = q_abs_f - |q_mean_f|      (the norm-term weight: zero when
 *              every token's pair points the same way, q_abs when the
 *              directions cancel; [WL] "Phase 9" keeps this additive term
 *              on |K_rot|)
 * q: T tokens x H heads x hd values (row-major, fp64); outputs [H][hd/2]. */
void orc_calib_stats(const double *q, int64_t T, int H, int hd, double *q_re, double *q_im,
                     double *q_abs, double *w)
{
    int F = hd / 2;
    for (int h = 0; h < H; h++) {
        for (int f = 0; f < F; f++) {
            double sr = 0.0, si = 0.0, sa = 0.0;
            for (int64_t t = 0; t < T; t++) {
                const double *row = q + (t * H + h) * (int64_t)hd;
                double re = row[f], im = row[f + F];
                sr += re;
                si += im;
                sa += sqrt(re * re + im * im);
            }
            int64_t o = (int64_t)h * F + f;
            double mr = T > 0 ? sr / (double)T : 0.0;
            double mi = T > 0 ? si / (double)T : 0.0;
            double ma = T > 0 ? sa / (double)T : 0.0;
            q_re[o] = mr;
            q_im[o] = mi;
            q_abs[o] = ma;
            w[o] = ma - sqrt(mr * mr + mi * mi);
        }
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
