/*
 * Sanitizer driver for the CPU oracle (tests/test_sanitizers.py builds it with
 * -fsanitize=address,undefined together with oracle/tria_oracle.c): calls every
 * entry point on small seeded inputs, edge sizes included, so that any
 * out-of-bounds access, use of freed memory or undefined arithmetic in the
 * oracle stops the run.  It checks no numbers; the pins do that.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_half_to_double(uint16_t h);
int64_t orc_row_bytes(int kv_type, int hd);
int orc_decode_row(int kv_type, const uint8_t *row, int hd, double *out);
double orc_omega(double theta, int hd, int f);
void orc_offset_mean(double theta, int hd, int64_t p, const int64_t *offsets, int n_off,
                     double *a_re, double *a_im);
int orc_raw_scores_unit(int kv_type, const uint8_t *k_rows, int64_t row_stride, int64_t n, int hd,
                        int G, const float *q_re, const float *q_im, const float *w, double theta,
                        int64_t p, const int64_t *offsets, int n_off, double *raw);
void orc_aggregate_unit(const double *raw, int64_t n, int G, double *agg, double *mu_out,
                        double *sigma_out);
int64_t orc_kept_count(int64_t n, int64_t budget, int64_t sink, int64_t window);
int64_t orc_select_unit(const double *agg, int64_t n, int64_t budget, int64_t sink,
                        int64_t window, int32_t *keep_idx);
int orc_compact_rows(uint8_t *rows, int64_t row_bytes, const int32_t *keep_idx, int64_t K);
int64_t orc_compact_holefill(uint8_t *rows, int64_t row_bytes, const int32_t *keep_idx, int64_t K,
                             int64_t n);
int64_t orc_evict_ex(int keep_mode, int compact_mode, int k_type, int v_type, int L, int Hkv,
                     int Hq, int hd, double theta, const int64_t *offsets, int n_off, uint8_t *k,
                     uint8_t *v, int32_t *pos, int64_t cap, int64_t n, int64_t budget,
                     int64_t sink, int64_t window, const float *q_re, const float *q_im,
                     const float *w, int32_t *keep_idx, double *raw, double *agg, int do_compact);
int orc_decode_attention_unit(int k_type, int v_type, const uint8_t *k_rows,
                              const uint8_t *v_rows, int64_t n, int hd, int G, const double *q,
                              double scale, double *out);
void orc_calib_stats(const double *q, int64_t T, int H, int hd, double *q_re, double *q_im,
                     double *q_abs, double *w);
void orc_last_stage_seconds(double *out);

static uint64_t rng_state = 88172645463325252ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 11);
}
static double urand(void) { return (rnd() & 0xffffff) / (double)0x1000000; }

/* Random row bytes of a type: fp16 values in (-4, 4), or q8_0 blocks with a
 * small finite scale (occasionally a non-finite one). */
static void fill_rows(int type, uint8_t *rows, int64_t n, int hd)
{
    int64_t rb = orc_row_bytes(type, hd);
    for (int64_t r = 0; r < n; r++) {
        uint8_t *row = rows + r * rb;
        if (type == 0) {
            for (int d = 0; d < hd; d++) {
                uint16_t h = (uint16_t)(0x3000 + (rnd() % 0x1800)) | (uint16_t)((rnd() & 1) << 15);
                memcpy(row + 2 * d, &h, 2);
            }
        } else {
            for (int b = 0; b < hd / 32; b++) {
                uint16_t dsc = (rnd() % 97 == 0) ? 0x7c00 : (uint16_t)(0x2000 + (rnd() % 0x1000));
                memcpy(row + 34 * b, &dsc, 2);
                for (int t = 0; t < 32; t++) row[34 * b + 2 + t] = (uint8_t)rnd();
            }
        }
    }
}

int main(void)
{
    volatile double sink_d = 0.0;
    for (uint32_t h = 0; h < 65536; h++) sink_d += isfinite(orc_half_to_double((uint16_t)h)) ? 1 : 0;
    const int hds[] = {32, 64, 96, 128, 256};
    const int64_t offs[] = {1, 2, 4, 8, 16, 32, 64, 128};
    for (int it = 0; it < 60; it++) {
        int hd = hds[rnd() % 5], F = hd / 2;
        int kt = rnd() & 1, vt = rnd() & 1;
        int L = 1 + rnd() % 2, Hkv = 1 + rnd() % 2, G = 1 + rnd() % 4, Hq = Hkv * G;
        int64_t n = (it % 7 == 0) ? (int64_t)(rnd() % 3) : (int64_t)(1 + rnd() % 700);
        int64_t cap = n + rnd() % 5;
        int64_t kb = orc_row_bytes(kt, hd), vb = orc_row_bytes(vt, hd);
        int64_t budget = rnd() % (n + 3), snk = rnd() % 9, win = rnd() % (n + 2);
        int n_off = 1 + rnd() % 8;
        size_t units = (size_t)L * Hkv;
        uint8_t *k = malloc(units * cap * kb + 1), *v = malloc(units * cap * vb + 1);
        int32_t *pos = malloc(units * cap * sizeof(int32_t) + 4);
        float *qr = malloc(sizeof(float) * L * Hq * F), *qi = malloc(sizeof(float) * L * Hq * F);
        float *w = malloc(sizeof(float) * L * Hq * F);
        for (size_t u = 0; u < units; u++) {
            fill_rows(kt, k + u * cap * kb, cap, hd);
            fill_rows(vt, v + u * cap * vb, cap, hd);
            for (int64_t r = 0; r < cap; r++) pos[u * cap + r] = (int32_t)(r + 5 * u);
        }
        for (int i = 0; i < L * Hq * F; i++) {
            qr[i] = (float)(urand() * 2 - 1);
            qi[i] = (float)(urand() * 2 - 1);
            w[i] = (float)urand();
        }
        int64_t K = orc_kept_count(n, budget, snk, win);
        int32_t *keep = malloc(sizeof(int32_t) * units * (K > 0 ? K : 1));
        double *raw = malloc(sizeof(double) * units * (n > 0 ? n : 1) * G);
        double *agg = malloc(sizeof(double) * units * (n > 0 ? n : 1));
        for (int mode = 0; mode < 3; mode++)
            for (int cm = 0; cm < 2; cm++)
                sink_d += (double)orc_evict_ex(mode, cm, kt, vt, L, Hkv, Hq, hd, 1e6, offs, n_off,
                                               k, v, pos, cap, n, budget, snk, win, qr, qi, w,
                                               keep, raw, agg, 1);
        /* the single-unit functions on the first unit */
        double *row = malloc(sizeof(double) * hd);
        if (n > 0) orc_decode_row(kt, k, hd, row);
        double are[128], aim[128];
        orc_offset_mean(1e6, hd, n + 3, offs, n_off, are, aim);
        sink_d += orc_omega(1e6, hd, F - 1);
        double *r1 = malloc(sizeof(double) * (n > 0 ? n : 1) * G);
        orc_raw_scores_unit(kt, k, kb, n, hd, G, qr, qi, w, 1e6, n + 2, offs, n_off, r1);
        double mu[8], sg[8];
        orc_aggregate_unit(r1, n, G, agg, mu, sg);
        if (n > 1) r1[0] = NAN;
        orc_aggregate_unit(r1, n, G, agg, mu, sg);
        int32_t *k1 = malloc(sizeof(int32_t) * (n > 0 ? n : 1));
        int64_t K1 = orc_select_unit(agg, n, budget, snk, win, k1);
        if (K1 > 0) {
            orc_compact_rows(k, kb, k1, K1);
            orc_compact_holefill(v, vb, k1, K1, n);
        }
        double *q = malloc(sizeof(double) * G * hd), *out = malloc(sizeof(double) * G * hd);
        for (int i = 0; i < G * hd; i++) q[i] = urand() - 0.5;
        orc_decode_attention_unit(kt, vt, k, v, n, hd, G, q, 0.1, out);
        int64_t T = 1 + rnd() % 40;
        double *qs = malloc(sizeof(double) * T * Hq * hd);
        double *s4 = malloc(sizeof(double) * 4 * Hq * F);
        for (int64_t i = 0; i < T * Hq * hd; i++) qs[i] = urand() - 0.5;
        orc_calib_stats(qs, T, Hq, hd, s4, s4 + Hq * F, s4 + 2 * Hq * F, s4 + 3 * Hq * F);
        double st[3];
        orc_last_stage_seconds(st);
        free(k); free(v); free(pos); free(qr); free(qi); free(w); free(keep); free(raw);
        free(agg); free(row); free(r1); free(k1); free(q); free(out); free(qs); free(s4);
    }
    printf("oracle driver ok %g\n", (double)(sink_d != 0.0));
    return 0;
}
