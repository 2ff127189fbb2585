/*
 * Sanitizer driver for the host side of libtria (tests/test_sanitizers.py
 * builds the library with host-only -fsanitize=address,undefined and links
 * this against it): calls the entry points that run on the host alone -- sizes,
 * kept counts, decode-loop policy, argument and eligibility checks, error
 * strings -- with valid, edge and invalid arguments, so that any out-of-bounds
 * access or undefined arithmetic in the host code stops the run.  Nothing here
 * launches a kernel; no GPU is needed.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tria.h"

static uint64_t s = 0x9E3779B97F4A7C15ull;
static int64_t rnd(int64_t m)
{
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return (int64_t)((s >> 11) % (uint64_t)(m > 0 ? m : 1));
}

int main(void)
{
    int64_t acc = 0;
    for (int code = -8; code <= 2; code++) acc += (int64_t)strlen(tria_strerror(code));
    for (int t = -1; t <= 2; t++)
        for (int hd = -32; hd <= 320; hd += 16) acc += tria_row_bytes(t, hd);
    for (int i = 0; i < 200000; i++) {
        int64_t n = rnd(5) == 0 ? rnd(4) - 1 : rnd(1 << 20);
        acc += tria_kept_count(n, rnd(n + 3) - (rnd(50) == 0), rnd(600), rnd(n + 2));
    }
    /* decode-loop policy over many states and policies, including bad ones */
    for (int i = 0; i < 200000; i++) {
        tria_policy p;
        p.trigger = (int32_t)rnd(3);
        p.protect_prefill = (int32_t)rnd(2);
        p.budget = rnd(10000) - 2;
        p.divide_length = rnd(2000) - 2;
        p.interval = rnd(300) - 2;
        p.sink = rnd(20) - 1;
        p.window = rnd(1000) - 1;
        tria_decode_state st;
        st.n_prompt = rnd(5000);
        st.n_rows = st.n_prompt + rnd(20000) - 3;
        st.steps = rnd(3000) - 1;
        st.passes = rnd(10);
        int64_t b = 0, sk = 0, w = 0;
        acc += tria_policy_due(&p, &st, &b, &sk, &w) + b + sk + w;
        acc += tria_policy_peak_rows(&p, rnd(5000) - 1);
    }
    acc += tria_policy_due(NULL, NULL, NULL, NULL, NULL);
    acc += tria_policy_peak_rows(NULL, 0);
    /* argument checks that return before any device work */
    tria_cache c;
    memset(&c, 0, sizeof(c));
    acc += tria_score(NULL, &c, 0, NULL, 0);
    acc += tria_select(NULL, NULL, 0, 0, 0, 0, NULL, NULL, 0);
    acc += tria_compact(NULL, &c, 0, NULL, 0, 0);
    acc += tria_evict(NULL, &c, 0, 0, 0, 0, 0);
    acc += tria_evict_noalloc(NULL, &c, 0, 0, 0, 0, 0);
    acc += tria_evict_paged_batch(NULL, NULL, 1, NULL, NULL, 0, 0, NULL, 0);
    acc += tria_decode_attention(NULL, &c, 0, NULL, 1.0f, NULL, 0);
    acc += tria_set_keep_mode(NULL, 0) + tria_set_compaction(NULL, 0);
    acc += tria_set_compaction_workgroups(NULL, 0) + tria_device_status(NULL);
    acc += tria_timing_enable(NULL, 1) + tria_timing_read(NULL, NULL, NULL);
    acc += tria_last_hip_error(NULL);
    acc += tria_calib_create(NULL, 1, 1, 2);
    acc += tria_calib_add(NULL, 0, NULL, 0, 0, 0, 0);
    acc += tria_calib_add_layers(NULL, 0, 1, NULL, 0, 0, 0, 0, 0);
    acc += tria_calib_tokens(NULL, 0) + tria_calib_finish(NULL, NULL, NULL, NULL, NULL, 0);
    tria_calib_free(NULL);
    tria_free(NULL);
    /* the eligibility gate and descriptor checks (all refused on the host) */
    static float stats[4096];
    int64_t offs[8] = {1, 2, 4, 8, 16, 32, 64, 128};
    for (int i = 0; i < 20000; i++) {
        tria_model_desc d;
        d.n_layers = (int32_t)rnd(4) - 1;
        d.n_kv_heads = (int32_t)rnd(5) - 1;
        d.n_q_heads = (int32_t)rnd(140) - 1;
        d.head_dim = (int32_t)(rnd(20) * 16) - 16;
        d.k_type = (int32_t)rnd(4) - 1;
        d.v_type = (int32_t)rnd(4) - 1;
        d.rope_theta = rnd(3) == 0 ? 1.0 : 1e6;
        d.n_offsets = (int32_t)rnd(9) - 1;
        d.offsets = rnd(10) == 0 ? NULL : offs;
        if (d.n_layers >= 1 && d.n_kv_heads >= 1 && d.n_q_heads >= 1 && d.n_offsets >= 1 &&
            d.offsets && d.rope_theta > 1.0 && d.n_q_heads % d.n_kv_heads == 0 &&
            d.n_q_heads / d.n_kv_heads <= 64 && d.head_dim >= 32 && d.head_dim <= 256 &&
            d.head_dim % 32 == 0 && d.k_type >= 0 && d.k_type <= 1 && d.v_type >= 0 &&
            d.v_type <= 1)
            d.head_dim = 100; /* keep every call off the device: make it ineligible */
        tria_ctx *ctx = NULL;
        acc += tria_load_stats(&ctx, &d, stats, stats, stats, 0);
        if (ctx) tria_free(ctx);
    }
    acc += tria_load_stats(NULL, NULL, NULL, NULL, NULL, 0);
    printf("host driver ok %lld\n", (long long)(acc != 0));
    return 0;
}
