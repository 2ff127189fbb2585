// Decode-loop policy around the eviction pass: when a pass runs and with
// which arguments (host logic; the pass itself is tria_evict).
//
// "TriAttention Native C++ Worklog": the runtime compacts once the cache
// length reaches kv_budget + divide_length (section on the sample9 replay:
// cache_length_ grows only with decode appends, so prompt tokens are not
// counted; the logged schedule is 3200 -> 3072 rows every 128 steps at
// budget 3072), keeps a physical capacity above the logical budget and
// protects the prompt ("4. Separate physical cache limit from logical
// TriAttention budget", "Phase 6: overflow bug during prompt prefill").
// llama.cpp page "TriAttention KV-Cache Eviction (--triattention)": the
// evictor runs every --tri-interval decode steps, in decode only (section 1
// flags, section 5 "Phase B").
#include "tria_internal.h"

namespace {

bool policy_ok(const tria_policy* p) {
    if (!p) return false;
    if (p->trigger != TRIA_TRIGGER_THRESHOLD && p->trigger != TRIA_TRIGGER_INTERVAL) return false;
    if (p->budget < 1 || p->sink < 0 || p->window < 0) return false;
    if (p->trigger == TRIA_TRIGGER_THRESHOLD && p->divide_length < 1) return false;
    if (p->trigger == TRIA_TRIGGER_INTERVAL && p->interval < 1) return false;
    return true;
}

}  // namespace

extern "C" {

int tria_policy_due(const tria_policy* p, const tria_decode_state* st, int64_t* budget_rows,
                    int64_t* sink_rows, int64_t* window_rows) {
    if (!policy_ok(p) || !st || !budget_rows || !sink_rows || !window_rows) return TRIA_E_INVAL;
    if (st->n_rows < 0 || st->n_prompt < 0 || st->steps < 0) return TRIA_E_INVAL;
    // protected prompt rows are never evicted, so they are all still there
    if (p->protect_prefill && st->n_prompt > st->n_rows) return TRIA_E_INVAL;
    const int64_t fixed = p->protect_prefill ? st->n_prompt : 0;
    const int64_t counted = st->n_rows - fixed;
    bool due;
    if (p->trigger == TRIA_TRIGGER_THRESHOLD)
        due = counted >= p->budget + p->divide_length;
    else
        due = st->steps >= p->interval && counted > p->budget;
    if (!due) return 0;
    *budget_rows = p->budget + fixed;
    *sink_rows = p->protect_prefill && st->n_prompt > p->sink ? st->n_prompt : p->sink;
    *window_rows = p->window;
    return 1;
}

int64_t tria_policy_peak_rows(const tria_policy* p, int64_t n_prompt) {
    if (!policy_ok(p) || n_prompt < 0) return TRIA_E_INVAL;
    const int64_t fixed = p->protect_prefill ? n_prompt : 0;
    if (p->trigger == TRIA_TRIGGER_THRESHOLD) {
        // counted rows never exceed budget + divide_length; an unprotected
        // prompt above that runs a pass at the first decode step
        const int64_t steady = fixed + p->budget + p->divide_length;
        const int64_t first = n_prompt + 1;
        return steady > first ? steady : first;
    }
    // a pass every `interval` steps leaves at most budget (+ the protected prompt)
    const int64_t base = n_prompt > fixed + p->budget ? n_prompt : fixed + p->budget;
    return base + p->interval;
}

int64_t tria_decode_step(tria_ctx* ctx, const tria_cache* cache, const tria_policy* p,
                         tria_decode_state* st, hipStream_t stream) {
    if (!ctx || !cache || !st) return TRIA_E_INVAL;
    if (st->n_rows > cache->cap) return TRIA_E_INVAL;  // the physical capacity was too small
    st->steps += 1;
    int64_t b = 0, s = 0, w = 0;
    const int due = tria_policy_due(p, st, &b, &s, &w);
    if (due < 0) return due;
    if (!due) return st->n_rows;
    const int64_t kept = tria_evict(ctx, cache, st->n_rows, b, s, w, stream);
    if (kept < 0) return kept;
    st->n_rows = kept;
    st->steps = 0;
    st->passes += 1;
    return kept;
}

}  // extern "C"
