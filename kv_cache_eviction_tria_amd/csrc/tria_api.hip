// Host side of the C ABI declared in include/tria.h: argument checks, the
// context (device statistics and scratch), and the launch sequence of one
// pass: prep -> score -> select -> compact, all stream-ordered.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "tria_group.h"

namespace tria {
int64_t select_key_scratch_rows(const Batch& b, int units_per_seq, int G);
hipError_t launch_moments(const Batch& b, int units_per_seq, int G, const float* raw,
                          PartRec* part, hipStream_t s);
hipError_t launch_holefill(const CacheView& cv, const Batch& b, int n_units, const int32_t* keep,
                           hipStream_t s);
void attention_splits(const Batch& b, int n_units, int* n_split, int* rows_per_split);
hipError_t launch_attention(const CacheView& cv, const Batch& b, int n_units, int G, int hd,
                            int k_type, int v_type, const float* q, float scale, int n_split,
                            int rows_per_split, void* parts, float* pacc, float* out,
                            hipStream_t s);
size_t attention_part_bytes();
hipError_t launch_select_impl(const Batch& b, int units_per_seq, int G, const float* raw,
                              const PartRec* part, int32_t* keep, float* agg,
                              uint32_t* key_scratch, int32_t* chunk_pb, uint32_t* ticket,
                              hipStream_t s);
}  // namespace tria

using namespace tria;

struct tria_ctx {
    int L, Hkv, Hq, G, hd, F, k_type, v_type;
    int kb, vb;
    double theta;
    // device
    float* q_re = nullptr;
    float* q_im = nullptr;
    float* w = nullptr;
    double* omega = nullptr;
    double* m_re = nullptr;
    double* m_im = nullptr;
    // scratch, grown on demand
    int32_t* coef = nullptr;
    size_t coef_bytes = 0;
    float* raw = nullptr;
    size_t raw_bytes = 0;
    int32_t* keep = nullptr;
    size_t keep_bytes = 0;
    uint32_t* keys = nullptr;
    size_t keys_bytes = 0;
    PartRec* part = nullptr;
    size_t part_bytes = 0;
    int32_t* pb = nullptr;  // chunk prefix counts (selector -> compaction)
    size_t pb_bytes = 0;
    CompactState cst = {nullptr, 0, nullptr, nullptr, 0};
    size_t flag_bytes = 0;
    // shared keep sets (tria_set_keep_mode): norms, group scores, kept rows
    int keep_mode = TRIA_KEEP_PER_UNIT;
    int compact_mode = TRIA_COMPACT_ORDERED;  // tria_set_compaction
    // decode attention (tria_decode_attention*): per-split partial results
    void* att_parts = nullptr;
    size_t att_parts_bytes = 0;
    float* att_acc = nullptr;
    size_t att_acc_bytes = 0;
    HeadNorm* norms = nullptr;
    size_t norms_bytes = 0;
    float* gagg = nullptr;
    size_t gagg_bytes = 0;
    int32_t* gkeep = nullptr;
    size_t gkeep_bytes = 0;
    int32_t* gpb = nullptr;
    size_t gpb_bytes = 0;
    // per-kernel timing (tria_timing_*)
    bool timing = false;
    hipEvent_t tev[TRIA_TIMED_MAX][2] = {};
    int tstage[TRIA_TIMED_MAX] = {};
    int ntimed = 0;
    int64_t untimed = 0;
    int last_hip = 0;
};

namespace {

constexpr int64_t kMaxRows = TRIA_MAX_ROWS;  // rows per unit the selector handles

int hip_fail(tria_ctx* ctx, hipError_t e) {
    if (ctx) ctx->last_hip = (int)e;
    return e == hipErrorOutOfMemory ? TRIA_E_NOMEM : TRIA_E_HIP;
}

// Grow a scratch buffer.  Work already enqueued on `s` may still use the old
// buffer, so the stream is drained before it is released.
int grow(tria_ctx* ctx, void** buf, size_t* have, size_t need, hipStream_t s) {
    if (need <= *have) return TRIA_OK;
    if (*buf) {
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(ctx, e);
        e = hipFree(*buf);
        *buf = nullptr;
        *have = 0;
        if (e != hipSuccess) return hip_fail(ctx, e);
    }
    const size_t bytes = (need + 4095) & ~(size_t)4095;
    hipError_t e = hipMalloc(buf, bytes);
    if (e != hipSuccess) {
        *buf = nullptr;
        return hip_fail(ctx, e);
    }
    *have = bytes;
    return TRIA_OK;
}

// Timing brackets: begin returns a record slot (or -1 when timing is off or
// the record is full), end closes it on the same stream.
hipError_t timed_begin(tria_ctx* ctx, int stage, hipStream_t s, int* slot) {
    *slot = -1;
    if (!ctx->timing) return hipSuccess;
    if (ctx->ntimed >= TRIA_TIMED_MAX) {
        ++ctx->untimed;
        return hipSuccess;
    }
    const int i = ctx->ntimed++;
    ctx->tstage[i] = stage;
    *slot = i;
    return hipEventRecord(ctx->tev[i][0], s);
}

hipError_t timed_end(tria_ctx* ctx, int slot, hipStream_t s) {
    return slot < 0 ? hipSuccess : hipEventRecord(ctx->tev[slot][1], s);
}

// Compaction flags for a launch over these units (zeroed when allocated).
int reserve_flags(tria_ctx* ctx, const Batch& b, int units, hipStream_t s) {
    const int64_t words = compact_flag_words(b, units);
    void* f = ctx->cst.flags;
    const size_t had = ctx->flag_bytes;
    int rc = grow(ctx, &f, &ctx->flag_bytes, (size_t)words * 4, s);
    ctx->cst.flags = static_cast<uint32_t*>(f);
    if (rc) return rc;
    if (ctx->flag_bytes != had) {
        hipError_t e = hipMemsetAsync(ctx->cst.flags, 0, ctx->flag_bytes, s);
        if (e != hipSuccess) return hip_fail(ctx, e);
    }
    ctx->cst.flag_words = (int64_t)(ctx->flag_bytes / 4);
    return TRIA_OK;
}

// A compaction launch, timed when timing is on.  pb: the selector's chunk
// prefix counts, or nullptr to derive them from keep into ctx->pb.
int compact_timed(tria_ctx* ctx, const CacheView& cv, const Batch& b, int units,
                  const int32_t* keep, const int32_t* pb, hipStream_t s) {
    int slot;
    hipError_t e = timed_begin(ctx, TRIA_STAGE_COMPACT, s, &slot);
    if (e == hipSuccess && ctx->compact_mode == TRIA_COMPACT_HOLE_FILL)
        e = launch_holefill(cv, b, units, keep, s);
    else if (e == hipSuccess)
        e = launch_compact(cv, b, units, keep, pb, ctx->pb, ctx->cst, ctx->cst.ticket, s);
    if (e == hipSuccess) e = timed_end(ctx, slot, s);
    return e == hipSuccess ? TRIA_OK : hip_fail(ctx, e);
}

struct Protect {
    int64_t kept, s_end, w_start;
};

Protect protect(int64_t n, int64_t budget, int64_t sink, int64_t window) {
    Protect p;
    if (budget >= n) {
        p.kept = n;
        p.s_end = p.w_start = n;  // everything kept
        return p;
    }
    p.s_end = sink < n ? sink : n;
    p.w_start = window >= n ? 0 : n - window;
    if (p.w_start < p.s_end) p.w_start = p.s_end;
    const int64_t np = p.s_end + (n - p.w_start);
    p.kept = budget > np ? budget : np;
    return p;
}

CacheView view_of(const tria_ctx* ctx, const tria_cache* c) {
    CacheView cv;
    cv.k = static_cast<uint8_t*>(c->k);
    cv.v = static_cast<uint8_t*>(c->v);
    cv.pos = c->pos;
    cv.cap = c->cap;
    cv.n_blocks = 0;
    cv.bt = nullptr;
    cv.max_blocks = 0;
    cv.L = ctx->L;
    cv.Hkv = ctx->Hkv;
    cv.kb = ctx->kb;
    cv.vb = ctx->vb;
    return cv;
}

Batch one_seq(int64_t n, const Protect& p) {
    Batch b;
    memset(&b, 0, sizeof(b));
    b.n_seq = 1;
    b.seq[0].n = n;
    b.seq[0].kept = p.kept;
    b.seq[0].s_end = p.s_end;
    b.seq[0].w_start = p.w_start;
    b.seq[0].raw_off = 0;
    b.seq[0].keep_off = 0;
    b.seq[0].part_off = 0;
    b.seq[0].pb_off = 0;
    return b;
}

// The kernels move rows in pieces of up to 16 bytes and scores in vectors of up
// to 16 bytes: the arrays must start on those boundaries (rows then keep them).
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_cache(const tria_cache* c, int64_t n) {
    if (!c || !c->k || !c->v || !c->pos) return TRIA_E_INVAL;
    if (!aligned(c->k, 16) || !aligned(c->v, 16) || !aligned(c->pos, 4)) return TRIA_E_INVAL;
    if (n < 0 || c->cap < 0 || n > c->cap || n > kMaxRows) return n > kMaxRows ? TRIA_E_UNSUPPORTED : TRIA_E_INVAL;
    return TRIA_OK;
}

// Coefficient tables for up to n_units units must fit before any work is queued.
int reserve_coef(tria_ctx* ctx, int n_units, hipStream_t s) {
    const CoefGeom cg = coef_geom(ctx->k_type, ctx->hd, ctx->G);
    return grow(ctx, reinterpret_cast<void**>(&ctx->coef), &ctx->coef_bytes,
                (size_t)n_units * cg.words * 4, s);
}

// Coefficient tables of every unit of the batch (laid out per unit of the
// whole model, see Batch::coef_L).
int run_prep(tria_ctx* ctx, const CacheView& cv, const Batch& b, int n_units, hipStream_t s) {
    int rc = reserve_coef(ctx, b.n_seq * ctx->L * ctx->Hkv, s);
    if (rc) return rc;
    hipError_t e = launch_prep(cv, b, n_units, ctx->k_type, ctx->G, ctx->hd, ctx->q_re, ctx->q_im,
                               ctx->w, ctx->omega, ctx->m_re, ctx->m_im, ctx->coef, s);
    return e == hipSuccess ? TRIA_OK : hip_fail(ctx, e);
}

// The score kernels of the units of cv, tables already prepared.
int run_score_only(tria_ctx* ctx, const CacheView& cv, const Batch& b, int n_units, float* raw,
                   PartRec* part, hipStream_t s) {
    int slot;
    hipError_t e = timed_begin(ctx, TRIA_STAGE_SCORE, s, &slot);
    if (e == hipSuccess)
        e = launch_score(cv, b, n_units, ctx->k_type, ctx->G, ctx->hd, ctx->coef, raw, part, s);
    if (e == hipSuccess) e = timed_end(ctx, slot, s);
    return e == hipSuccess ? TRIA_OK : hip_fail(ctx, e);
}

// prep + score.
int run_score(tria_ctx* ctx, const CacheView& cv, const Batch& b, int n_units, float* raw,
              PartRec* part, hipStream_t s) {
    int rc = run_prep(ctx, cv, b, n_units, s);
    return rc ? rc : run_score_only(ctx, cv, b, n_units, raw, part, s);
}

// Chunk prefix counts of a batch whose units are units_per_seq per sequence.
int reserve_pb(tria_ctx* ctx, const Batch& b, int units_per_seq, hipStream_t s) {
    int64_t words = 0;
    for (int i = 0; i < b.n_seq; ++i) {
        const SeqDesc& sd = b.seq[i];
        const int64_t e = sd.pb_off + (int64_t)units_per_seq * chunk_bounds(sd.kept);
        words = e > words ? e : words;
    }
    return grow(ctx, reinterpret_cast<void**>(&ctx->pb), &ctx->pb_bytes, (size_t)words * 4, s);
}

// Scratch for the moment partials and the key array of a batch whose units
// are units_per_seq per sequence (the largest end offset over the sequences).
int reserve_select(tria_ctx* ctx, const Batch& b, int units_per_seq, hipStream_t s) {
    int64_t recs = 0;
    for (int i = 0; i < b.n_seq; ++i) {
        const SeqDesc& sd = b.seq[i];
        const int64_t e = (sd.part_off + (int64_t)units_per_seq * part_tiles(sd.n)) * ctx->G;
        recs = e > recs ? e : recs;
    }
    int rc = grow(ctx, reinterpret_cast<void**>(&ctx->part), &ctx->part_bytes,
                  (size_t)recs * sizeof(PartRec), s);
    if (rc) return rc;
    rc = reserve_pb(ctx, b, units_per_seq, s);
    if (rc) return rc;
    const int64_t krows = select_key_scratch_rows(b, units_per_seq, ctx->G);
    if (krows > 0)
        rc = grow(ctx, reinterpret_cast<void**>(&ctx->keys), &ctx->keys_bytes, (size_t)krows * 4, s);
    return rc;
}

// Scratch of a shared-keep-set selection over a whole batch (all layers).
int reserve_shared(tria_ctx* ctx, const Batch& b, hipStream_t s) {
    const int ng = keep_groups(ctx->keep_mode, ctx->L, ctx->Hkv);
    const GroupOff tot = group_offsets(b, b.n_seq, ng);
    const size_t units = (size_t)b.n_seq * ctx->L * ctx->Hkv;
    int rc = grow(ctx, reinterpret_cast<void**>(&ctx->norms), &ctx->norms_bytes,
                  units * ctx->G * sizeof(HeadNorm), s);
    if (!rc)
        rc = grow(ctx, reinterpret_cast<void**>(&ctx->gagg), &ctx->gagg_bytes,
                  (size_t)tot.agg * sizeof(float), s);
    if (!rc)
        rc = grow(ctx, reinterpret_cast<void**>(&ctx->gkeep), &ctx->gkeep_bytes,
                  (size_t)tot.keep * sizeof(int32_t), s);
    if (!rc)
        rc = grow(ctx, reinterpret_cast<void**>(&ctx->gpb), &ctx->gpb_bytes,
                  (size_t)tot.pb * sizeof(int32_t), s);
    const int64_t krows = select_key_scratch_rows(group_batch(b, ng), ng, 1);
    if (!rc && krows > 0)
        rc = grow(ctx, reinterpret_cast<void**>(&ctx->keys), &ctx->keys_bytes, (size_t)krows * 4, s);
    return rc;
}

// Select over `layers` layers per sequence (all by default).  have_part: the
// scorer already wrote the moment partials of these scores into ctx->part.
// A shared keep mode needs all layers (layers < 0).
int run_select(tria_ctx* ctx, const Batch& b, const float* raw, int32_t* keep, float* agg,
               bool have_part, hipStream_t s) {
    const int ups = ctx->L * ctx->Hkv;
    const bool shared = ctx->keep_mode != TRIA_KEEP_PER_UNIT;
    int rc = reserve_select(ctx, b, ups, s);
    if (!rc && shared) rc = reserve_shared(ctx, b, s);
    if (rc) return rc;
    int slot;
    hipError_t e = timed_begin(ctx, TRIA_STAGE_SELECT, s, &slot);
    if (e == hipSuccess && !have_part) e = launch_moments(b, ups, ctx->G, raw, ctx->part, s);
    if (e == hipSuccess) {
        if (shared)
            e = launch_shared_select(b, ctx->L, ctx->Hkv, ctx->G, ctx->keep_mode, raw, ctx->part,
                                     ctx->norms, ctx->gagg, ctx->gkeep, ctx->gpb, ctx->keys, keep,
                                     ctx->pb, agg, ctx->cst.ticket, s);
        else
            e = launch_select_impl(b, ups, ctx->G, raw, ctx->part, keep, agg, ctx->keys, ctx->pb,
                                   ctx->cst.ticket, s);
    }
    if (e == hipSuccess) e = timed_end(ctx, slot, s);
    if (e != hipSuccess) return hip_fail(ctx, e);
    return TRIA_OK;
}

// The layers [l0, l0 + lg) of a cache as a cache of lg layers.
CacheView sub_view(const CacheView& cv, int l0, int lg) {
    CacheView s = cv;
    s.L = lg;
    const int64_t rows = cv.bt ? (int64_t)l0 * cv.n_blocks * cv.Hkv * kBlockRows
                               : (int64_t)l0 * cv.Hkv * cv.cap;
    s.k += rows * cv.kb;
    s.v += rows * cv.vb;
    s.pos += rows;
    return s;
}

// One whole pass (score -> select -> compact) over every unit of the batch, on `s`.
int run_pass(tria_ctx* ctx, const CacheView& cv, const Batch& b, hipStream_t s) {
    const int all_units = b.n_seq * ctx->L * ctx->Hkv;
    // all scratch is sized for the whole pass before any work is queued
    int rc = reserve_select(ctx, b, ctx->L * ctx->Hkv, s);
    if (rc) return rc;
    rc = reserve_flags(ctx, b, all_units, s);
    if (rc) return rc;
    rc = run_prep(ctx, cv, b, all_units, s);
    if (rc) return rc;
    rc = run_score_only(ctx, cv, b, all_units, ctx->raw, ctx->part, s);
    if (rc) return rc;
    rc = run_select(ctx, b, ctx->raw, ctx->keep, nullptr, true, s);
    if (rc) return rc;
    return compact_timed(ctx, cv, b, all_units, ctx->keep, ctx->pb, s);
}

// One decode step's attention over every unit of the batch (q, out: [seq][L]
// [Hq][hd] fp32).
int run_attention(tria_ctx* ctx, const CacheView& cv, const Batch& b, const float* q, float scale,
                  float* out, hipStream_t s) {
    const int units = b.n_seq * ctx->L * ctx->Hkv;
    int n_split = 1, rps = 64;
    attention_splits(b, units, &n_split, &rps);
    const size_t recs = (size_t)units * n_split * ctx->G;
    int rc = grow(ctx, &ctx->att_parts, &ctx->att_parts_bytes, recs * attention_part_bytes(), s);
    if (!rc)
        rc = grow(ctx, reinterpret_cast<void**>(&ctx->att_acc), &ctx->att_acc_bytes,
                  recs * ctx->hd * sizeof(float), s);
    if (rc) return rc;
    const hipError_t e = launch_attention(cv, b, units, ctx->G, ctx->hd, ctx->k_type, ctx->v_type,
                                          q, scale, n_split, rps, ctx->att_parts, ctx->att_acc,
                                          out, s);
    return e == hipSuccess ? TRIA_OK : hip_fail(ctx, e);
}

// Why a model is outside the kernels' eligibility gate, or nullptr (llama.cpp
// page, section 4 "GPU scoring requirements": integer GQA ratio, head_dim <=
// 256 and a multiple of 32; every dimension rotary, which tria_model_desc
// cannot express otherwise).
const char* gate_reason(const tria_model_desc* d) {
    if (d->n_q_heads % d->n_kv_heads != 0) return "query heads not a multiple of KV heads";
    if (d->n_q_heads / d->n_kv_heads > 64) return "more than 64 query heads per KV head";
    if (d->head_dim < 32 || d->head_dim > 256 || d->head_dim % 32 != 0)
        return "head_dim not a multiple of 32 in [32, 256]";
    if (d->k_type != TRIA_KV_F16 && d->k_type != TRIA_KV_Q8_0) return "unknown K type";
    if (d->v_type != TRIA_KV_F16 && d->v_type != TRIA_KV_Q8_0) return "unknown V type";
    return nullptr;
}

// With TRIA_DEBUG set (and not "0") in the environment, the first model
// description a process passes to tria_load_stats is reported on stderr, once:
// its shape and whether the kernels take it (the llama.cpp page prints the same
// decision once at startup).
void log_gate_once(const tria_model_desc* d, const char* why) {
    static std::atomic<int> done{0};
    const char* env = getenv("TRIA_DEBUG");
    if (!env || !env[0] || (env[0] == '0' && !env[1])) return;
    if (done.exchange(1)) return;
    auto kt = [](int t) { return t == TRIA_KV_F16 ? "f16" : (t == TRIA_KV_Q8_0 ? "q8_0" : "?"); };
    fprintf(stderr, "tria: gpu gate - k=%s v=%s nq=%d nkv=%d hd=%d nonrot=0 -> %s%s\n",
            kt(d->k_type), kt(d->v_type), d->n_q_heads, d->n_kv_heads, d->head_dim,
            why ? "not eligible: " : "eligible", why ? why : "");
}

// ---------------------------------------------------------------------------
// Scratch of tria_evict_noalloc: one fixed array per GPU, in the library's code
// object, so that the call itself allocates nothing.  Layout:
//   [0, kNaFlagBytes)                compaction flags (only ever written with
//                                    compaction epochs, so a stale word never
//                                    equals a later epoch)
//   [kNaFlagBytes, + 256)            the compaction's task counter and flag epoch
//   [kNaDataOff, kNoAllocScratchBytes) coefficient tables of every unit, then
//                                    one group of layers' raw scores, moment
//                                    partials, kept indices, chunk prefix
//                                    counts and (above 128K rows) selector keys
constexpr size_t kNaFlagBytes = (size_t)1 << 20;
constexpr size_t kNaDataOff = kNaFlagBytes + 256;
constexpr int kNaMaxDevices = 64;

struct NoAllocDevice {
    uint8_t* ptr = nullptr;  // device address of `scratch` on this GPU
};
std::mutex g_na_mu;
NoAllocDevice g_na[kNaMaxDevices];

}  // namespace

// In host code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device is ever used.
static __device__ __align__(256) uint8_t scratch[TRIA_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's scratch address, looked up once per device (with that
// device current).  TRIA_E_HIP if the lookup fails.
int noalloc_device(tria_ctx* ctx, int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(ctx, e);
    if (dev < 0 || dev >= kNaMaxDevices) return TRIA_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_na_mu);
    if (!g_na[dev].ptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(ctx, e != hipSuccess ? e : hipErrorUnknown);
        g_na[dev].ptr = static_cast<uint8_t*>(p);
    }
    *dev_out = dev;
    return TRIA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bytes one layer of a pass needs in the data region (per-layer buffers).
struct NaLayer {
    size_t raw, part, keep, pb, keys;
    int64_t flag_words;
    size_t total() const { return raw + part + keep + pb + keys; }
};

NaLayer noalloc_layer(const tria_ctx* ctx, int64_t n, int64_t kept) {
    NaLayer x;
    const int64_t H = ctx->Hkv, G = ctx->G;
    x.raw = align256((size_t)(H * n * G) * sizeof(float));
    x.part = align256((size_t)(H * part_tiles(n) * G) * sizeof(PartRec));
    x.keep = align256((size_t)(H * kept) * sizeof(int32_t));
    x.pb = align256((size_t)(H * chunk_bounds(kept)) * sizeof(int32_t));
    x.keys = n > (int64_t)128 * 1024 ? align256((size_t)(H * n) * sizeof(uint32_t)) : 0;
    x.flag_words = H * chunk_count(kept);
    return x;
}

}  // namespace

extern "C" {

int64_t tria_evict_noalloc(tria_ctx* ctx, const tria_cache* cache, int64_t n_tokens,
                           int64_t budget, int64_t sink, int64_t window, hipStream_t stream) {
    if (!ctx) return TRIA_E_INVAL;
    int rc = check_cache(cache, n_tokens);
    if (rc) return rc;
    if (budget < 0 || sink < 0 || window < 0) return TRIA_E_INVAL;
    const Protect p = protect(n_tokens, budget, sink, window);
    if (p.kept == n_tokens) return n_tokens;  // nothing to evict: no work, no writes
    if (ctx->keep_mode != TRIA_KEEP_PER_UNIT) return TRIA_E_UNSUPPORTED;
    // layers per group: as many as the data region holds (at least one)
    const CoefGeom cg = coef_geom(ctx->k_type, ctx->hd, ctx->G);
    const size_t coef_bytes = align256((size_t)ctx->L * ctx->Hkv * cg.words * 4);
    const NaLayer per = noalloc_layer(ctx, n_tokens, p.kept);
    const size_t room = TRIA_NOALLOC_SCRATCH_BYTES - kNaDataOff;
    if (coef_bytes + per.total() > room || per.flag_words > (int64_t)(kNaFlagBytes / 4))
        return TRIA_E_UNSUPPORTED;
    int lg = (int)((room - coef_bytes) / per.total());
    const int lf = (int)((int64_t)(kNaFlagBytes / 4) / (per.flag_words > 0 ? per.flag_words : 1));
    lg = lg < lf ? lg : lf;
    lg = lg < ctx->L ? lg : ctx->L;
    int dev = 0;
    rc = noalloc_device(ctx, &dev);
    if (rc) return rc;

    uint8_t* base = g_na[dev].ptr;
    uint32_t* flags = reinterpret_cast<uint32_t*>(base);
    uint32_t* ticket = reinterpret_cast<uint32_t*>(base + kNaFlagBytes);
    int32_t* coef = reinterpret_cast<int32_t*>(base + kNaDataOff);
    uint8_t* grp = base + kNaDataOff + coef_bytes;
    float* raw = reinterpret_cast<float*>(grp);
    PartRec* part = reinterpret_cast<PartRec*>(grp + (size_t)lg * per.raw);
    int32_t* keep = reinterpret_cast<int32_t*>(grp + (size_t)lg * (per.raw + per.part));
    int32_t* pb = reinterpret_cast<int32_t*>(grp + (size_t)lg * (per.raw + per.part + per.keep));
    uint32_t* keys = per.keys ? reinterpret_cast<uint32_t*>(
                                    grp + (size_t)lg * (per.raw + per.part + per.keep + per.pb))
                              : nullptr;

    const CacheView cv = view_of(ctx, cache);
    Batch b = one_seq(n_tokens, p);
    const int units = ctx->L * ctx->Hkv;
    hipError_t e = launch_prep(cv, b, units, ctx->k_type, ctx->G, ctx->hd, ctx->q_re, ctx->q_im,
                               ctx->w, ctx->omega, ctx->m_re, ctx->m_im, coef, stream);
    CompactState cs = {flags, (int64_t)(kNaFlagBytes / 4), ticket, ctx->cst.err,
                       ctx->cst.max_groups};
    for (int l0 = 0; l0 < ctx->L && e == hipSuccess; l0 += lg) {
        const int lc = ctx->L - l0 < lg ? ctx->L - l0 : lg;
        const CacheView sv = sub_view(cv, l0, lc);
        Batch gb = b;  // this group's buffers start at offset 0
        gb.coef_L = ctx->L;
        gb.coef_l0 = l0;
        const int gu = lc * ctx->Hkv;
        e = launch_score(sv, gb, gu, ctx->k_type, ctx->G, ctx->hd, coef, raw, part, stream);
        if (e == hipSuccess)
            e = launch_select_impl(gb, gu, ctx->G, raw, part, keep, nullptr, keys, pb, ticket,
                                   stream);
        if (e == hipSuccess && ctx->compact_mode == TRIA_COMPACT_HOLE_FILL)
            e = launch_holefill(sv, gb, gu, keep, stream);
        else if (e == hipSuccess)
            e = launch_compact(sv, gb, gu, keep, pb, nullptr, cs, ticket, stream);
    }
    if (e != hipSuccess) return hip_fail(ctx, e);
    return p.kept;
}

int tria_decode_attention(tria_ctx* ctx, const tria_cache* cache, int64_t n_tokens, const float* q,
                          float scale, float* out, hipStream_t stream) {
    if (!ctx || !q || !out) return TRIA_E_INVAL;
    if (!aligned(q, 4) || !aligned(out, 4)) return TRIA_E_INVAL;
    int rc = check_cache(cache, n_tokens);
    if (rc) return rc;
    Protect p;
    p.kept = n_tokens;
    p.s_end = p.w_start = n_tokens;
    const Batch b = one_seq(n_tokens, p);
    return run_attention(ctx, view_of(ctx, cache), b, q, scale, out, stream);
}

int tria_decode_attention_paged_batch(tria_ctx* ctx, const tria_paged_cache* cache, int32_t n_seq,
                                      const int64_t* n_tokens, const float* q, float scale,
                                      float* out, hipStream_t stream) {
    if (!ctx || !cache || !n_tokens || !q || !out) return TRIA_E_INVAL;
    if (!aligned(q, 4) || !aligned(out, 4)) return TRIA_E_INVAL;
    if (!cache->k_pool || !cache->v_pool || !cache->pos_pool || !cache->block_table)
        return TRIA_E_INVAL;
    if (!aligned(cache->k_pool, 16) || !aligned(cache->v_pool, 16) ||
        !aligned(cache->pos_pool, 4) || !aligned(cache->block_table, 4))
        return TRIA_E_INVAL;
    if (n_seq < 1 || n_seq > TRIA_MAX_SEQ || cache->n_blocks < 1 || cache->max_blocks < 1)
        return TRIA_E_INVAL;
    Batch b;
    memset(&b, 0, sizeof(b));
    b.n_seq = n_seq;
    for (int i = 0; i < n_seq; ++i) {
        if (n_tokens[i] < 0 || n_tokens[i] > (int64_t)cache->max_blocks * TRIA_BLOCK)
            return TRIA_E_INVAL;
        b.seq[i].n = n_tokens[i];
        b.seq[i].kept = n_tokens[i];
    }
    CacheView cv;
    cv.k = static_cast<uint8_t*>(cache->k_pool);
    cv.v = static_cast<uint8_t*>(cache->v_pool);
    cv.pos = cache->pos_pool;
    cv.cap = 0;
    cv.n_blocks = cache->n_blocks;
    cv.bt = cache->block_table;
    cv.max_blocks = cache->max_blocks;
    cv.L = ctx->L;
    cv.Hkv = ctx->Hkv;
    cv.kb = ctx->kb;
    cv.vb = ctx->vb;
    return run_attention(ctx, cv, b, q, scale, out, stream);
}

const char* tria_strerror(int code) {
    switch (code) {
        case TRIA_OK: return "ok";
        case TRIA_E_INVAL: return "invalid argument";
        case TRIA_E_UNSUPPORTED: return "shape not supported by the gfx950 kernels";
        case TRIA_E_HIP: return "HIP runtime error";
        case TRIA_E_NOMEM: return "out of memory";
        case TRIA_E_DEVICE: return "a compaction workgroup gave up a bounded wait";
        default: return "unknown error";
    }
}

int tria_last_hip_error(const tria_ctx* ctx) { return ctx ? ctx->last_hip : 0; }

int64_t tria_row_bytes(int32_t kv_type, int32_t head_dim) {
    if (head_dim <= 0 || head_dim % 32 != 0) return TRIA_E_UNSUPPORTED;
    if (kv_type == TRIA_KV_F16) return 2 * (int64_t)head_dim;
    if (kv_type == TRIA_KV_Q8_0) return 34 * (int64_t)(head_dim / 32);
    return TRIA_E_UNSUPPORTED;
}

int64_t tria_kept_count(int64_t n_tokens, int64_t budget, int64_t sink, int64_t window) {
    if (n_tokens < 0 || budget < 0 || sink < 0 || window < 0) return TRIA_E_INVAL;
    return protect(n_tokens, budget, sink, window).kept;
}

void tria_free(tria_ctx* ctx) {
    if (!ctx) return;
    void* bufs[] = {ctx->q_re, ctx->q_im, ctx->w,    ctx->omega, ctx->m_re,      ctx->m_im,
                    ctx->coef, ctx->raw,  ctx->keep, ctx->keys,  ctx->part,      ctx->pb,
                    ctx->cst.flags,       ctx->cst.err,          ctx->cst.ticket,
                    ctx->norms, ctx->gagg, ctx->gkeep, ctx->gpb, ctx->att_parts, ctx->att_acc};
    for (void* p : bufs)
        if (p) (void)hipFree(p);
    for (auto& pr : ctx->tev)
        for (hipEvent_t ev : pr)
            if (ev) (void)hipEventDestroy(ev);
    delete ctx;
}

int tria_load_stats(tria_ctx** out, const tria_model_desc* d, const float* q_re,
                    const float* q_im, const float* norm_w, hipStream_t stream) {
    (void)stream;
    if (!out) return TRIA_E_INVAL;
    *out = nullptr;
    if (!d || !q_re || !q_im || !norm_w || !d->offsets) return TRIA_E_INVAL;
    if (d->n_layers < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1 || d->n_offsets < 1)
        return TRIA_E_INVAL;
    if (!(d->rope_theta > 1.0) || !isfinite(d->rope_theta)) return TRIA_E_INVAL;
    for (int i = 0; i < d->n_offsets; ++i) {
        if (d->offsets[i] <= 0) return TRIA_E_INVAL;
        if (i > 0 && d->offsets[i] <= d->offsets[i - 1]) return TRIA_E_INVAL;
    }
    // eligibility gate (llama.cpp page, section 4 "GPU scoring requirements")
    const char* why = gate_reason(d);
    log_gate_once(d, why);
    if (why) return TRIA_E_UNSUPPORTED;

    tria_ctx* ctx = new (std::nothrow) tria_ctx();
    if (!ctx) return TRIA_E_NOMEM;
    ctx->L = d->n_layers;
    ctx->Hkv = d->n_kv_heads;
    ctx->Hq = d->n_q_heads;
    ctx->G = d->n_q_heads / d->n_kv_heads;
    ctx->hd = d->head_dim;
    ctx->F = d->head_dim / 2;
    ctx->k_type = d->k_type;
    ctx->v_type = d->v_type;
    ctx->kb = (int)tria_row_bytes(d->k_type, d->head_dim);
    ctx->vb = (int)tria_row_bytes(d->v_type, d->head_dim);
    ctx->theta = d->rope_theta;

    const size_t nstat = (size_t)ctx->L * ctx->Hq * ctx->F;
    const int F = ctx->F;
    double* host = (double*)malloc(sizeof(double) * 3 * F);
    if (!host) {
        delete ctx;
        return TRIA_E_NOMEM;
    }
    // omega_f = theta^(-2f/hd); M_f = mean over the offsets of exp(i omega_f delta)
    for (int f = 0; f < F; ++f) {
        const double om = pow(d->rope_theta, -2.0 * (double)f / (double)ctx->hd);
        double sr = 0.0, si = 0.0;
        for (int i = 0; i < d->n_offsets; ++i) {
            sr += cos(om * (double)d->offsets[i]);
            si += sin(om * (double)d->offsets[i]);
        }
        host[f] = om;
        host[F + f] = sr / d->n_offsets;
        host[2 * F + f] = si / d->n_offsets;
    }
    hipError_t e = hipSuccess;
    float** fdst[3] = {&ctx->q_re, &ctx->q_im, &ctx->w};
    const float* fsrc[3] = {q_re, q_im, norm_w};
    for (int i = 0; i < 3 && e == hipSuccess; ++i) {
        e = hipMalloc(reinterpret_cast<void**>(fdst[i]), nstat * sizeof(float));
        if (e == hipSuccess) e = hipMemcpy(*fdst[i], fsrc[i], nstat * sizeof(float), hipMemcpyHostToDevice);
    }
    double** ddst[3] = {&ctx->omega, &ctx->m_re, &ctx->m_im};
    for (int i = 0; i < 3 && e == hipSuccess; ++i) {
        e = hipMalloc(reinterpret_cast<void**>(ddst[i]), F * sizeof(double));
        if (e == hipSuccess) e = hipMemcpy(*ddst[i], host + i * F, F * sizeof(double), hipMemcpyHostToDevice);
    }
    free(host);
    // error word of the compaction's bounded waits, and its task ticket
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&ctx->cst.err), sizeof(int));
    if (e == hipSuccess) e = hipMemset(ctx->cst.err, 0, sizeof(int));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&ctx->cst.ticket), 2 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(ctx->cst.ticket, 0, 2 * sizeof(uint32_t));
    if (e != hipSuccess) {
        const int rc = e == hipErrorOutOfMemory ? TRIA_E_NOMEM : TRIA_E_HIP;
        tria_free(ctx);
        return rc;
    }
    // the current device's tria_evict_noalloc scratch address, looked up once
    int dev = 0;
    const int rc = noalloc_device(ctx, &dev);
    if (rc) {
        tria_free(ctx);
        return rc;
    }
    *out = ctx;
    return TRIA_OK;
}

int tria_score(tria_ctx* ctx, const tria_cache* cache, int64_t n_tokens, float* raw_scores,
               hipStream_t stream) {
    if (!ctx || !raw_scores) return TRIA_E_INVAL;
    if (!aligned(raw_scores, 16)) return TRIA_E_INVAL;
    int rc = check_cache(cache, n_tokens);
    if (rc) return rc;
    if (n_tokens == 0) return TRIA_OK;
    const CacheView cv = view_of(ctx, cache);
    const Batch b = one_seq(n_tokens, protect(n_tokens, n_tokens, 0, 0));
    return run_score(ctx, cv, b, ctx->L * ctx->Hkv, raw_scores, nullptr, stream);
}

int64_t tria_select(tria_ctx* ctx, const float* raw_scores, int64_t n_tokens, int64_t budget,
                    int64_t sink, int64_t window, int32_t* keep_idx, float* agg_out,
                    hipStream_t stream) {
    if (!ctx || !raw_scores || !keep_idx) return TRIA_E_INVAL;
    if (!aligned(raw_scores, 16) || !aligned(keep_idx, 4) || !aligned(agg_out, 4))
        return TRIA_E_INVAL;
    if (n_tokens < 0 || budget < 0 || sink < 0 || window < 0) return TRIA_E_INVAL;
    if (n_tokens > kMaxRows) return TRIA_E_UNSUPPORTED;
    if (n_tokens == 0) return 0;
    const Protect p = protect(n_tokens, budget, sink, window);
    const Batch b = one_seq(n_tokens, p);
    int rc = run_select(ctx, b, raw_scores, keep_idx, agg_out, false, stream);
    return rc ? rc : p.kept;
}

int tria_compact(tria_ctx* ctx, const tria_cache* cache, int64_t n_tokens,
                 const int32_t* keep_idx, int64_t kept, hipStream_t stream) {
    if (!ctx || !keep_idx) return TRIA_E_INVAL;
    if (!aligned(keep_idx, 4)) return TRIA_E_INVAL;
    int rc = check_cache(cache, n_tokens);
    if (rc) return rc;
    if (kept < 0 || kept > n_tokens) return TRIA_E_INVAL;
    if (kept == 0 || kept == n_tokens) return TRIA_OK;
    Protect p;
    p.kept = kept;
    p.s_end = p.w_start = 0;
    const Batch b = one_seq(n_tokens, p);
    const int units = ctx->L * ctx->Hkv;
    rc = reserve_pb(ctx, b, units, stream);
    if (rc) return rc;
    rc = reserve_flags(ctx, b, units, stream);
    if (rc) return rc;
    return compact_timed(ctx, view_of(ctx, cache), b, units, keep_idx, nullptr, stream);
}

int64_t tria_evict(tria_ctx* ctx, const tria_cache* cache, int64_t n_tokens, int64_t budget,
                   int64_t sink, int64_t window, hipStream_t stream) {
    if (!ctx) return TRIA_E_INVAL;
    int rc = check_cache(cache, n_tokens);
    if (rc) return rc;
    if (budget < 0 || sink < 0 || window < 0) return TRIA_E_INVAL;
    const Protect p = protect(n_tokens, budget, sink, window);
    if (p.kept == n_tokens) return n_tokens;  // nothing to evict: no work, no writes
    const int units = ctx->L * ctx->Hkv;
    rc = grow(ctx, reinterpret_cast<void**>(&ctx->raw), &ctx->raw_bytes,
              (size_t)units * n_tokens * ctx->G * sizeof(float), stream);
    if (rc) return rc;
    rc = grow(ctx, reinterpret_cast<void**>(&ctx->keep), &ctx->keep_bytes,
              (size_t)units * p.kept * sizeof(int32_t), stream);
    if (rc) return rc;
    const CacheView cv = view_of(ctx, cache);
    const Batch b = one_seq(n_tokens, p);
    rc = run_pass(ctx, cv, b, stream);
    return rc ? rc : p.kept;
}

int tria_evict_paged_batch(tria_ctx* ctx, const tria_paged_cache* cache, int32_t n_seq,
                           const int64_t* n_tokens, const int64_t* budget, int64_t sink,
                           int64_t window, int64_t* kept_out, hipStream_t stream) {
    if (!ctx || !cache || !n_tokens || !budget || !kept_out) return TRIA_E_INVAL;
    if (!cache->k_pool || !cache->v_pool || !cache->pos_pool || !cache->block_table)
        return TRIA_E_INVAL;
    if (!aligned(cache->k_pool, 16) || !aligned(cache->v_pool, 16) ||
        !aligned(cache->pos_pool, 4) || !aligned(cache->block_table, 4))
        return TRIA_E_INVAL;
    if (n_seq < 1 || n_seq > TRIA_MAX_SEQ || sink < 0 || window < 0) return TRIA_E_INVAL;
    if (cache->n_blocks < 1 || cache->max_blocks < 1) return TRIA_E_INVAL;
    const int units_per_seq = ctx->L * ctx->Hkv;
    Batch b;
    memset(&b, 0, sizeof(b));
    b.n_seq = n_seq;
    int64_t raw_off = 0, keep_off = 0, part_off = 0, pb_off = 0;
    bool any = false;
    for (int i = 0; i < n_seq; ++i) {
        const int64_t n = n_tokens[i];
        if (n < 0 || budget[i] < 0) return TRIA_E_INVAL;
        if (n > (int64_t)cache->max_blocks * TRIA_BLOCK) return TRIA_E_INVAL;
        if (n > kMaxRows) return TRIA_E_UNSUPPORTED;
        const Protect p = protect(n, budget[i], sink, window);
        SeqDesc& sd = b.seq[i];
        // a sequence with nothing to evict takes no part in the pass
        sd.n = p.kept == n ? 0 : n;
        sd.kept = p.kept == n ? 0 : p.kept;
        sd.s_end = p.s_end;
        sd.w_start = p.w_start;
        sd.raw_off = raw_off;
        sd.keep_off = keep_off;
        sd.part_off = part_off;
        sd.pb_off = pb_off;
        raw_off += (int64_t)units_per_seq * sd.n * ctx->G;
        part_off += (int64_t)units_per_seq * part_tiles(sd.n);
        pb_off += (int64_t)units_per_seq * chunk_bounds(sd.kept);
        keep_off += (int64_t)units_per_seq * sd.kept;
        kept_out[i] = p.kept;
        any |= sd.n > 0;
    }
    if (!any) return TRIA_OK;
    int rc = grow(ctx, reinterpret_cast<void**>(&ctx->raw), &ctx->raw_bytes,
                  (size_t)raw_off * sizeof(float), stream);
    if (rc) return rc;
    rc = grow(ctx, reinterpret_cast<void**>(&ctx->keep), &ctx->keep_bytes,
              (size_t)keep_off * sizeof(int32_t), stream);
    if (rc) return rc;
    CacheView cv;
    cv.k = static_cast<uint8_t*>(cache->k_pool);
    cv.v = static_cast<uint8_t*>(cache->v_pool);
    cv.pos = cache->pos_pool;
    cv.cap = 0;
    cv.n_blocks = cache->n_blocks;
    cv.bt = cache->block_table;
    cv.max_blocks = cache->max_blocks;
    cv.L = ctx->L;
    cv.Hkv = ctx->Hkv;
    cv.kb = ctx->kb;
    cv.vb = ctx->vb;
    return run_pass(ctx, cv, b, stream);
}

int tria_set_compaction(tria_ctx* ctx, int32_t mode) {
    if (!ctx) return TRIA_E_INVAL;
    if (mode != TRIA_COMPACT_ORDERED && mode != TRIA_COMPACT_HOLE_FILL) return TRIA_E_INVAL;
    ctx->compact_mode = mode;
    return TRIA_OK;
}

int tria_set_compaction_workgroups(tria_ctx* ctx, int32_t max_workgroups) {
    if (!ctx || max_workgroups < 0) return TRIA_E_INVAL;
    ctx->cst.max_groups = max_workgroups;
    return TRIA_OK;
}

int tria_set_keep_mode(tria_ctx* ctx, int32_t mode) {
    if (!ctx) return TRIA_E_INVAL;
    if (mode != TRIA_KEEP_PER_UNIT && mode != TRIA_KEEP_PER_KV_HEAD && mode != TRIA_KEEP_GLOBAL)
        return TRIA_E_INVAL;
    ctx->keep_mode = mode;
    return TRIA_OK;
}

int tria_device_status(tria_ctx* ctx) {
    if (!ctx) return TRIA_E_INVAL;
    hipError_t e = hipDeviceSynchronize();
    int flag = 0;
    if (e == hipSuccess) e = hipMemcpy(&flag, ctx->cst.err, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess && flag) e = hipMemset(ctx->cst.err, 0, sizeof(int));
    if (e != hipSuccess) return hip_fail(ctx, e);
    return flag ? TRIA_E_DEVICE : TRIA_OK;
}

int tria_timing_enable(tria_ctx* ctx, int32_t enable) {
    if (!ctx) return TRIA_E_INVAL;
    if (enable && !ctx->tev[0][0]) {
        for (auto& pr : ctx->tev)
            for (hipEvent_t& ev : pr) {
                hipError_t e = hipEventCreate(&ev);
                if (e != hipSuccess) return hip_fail(ctx, e);
            }
    }
    ctx->timing = enable != 0;
    ctx->ntimed = 0;
    ctx->untimed = 0;
    return TRIA_OK;
}

int tria_timing_read(tria_ctx* ctx, double* ms, int64_t* launches) {
    if (!ctx || !ms || !launches) return TRIA_E_INVAL;
    for (int i = 0; i < ctx->ntimed; ++i) {
        hipError_t e = hipEventSynchronize(ctx->tev[i][1]);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, ctx->tev[i][0], ctx->tev[i][1]);
        if (e != hipSuccess) return hip_fail(ctx, e);
        ms[ctx->tstage[i]] += (double)t;
        launches[ctx->tstage[i]] += 1;
    }
    const int64_t untimed = ctx->untimed;
    ctx->ntimed = 0;
    ctx->untimed = 0;
    return (int)(untimed > 0x7fffffff ? 0x7fffffff : untimed);
}

}  // extern "C"
