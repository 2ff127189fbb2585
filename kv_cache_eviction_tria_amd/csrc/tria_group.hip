// Shared keep sets: one keep set per KV head across all layers, or one for
// the whole cache ("TriAttention Native C++ Worklog", section "Later
// correction: selector and compaction are now cleared on the aggressive
// sample7 path": one keep-index list per KV head, gathered in every layer;
// llama.cpp page "TriAttention KV-Cache Eviction (--triattention)", section 5,
// "Phase C": a global z-normalisation shader).  The group score of a row is
// the max of the z-scores of every member query head, each z-normalised over
// its own unit, -inf if any member score is not finite; the group then keeps
// its protected rows and highest-scoring candidates like a single unit.
//
// Kernels (all HBM-light next to the score and the compaction):
//   norm_kernel       per-head mean / 1/sigma of every unit from the scorer's
//                     tile partials (one wavefront per head);
//   group_agg_kernel  64 rows of one group per block, the members split over
//                     its four wavefronts (lane = row, so every member's G
//                     scores come in coalesced 16-byte loads), maxima combined
//                     in LDS; writes the group score;
//   the selector      over the group scores with identity norms;
//   broadcast_kernel  copies each group's kept rows and chunk prefix counts to
//                     its member units, whose compaction then runs unchanged.
#include "tria_group.h"

namespace tria {

hipError_t launch_select_impl(const Batch& b, int units_per_seq, int G, const float* raw,
                              const PartRec* part, int32_t* keep, float* agg,
                              uint32_t* key_scratch, int32_t* chunk_pb, uint32_t* ticket,
                              hipStream_t s);

namespace {

constexpr int kGroupThreads = 256;

// Block u: unit u of the batch (sequence u / ups); wavefront w merges heads
// w, w + 4, ...  norms[u*G + h] = (hi, lo, 1/sigma) of query head h.
__global__ __launch_bounds__(kGroupThreads) void norm_kernel(Batch b, int ups, int G,
                                                             const PartRec* __restrict__ part,
                                                             HeadNorm* __restrict__ norms) {
    const int u = blockIdx.x;
    const int seq = u / ups, uu = u - seq * ups;
    const SeqDesc sd = b.seq[seq];
    if (sd.n <= 0) return;
    const int64_t tiles = part_tiles(sd.n);
    const PartRec* P = part + (sd.part_off + (int64_t)uu * tiles) * G;
    for (int h = threadIdx.x >> 6; h < G; h += kGroupThreads / 64) {
        const HeadNorm hn = merge_head_norm(P, tiles, G, h);
        if ((threadIdx.x & 63) == 0) norms[(int64_t)u * G + h] = hn;
    }
}

// Member m of group grp: the unit index within its sequence.
__device__ __forceinline__ int member_unit(int mode, int Hkv, int grp, int m) {
    return mode == TRIA_KEEP_PER_KV_HEAD ? m * Hkv + grp : m;
}

// grid (row blocks of kAggRows, groups, sequences).  Wavefront w of a block
// takes members w, w + kAggSlices, ... of the group for the block's 64 rows
// (lane = row, so each member's scores come in one coalesced sweep); the
// slices' maxima are combined through LDS.  GV: scores per row read as
// float4 (G when G % 4 == 0), 0 for scalar loads.
constexpr int kAggRows = 64;
constexpr int kAggSlices = kGroupThreads / kAggRows;

template <int GV>
__global__ __launch_bounds__(kGroupThreads) void group_agg_kernel(
    Batch b, int L, int Hkv, int G, int mode, const float* __restrict__ raw,
    const HeadNorm* __restrict__ norms, float* __restrict__ gagg) {
    __shared__ float best_sh[kAggSlices][kAggRows];
    __shared__ int bad_sh[kAggSlices][kAggRows];
    const int seq = blockIdx.z, grp = blockIdx.y;
    const SeqDesc sd = b.seq[seq];
    const int64_t n = sd.n;
    const int lane = threadIdx.x & 63, slice = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * kAggRows + lane;
    if ((int64_t)blockIdx.x * kAggRows >= n) return;  // whole block past the end
    const bool in = r < n;
    const int ups = L * Hkv;
    const int ng = keep_groups(mode, L, Hkv);
    const int members = mode == TRIA_KEEP_PER_KV_HEAD ? L : ups;
    // z-scores are finite or +-inf, so -inf is the identity of the max
    float best = -INFINITY;
    bool bad = false;
    for (int m = slice; in && m < members; m += kAggSlices) {
        const int uu = member_unit(mode, Hkv, grp, m);
        const float* R = raw + sd.raw_off + ((int64_t)uu * n + r) * G;
        const HeadNorm* NU = norms + ((int64_t)seq * ups + uu) * G;
        if constexpr (GV > 0) {
#pragma unroll
            for (int q = 0; q < GV / 4; ++q) {
                // raw scores are read once here: streaming (non-temporal) loads
                typedef float f4e __attribute__((ext_vector_type(4)));
                const f4e v = __builtin_nontemporal_load(reinterpret_cast<const f4e*>(R) + q);
                const float sv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!isfinite(sv[i])) bad = true;
                    const float z = znorm(sv[i], NU[4 * q + i]);
                    best = z > best ? z : best;
                }
            }
        } else {
            for (int h = 0; h < G; ++h) {
                const float s = R[h];
                if (!isfinite(s)) bad = true;
                const float z = znorm(s, NU[h]);
                best = z > best ? z : best;
            }
        }
    }
    best_sh[slice][lane] = best;
    bad_sh[slice][lane] = bad ? 1 : 0;
    __syncthreads();
    if (slice == 0 && in) {
#pragma unroll
        for (int q = 1; q < kAggSlices; ++q) {
            const float o = best_sh[q][lane];
            best = o > best ? o : best;
            bad = bad || bad_sh[q][lane];
        }
        const GroupOff go = group_offsets(b, seq, ng);
        gagg[go.agg + (int64_t)grp * n + r] = bad ? -INFINITY : best + 0.0f;
    }
}

// Block u: unit u of the batch; copies its group's kept rows, chunk prefix
// counts and (optionally) group scores into the unit's slots.
__global__ __launch_bounds__(kGroupThreads) void broadcast_kernel(
    Batch b, int L, int Hkv, int G, int mode, const int32_t* __restrict__ gkeep,
    const int32_t* __restrict__ gpb, const float* __restrict__ gagg, int32_t* __restrict__ keep,
    int32_t* __restrict__ pb, float* __restrict__ agg_out) {
    const int ups = L * Hkv;
    const int u = blockIdx.x;
    const int seq = u / ups, uu = u - seq * ups;
    const SeqDesc sd = b.seq[seq];
    if (sd.n <= 0) return;
    const int ng = keep_groups(mode, L, Hkv);
    const int grp = mode == TRIA_KEEP_PER_KV_HEAD ? uu % Hkv : 0;
    const GroupOff go = group_offsets(b, seq, ng);
    const int64_t K = sd.kept;
    const int32_t* src = gkeep + go.keep + (int64_t)grp * K;
    int32_t* dst = keep + sd.keep_off + (int64_t)uu * K;
    for (int64_t i = threadIdx.x; i < K; i += kGroupThreads) dst[i] = src[i];
    const int64_t nb = chunk_bounds(K);
    if (pb) {
        const int32_t* ps = gpb + go.pb + (int64_t)grp * nb;
        int32_t* pd = pb + sd.pb_off + (int64_t)uu * nb;
        for (int64_t i = threadIdx.x; i < nb; i += kGroupThreads) pd[i] = ps[i];
    }
    if (agg_out) {
        const float* as = gagg + go.agg + (int64_t)grp * sd.n;
        float* ad = agg_out + sd.raw_off / G + (int64_t)uu * sd.n;
        for (int64_t i = threadIdx.x; i < sd.n; i += kGroupThreads) ad[i] = as[i];
    }
}

}  // namespace

Batch group_batch(const Batch& b, int ng) {
    Batch gb = b;
    for (int i = 0; i < b.n_seq; ++i) {
        const GroupOff go = group_offsets(b, i, ng);
        gb.seq[i].raw_off = go.agg;
        gb.seq[i].keep_off = go.keep;
        gb.seq[i].pb_off = go.pb;
        gb.seq[i].part_off = 0;
    }
    return gb;
}

hipError_t launch_shared_select(const Batch& b, int L, int Hkv, int G, int mode, const float* raw,
                                const PartRec* part, HeadNorm* norms, float* gagg, int32_t* gkeep,
                                int32_t* gpb, uint32_t* key_scratch, int32_t* keep, int32_t* pb,
                                float* agg_out, uint32_t* ticket, hipStream_t s) {
    const int ups = L * Hkv;
    const int ng = keep_groups(mode, L, Hkv);
    int64_t max_n = 0;
    for (int i = 0; i < b.n_seq; ++i) max_n = b.seq[i].n > max_n ? b.seq[i].n : max_n;
    if (max_n <= 0) return hipSuccess;
    const unsigned units = (unsigned)(b.n_seq * ups);
    hipLaunchKernelGGL(norm_kernel, dim3(units), dim3(kGroupThreads), 0, s, b, ups, G, part, norms);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((max_n + kAggRows - 1) / kAggRows), (unsigned)ng,
                    (unsigned)b.n_seq);
    if (G % 4 == 0 && G <= 8) {
        if (G == 4)
            hipLaunchKernelGGL(group_agg_kernel<4>, grid, dim3(kGroupThreads), 0, s, b, L, Hkv, G,
                               mode, raw, norms, gagg);
        else
            hipLaunchKernelGGL(group_agg_kernel<8>, grid, dim3(kGroupThreads), 0, s, b, L, Hkv, G,
                               mode, raw, norms, gagg);
    } else {
        hipLaunchKernelGGL(group_agg_kernel<0>, grid, dim3(kGroupThreads), 0, s, b, L, Hkv, G,
                           mode, raw, norms, gagg);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const Batch gb = group_batch(b, ng);
    e = launch_select_impl(gb, ng, 1, gagg, nullptr, gkeep, nullptr, key_scratch, gpb, ticket, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(broadcast_kernel, dim3(units), dim3(kGroupThreads), 0, s, b, L, Hkv, G,
                       mode, gkeep, gpb, gagg, keep, pb, agg_out);
    return hipGetLastError();
}

}  // namespace tria
