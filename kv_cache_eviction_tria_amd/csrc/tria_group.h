// Per-query-head z-normalisation constants and the geometry of shared keep
// sets, used by the selector and by the shared-keep-set aggregation.
#pragma once

#include "tria_internal.h"

namespace tria {

// Per-head z-normalisation constants: mu as an unevaluated sum of two floats
// (hi + lo) and 1/sigma.  z = ((s - hi) - lo) * isg in fp32: the subtraction
// removes the head's common offset first, so z keeps ~1e-6 relative accuracy.
struct HeadNorm {
    float hi, lo, isg;
};

__device__ __forceinline__ float znorm(float s, const HeadNorm& c) {
    return ((s - c.hi) - c.lo) * c.isg;
}

// Mean and 1/sigma of query head h of a unit from its tile partials P (record
// i*G + h of tile i), merged in fp64 by one wavefront in a fixed order (lanes
// stride over the tiles).  Population statistics over the finite scores;
// sigma = 0 gives 1/sigma = 0, i.e. z = 0.  The result is valid in every lane.
__device__ __forceinline__ HeadNorm merge_head_norm(const PartRec* __restrict__ P, int64_t tiles,
                                                    int G, int h) {
    const int lane = threadIdx.x & 63;
    double c = 0.0, a = 0.0;
    for (int64_t i = lane; i < tiles; i += 64) {
        const PartRec pr = P[i * G + h];
        double mean, m2;
        part_stats(pr, &mean, &m2);
        c += pr.cnt;
        a += pr.cnt * mean;
    }
    c = wave_sum_f64(c);
    a = wave_sum_f64(a);
    const double mu = c > 0.0 ? a / c : 0.0;
    double m2 = 0.0;
    for (int64_t i = lane; i < tiles; i += 64) {
        const PartRec pr = P[i * G + h];
        double mean, mt;
        part_stats(pr, &mean, &mt);
        const double d = mean - mu;
        m2 += mt + pr.cnt * d * d;
    }
    m2 = wave_sum_f64(m2);
    const double var = c > 0.0 ? m2 / c : 0.0;
    const float hi = (float)mu;
    return HeadNorm{hi, (float)(mu - (double)hi), var > 0.0 ? (float)(1.0 / sqrt(var)) : 0.0f};
}

// Keep-set sharing (TRIA_KEEP_* in tria.h): the units of a sequence form
// keep_groups() groups; each group is selected once on the max over its
// members' z-scores, and every member is compacted with the group's keep set.
//   per unit:    group = unit (l, g)      (the plain per-unit pass)
//   per KV head: group g = units (l, g) for every layer l
//   global:      one group of every unit
__host__ __device__ inline int keep_groups(int mode, int L, int Hkv) {
    return mode == TRIA_KEEP_PER_KV_HEAD ? Hkv : (mode == TRIA_KEEP_GLOBAL ? 1 : L * Hkv);
}

// Offsets of sequence `seq`'s blocks in the group-level arrays (group score
// [ng][n], kept rows [ng][kept], chunk prefix counts [ng][chunk_bounds(kept)])
// when every sequence has ng groups, in sequence order.  seq = n_seq gives the
// totals.
struct GroupOff {
    int64_t agg, keep, pb;
};
__host__ __device__ inline GroupOff group_offsets(const Batch& b, int seq, int ng) {
    GroupOff o = {0, 0, 0};
    for (int i = 0; i < seq; ++i) {
        o.agg += (int64_t)ng * b.seq[i].n;
        o.keep += (int64_t)ng * b.seq[i].kept;
        o.pb += (int64_t)ng * chunk_bounds(b.seq[i].kept);
    }
    return o;
}

// Shared-keep-set selection of a batch whose units are L*Hkv per sequence:
// per-head norms from the partials, the group scores, one selection per group
// (the selector with identity norms over the group scores) and the copy of
// each group's kept rows and chunk prefix counts to its members.  Scratch:
// norms [n_seq*L*Hkv*G], gagg / gkeep / gpb sized by group_offsets(b, n_seq,
// ng), key_scratch as select_key_scratch_rows(group batch, ng, 1).  agg_out
// (optional, [.. units][n]) receives each unit's group score.
hipError_t launch_shared_select(const Batch& b, int L, int Hkv, int G, int mode, const float* raw,
                                const PartRec* part, HeadNorm* norms, float* gagg, int32_t* gkeep,
                                int32_t* gpb, uint32_t* key_scratch, int32_t* keep, int32_t* pb,
                                float* agg_out, uint32_t* ticket, hipStream_t s);

// The batch the group-level selection runs on: G = 1 score per row, offsets
// of the group-level arrays.
Batch group_batch(const Batch& b, int ng);

}  // namespace tria
