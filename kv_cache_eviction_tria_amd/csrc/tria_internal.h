// Internal definitions shared by the gfx950 kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tria.h"

namespace tria {

// Native vector types (the non-temporal load/store builtins take these).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockRows = TRIA_BLOCK;  // rows per paged block
constexpr int kMaxSeq = TRIA_MAX_SEQ;

// Per-sequence pass geometry (a contiguous cache is one sequence).
struct SeqDesc {
    int64_t n;         // cached rows of every unit of the sequence
    int64_t kept;      // rows kept by the pass
    int64_t s_end;     // candidates are rows [s_end, w_start); the rest are protected
    int64_t w_start;
    int64_t raw_off;   // float offset of the sequence's [L][Hkv][n][G] raw-score block
    int64_t keep_off;  // int offset of the sequence's [L][Hkv][kept] keep-index block
};

struct Batch {
    int32_t n_seq;
    int32_t max_tiles;  // score tiles of the longest sequence
    SeqDesc seq[kMaxSeq];
};

// Where the rows of a unit live.  bt == nullptr: contiguous [L][Hkv][cap];
// otherwise paged [L][n_blocks][Hkv][16] through the block table.
struct CacheView {
    uint8_t* k;
    uint8_t* v;
    int32_t* pos;
    int64_t cap;
    int64_t n_blocks;
    const int32_t* bt;
    int32_t max_blocks;
    int32_t L;
    int32_t Hkv;
    int32_t kb;  // K row bytes
    int32_t vb;  // V row bytes
};

struct UnitId {
    int seq, l, g;
};

__device__ __forceinline__ UnitId unit_id(const CacheView& c, int u) {
    const int per_seq = c.L * c.Hkv;
    UnitId id;
    id.seq = u / per_seq;
    const int rem = u - id.seq * per_seq;
    id.l = rem / c.Hkv;
    id.g = rem - id.l * c.Hkv;
    return id;
}

// Index of logical row r of a unit in its row array (multiply by the row size).
__device__ __forceinline__ int64_t row_index(const CacheView& c, const UnitId& id, int64_t r) {
    if (c.bt == nullptr) return ((int64_t)id.l * c.Hkv + id.g) * c.cap + r;
    const int32_t blk = c.bt[(int64_t)id.seq * c.max_blocks + (r >> 4)];
    return (((int64_t)id.l * c.n_blocks + blk) * c.Hkv + id.g) * kBlockRows + (r & (kBlockRows - 1));
}

// Query heads of a group are scored in sub-groups of 8, 4, 2, 1 heads (one
// kernel instantiation per sub-group size); sub-group (j0, gt) covers heads
// j0 .. j0+gt-1.
__host__ __device__ inline int subgroup_size(int G, int j0) {
    const int rem = G - j0;
    return rem >= 8 ? 8 : (rem >= 4 ? 4 : (rem >= 2 ? 2 : 1));
}
__host__ __device__ inline int subgroup_start(int G, int j) {
    int j0 = 0;
    while (j0 + subgroup_size(G, j0) <= j) j0 += subgroup_size(G, j0);
    return j0;
}

// Coefficient-table geometry of one unit (4-byte words), shared by prep and score.
// Per-head arrays are stored sub-group by sub-group so that the score kernel
// addresses its sub-group with compile-time strides:
//   f16 : float, sub-group block at j0*F*3: [F][gt][3] = {Re C, Im C, w}
//   q8_0: int32 hi[G][W], int32 lo[G][W], float sig[G][NB],
//         float w with sub-group block at j0*F: [F][gt]
//         (hi, lo: balanced base-256 digits of the quantised trig coefficients,
//          packed in the byte order of the stored row; W = words per row)
struct CoefGeom {
    int hd, F, G, NB, W;
    int hi_off, lo_off, sig_off, w_off;
    int words;
};

__host__ __device__ inline CoefGeom coef_geom(int k_type, int hd, int G) {
    CoefGeom cg;
    cg.hd = hd;
    cg.F = hd / 2;
    cg.G = G;
    cg.NB = hd / 32;
    cg.W = (34 * cg.NB + 3) / 4;
    if (k_type == TRIA_KV_F16) {
        cg.hi_off = cg.lo_off = cg.sig_off = cg.w_off = 0;
        cg.words = cg.F * G * 3;
    } else {
        cg.hi_off = 0;
        cg.lo_off = G * cg.W;
        cg.sig_off = 2 * G * cg.W;
        cg.w_off = cg.sig_off + G * cg.NB;
        cg.words = cg.w_off + cg.F * G;
    }
    // keep every unit's table 64-byte aligned for wide scalar loads
    cg.words = (cg.words + 15) & ~15;
    return cg;
}

// Launch helpers implemented in the kernel files.
hipError_t launch_prep(const CacheView& cv, const Batch& b, int n_units, int k_type, int G,
                       int hd, const float* q_re, const float* q_im, const float* w,
                       const double* omega, const double* m_re, const double* m_im,
                       int32_t* coef, hipStream_t s);
hipError_t launch_score(const CacheView& cv, const Batch& b, int n_units, int k_type, int G,
                        int hd, const int32_t* coef, float* raw, hipStream_t s);
hipError_t launch_select(const Batch& b, int n_units_per_seq, int G, const float* raw,
                         int32_t* keep, float* agg, hipStream_t s);
hipError_t launch_compact(const CacheView& cv, const Batch& b, int n_units,
                          const int32_t* keep, hipStream_t s);

}  // namespace tria
