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
    int64_t part_off;  // tile offset of the sequence's [L][Hkv][tiles(n)] moment partials
    int64_t pb_off;    // int offset of the sequence's [L][Hkv][chunk_bounds(kept)] prefix counts
};

struct Batch {
    int32_t n_seq;
    // Coefficient tables are laid out per unit of the whole model; a batch
    // over layers [coef_l0, coef_l0 + L) of a coef_L-layer model finds unit
    // (seq, l, g)'s table at ((seq * coef_L + coef_l0 + l) * Hkv + g).
    // coef_L == 0: the batch covers the whole model.
    int32_t coef_l0;
    int32_t coef_L;
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

// Moment partials: the raw scores of a unit are summarised per tile of
// kPartRows rows and per query head as {finite count c, shift a (the tile's
// first finite score), sum of d = s - a, sum of d^2} in fp32 (exact for equal
// scores; d is small against the scores' common offset), record
// ((part_off + unit*tiles + tile)*G + head).  One wavefront summarises a tile:
// lane i holds rows i, i + 64, i + 128 and i + 192.  The selector forms the
// tile mean m = a + sum(d)/c and M2 = sum(d^2) - sum(d)^2/c, then merges the
// tiles exactly in fp64:  N = sum c_t,  mu = sum c_t m_t / N,
// M2 = sum (M2_t + c_t (m_t - mu)^2).
constexpr int kPartRows = 256;
constexpr int kPartLaneRows = kPartRows / 64;
struct PartRec {
    float cnt, shift, sum, sumsq;
};
__host__ __device__ inline int64_t part_tiles(int64_t n) { return (n + kPartRows - 1) / kPartRows; }

// The DPP move of v (old value 0 where the row mask excludes a row).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sums over the 64 lanes of a wavefront (fixed order), returned to every lane:
// pairs and quads by quad permutes, rows of 8 and 16 by mirrors, then the row
// broadcasts of lanes 15 and 31 leave the total in lane 63.
template <typename T, T (*MOV)(T), T (*MOV2)(T), T (*MOV3)(T), T (*MOV4)(T), T (*MOV5)(T),
          T (*MOV6)(T)>
__device__ __forceinline__ T wave_sum_dpp(T v) {
    v += MOV(v);
    v += MOV2(v);
    v += MOV3(v);
    v += MOV4(v);
    v += MOV5(v);
    v += MOV6(v);
    return v;  // total in lane 63
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = wave_sum_dpp<float, dpp_f32<0xB1, 0xf>, dpp_f32<0x4E, 0xf>, dpp_f32<0x141, 0xf>,
                     dpp_f32<0x140, 0xf>, dpp_f32<0x142, 0xa>, dpp_f32<0x143, 0xc>>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = wave_sum_dpp<double, dpp_f64<0xB1, 0xf>, dpp_f64<0x4E, 0xf>, dpp_f64<0x141, 0xf>,
                     dpp_f64<0x140, 0xf>, dpp_f64<0x142, 0xa>, dpp_f64<0x143, 0xc>>(v);
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Moment partial of one wavefront's tile for NH heads, fed one 64-row slice
// at a time in row order: lane i holds row i of the slice in s[] (valid[]
// false for rows past the end and non-finite scores).  The shift is the
// tile's first finite score, so counts and shifts are wavefront-uniform.
template <int NH>
struct WaveMoments {
    float shift[NH], sd[NH], sq[NH];
    int cnt[NH];
    __device__ __forceinline__ WaveMoments() {
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            shift[j] = 0.0f;
            sd[j] = 0.0f;
            sq[j] = 0.0f;
            cnt[j] = 0;
        }
    }
    __device__ __forceinline__ void add(const float (&s)[NH], const bool (&valid)[NH]) {
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            const uint64_t m = __ballot(valid[j]);
            if (cnt[j] == 0 && m) {
                const int first = __ffsll((unsigned long long)m) - 1;
                shift[j] = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s[j]), first));
            }
            cnt[j] += __popcll(m);
            const float d = valid[j] ? s[j] - shift[j] : 0.0f;
            sd[j] += d;
            sq[j] = fmaf(d, d, sq[j]);
        }
    }
    // Lane 0 writes head j's record to out[j] for j < nh.
    __device__ __forceinline__ void emit(PartRec* out, int nh = NH) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            const float a = wave_sum_f32(sd[j]);
            const float b = wave_sum_f32(sq[j]);
            if (lane == 0 && j < nh) out[j] = PartRec{(float)cnt[j], shift[j], a, b};
        }
    }
};

// Mean and M2 of a tile record (fp64).
__device__ __forceinline__ void part_stats(const PartRec& p, double* mean, double* m2) {
    if (p.cnt > 0.0f) {
        const double c = p.cnt, sd = p.sum;
        *mean = (double)p.shift + sd / c;
        const double v = (double)p.sumsq - sd * sd / c;
        *m2 = v > 0.0 ? v : 0.0;
    } else {
        *mean = 0.0;
        *m2 = 0.0;
    }
}

// Compaction works in chunks of kChunkRows destination rows.  For every unit
// the selector also writes P(64 e) for e < chunk_bounds(kept), where P(x) is
// the number of kept rows below row x: the moves that read rows of chunk c are
// exactly those with ranks P(64 c) .. P(64 c + 64) - 1.
constexpr int kChunkRows = 64;
__host__ __device__ inline int64_t chunk_count(int64_t kept) {
    return (kept + kChunkRows - 1) / kChunkRows;
}
__host__ __device__ inline int64_t chunk_bounds(int64_t kept) { return chunk_count(kept) + 1; }

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

__device__ __forceinline__ int64_t coef_unit(const Batch& b, const CacheView& c, const UnitId& id) {
    const int cl = b.coef_L ? b.coef_L : c.L;
    return ((int64_t)id.seq * cl + b.coef_l0 + id.l) * c.Hkv + id.g;
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
//   q8_0, hd % 128 == 0 (q8_f16): trig coefficients as fp16 pairs hi + lo,
//         laid out like the stored row: for stored word k (bytes 4k..4k+3) of
//         head j, the coefficients of those four bytes (zero for scale bytes)
//         as four halves in two words: hi[G][W][2], lo[G][W][2]; each head's
//         coefficients carry a power-of-two scale, undone by osc[G] (float);
//         float w with sub-group block at j0*F: [F][gt]
//   q8_0, other widths: int32 digit[kCoefDigits][G][W], float sig[G][NB],
//         float w with sub-group block at j0*F: [F][gt]
//         (digit i: base-256 digit i, least significant first, of the
//          32-bit quantised trig coefficients, packed in the byte order of the
//          stored row; W = words per row)
constexpr int kCoefDigits = 4;
struct CoefGeom {
    int hd, F, G, NB, W;
    bool q8_f16;
    int hi_off, lo_off, osc_off;  // q8_f16
    int digit_off, sig_off;       // integer digits
    int w_off;
    int words;
};

__host__ __device__ inline CoefGeom coef_geom(int k_type, int hd, int G) {
    CoefGeom cg;
    cg.hd = hd;
    cg.F = hd / 2;
    cg.G = G;
    cg.NB = hd / 32;
    cg.W = (34 * cg.NB + 3) / 4;
    cg.q8_f16 = k_type == TRIA_KV_Q8_0 && hd % 128 == 0;
    cg.hi_off = cg.lo_off = cg.osc_off = cg.digit_off = cg.sig_off = cg.w_off = 0;
    if (k_type == TRIA_KV_F16) {
        cg.words = cg.F * G * 3;
    } else if (cg.q8_f16) {
        cg.hi_off = 0;
        cg.lo_off = 2 * G * cg.W;
        cg.osc_off = 4 * G * cg.W;
        cg.w_off = cg.osc_off + G;
        cg.words = cg.w_off + cg.F * G;
    } else {
        cg.digit_off = 0;  // digit i of head j at i * G * W + j * W
        cg.sig_off = kCoefDigits * G * cg.W;
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
// part == nullptr: no moment partials.
hipError_t launch_score(const CacheView& cv, const Batch& b, int n_units, int k_type, int G,
                        int hd, const int32_t* coef, float* raw, PartRec* part, hipStream_t s);
// Compaction state owned by a context: per-(unit, chunk) flags (zeroed once
// when allocated, then stamped with a new epoch by every launch), the task
// counter and epoch words, and an error word set by a workgroup that gave up
// waiting.
struct CompactState {
    uint32_t* flags;
    int64_t flag_words;
    uint32_t* ticket;  // [0] task counter, [1] flag epoch (see reset_ticket)
    int* err;
    int max_groups;    // > 0: at most this many workgroups (1: every task in order)
};

// Run by one thread of the kernel that precedes a compaction on its stream
// (the selector, or the prefix-count kernel): the task counter restarts and
// the epoch the compaction stamps its flags with advances (0, the flags'
// initial value, is skipped).  The epoch lives on the device, not in a kernel
// argument, so that a captured graph replayed many times still gives every
// compaction a new epoch and stale flags of an earlier replay never match.
__device__ __forceinline__ void reset_ticket(uint32_t* ticket) {
    ticket[0] = 0u;
    const uint32_t e = ticket[1] + 1u;
    ticket[1] = e ? e : 1u;
}
// pb: the selector's chunk prefix counts for these units, or nullptr to
// derive them from keep (caller-provided kept indices).
hipError_t launch_compact(const CacheView& cv, const Batch& b, int n_units, const int32_t* keep,
                          const int32_t* pb, int32_t* pb_scratch, CompactState& st,
                          uint32_t* ticket, hipStream_t s);
// Flags a launch over these units needs.
int64_t compact_flag_words(const Batch& b, int n_units);

}  // namespace tria
