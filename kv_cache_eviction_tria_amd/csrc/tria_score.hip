// score: raw per-query-head score of every cached row.
//
//   s_j(r) = sum_f Re(C_{j,f} conj(K_f(r))) + sum_f w_{j,f} |K_f(r)|,
//   K_f = k[f] + i k[f + hd/2]
//
// scored directly on the stored rotated key ("TriAttention Native C++
// Worklog", section "Phase 9: final root cause - native scorer used the wrong
// formulation": query-side phase term plus the additive term on |K_rot|), for
// the G query heads of the row's KV head (llama.cpp page "TriAttention
// KV-Cache Eviction (--triattention)", section 5 "Phase C").
//
// Row-per-lane kernels (q8_0, and fp16 widths that are not a multiple of 64):
// one lane per cached row at a time; a wavefront scores a tile of 256 rows
// (four per lane), 1024 rows per workgroup.  Every lane of a wave needs the
// same coefficient at the same time, so the unit's table (built by prep) is
// read through scalar loads into SGPRs and fed to the VALU as the scalar
// operand.  Each lane reads its whole row with wide loads; one load
// instruction touches a cache line per lane and the following loads of the
// row hit the same lines in L1, so K crosses HBM once.  The sqrt of |K_f|^2
// is shared by all G heads.
//
// q8_0 rows: the trig part is an integer dot product per 32-value block:
// sum_d q_d c_d = sig * sum_d q_d v_d with v the 32-bit quantised coefficient
// split into four base-256 digits, taken straight from the stored bytes (the
// digit tables follow the row's byte layout, scale bytes carry zero digits) on
// the matrix cores as 4x4x4 int8 blocks whose lanes are the rows (see the
// kernel); the block scale d and sig are applied once per block.  The |K_f|
// term dequantises q * d in fp32.
//
// fp16 rows with hd % 64 == 0 take the matrix-core path instead: the trig
// series and the norm-term sum are both contractions of a row over its
// dimensions (pairs) against G per-head coefficient vectors, i.e. a
// [16 rows x hd] x [hd x 16 heads] product per step, run as
// v_mfma_f32_16x16x32_f16 with the fp16 key as the B operand as stored and the
// coefficients split into two fp16 parts (hi + lo, per-head power-of-two
// scale) so the products keep fp32-level accuracy; |K_f| is formed on the
// VALU and split the same way.  The VALU then only forms |K_f| and the
// statistics, about half of its work in the row-per-lane kernel.
//
// Each wavefront also summarises its rows' scores per head (count, mean,
// squared deviations; fp64) for the selector's z-normalisation, so the raw
// scores are not read an extra time to form the head statistics.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kScoreThreads = 256;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}
__device__ __forceinline__ float sbyte(uint32_t x, int i) {
    return (float)(int8_t)(x >> (8 * i));
}

// A wave-uniform zero the compiler cannot see through.
__device__ __forceinline__ int opaque_zero_s() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// An empty asm that "reads and writes" every accumulator: all work on the
// accumulators before it completes before any work after it.  Placed between
// chunks of frequency pairs it keeps each chunk's coefficients (scalar
// registers) live only for that chunk; without it the scheduler interleaves
// the per-head chains freely and spills the coefficient table.
template <int GT>
__device__ __forceinline__ void sync_acc(float (&acc)[GT]) {
    if constexpr (GT == 1) {
        asm volatile("" : "+v"(acc[0]));
    } else if constexpr (GT == 2) {
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
    } else if constexpr (GT == 4) {
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
    } else {
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]),
                     "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]));
    }
}

// Raw scores are written once and read once, by the selector: streaming
// (non-temporal) stores (the q8_0 scorer measured 3-5 % faster with them).
template <int GT>
__device__ __forceinline__ void store_scores(float* dst, const float (&acc)[GT], bool packed) {
    typedef float f2e __attribute__((ext_vector_type(2)));
    typedef float f4e __attribute__((ext_vector_type(4)));
    if (packed) {
        if constexpr (GT == 1) {
            __builtin_nontemporal_store(acc[0], dst);
        } else if constexpr (GT == 2) {
            __builtin_nontemporal_store(f2e{acc[0], acc[1]}, reinterpret_cast<f2e*>(dst));
        } else if constexpr (GT == 4) {
            __builtin_nontemporal_store(f4e{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<f4e*>(dst));
        } else {
            __builtin_nontemporal_store(f4e{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<f4e*>(dst));
            __builtin_nontemporal_store(f4e{acc[4], acc[5], acc[6], acc[7]}, reinterpret_cast<f4e*>(dst + 4));
        }
    } else {
#pragma unroll
        for (int j = 0; j < GT; ++j) __builtin_nontemporal_store(acc[j], dst + j);
    }
}

// First row of this wavefront's tile: each wavefront scores kPartRows rows,
// lane i taking rows i, i + 64, ... (each load instruction still covers 64
// consecutive rows), so the per-wavefront set-up and the moment reduction are
// paid once per kPartRows rows.
__device__ __forceinline__ int64_t wave_tile() {
    return (int64_t)blockIdx.x * (kScoreThreads / 64) + (threadIdx.x >> 6);
}

// Moment partial of this wavefront's tile for heads j0 .. j0+GT-1.
template <int GT>
__device__ __forceinline__ void emit_moments(const WaveMoments<GT>& mom, const SeqDesc& sd,
                                             const UnitId& id, int Hkv, int64_t n, int G, int j0,
                                             PartRec* part) {
    const int64_t tile = sd.part_off + ((int64_t)id.l * Hkv + id.g) * part_tiles(n) + wave_tile();
    mom.emit(part + tile * G + j0);
}

template <int GT>
__device__ __forceinline__ void add_moments(WaveMoments<GT>& mom, const float (&acc)[GT],
                                            bool in_range) {
    bool valid[GT];
#pragma unroll
    for (int j = 0; j < GT; ++j) valid[j] = in_range && isfinite(acc[j]);
    mom.add(acc, valid);
}

// Pieces an fp16 row is walked in: the fewest that divide its HD/16 chunks per
// half-row into groups of at most 8 (one 128-byte line per half-row piece, 32
// registers).  Smaller pieces read each line in two visits, and the line is
// often gone from L2 by the second: HBM traffic rose to 1.8x the row bytes.
constexpr int f16_pieces(int hd) {
    const int c = hd / 16;
    for (int p = 1; p <= c; ++p)
        if (c % p == 0 && c / p <= 8) return p;
    return c;
}

template <int HD, int GT>
__global__ __launch_bounds__(kScoreThreads) void score_f16_kernel(
    CacheView cv, Batch b, int G, int j0, const float* __restrict__ coef, int coef_words,
    float* __restrict__ raw, PartRec* __restrict__ part) {
    constexpr int F = HD / 2;
    constexpr int NV = HD / 8;  // 16-byte chunks per row
    constexpr int PIECES = f16_pieces(HD);
    const int u = blockIdx.y;
    const UnitId id = unit_id(cv, u);
    const int64_t n = b.seq[id.seq].n;
    const int64_t wbase = wave_tile() * kPartRows;
    if (wbase >= n) return;
    const float* __restrict__ C = coef + coef_unit(b, cv, id) * coef_words + j0 * F * 3;
    float* rout = raw + b.seq[id.seq].raw_off + ((int64_t)id.l * cv.Hkv + id.g) * n * G + j0;
    const bool packed = (G == GT);
    WaveMoments<GT> mom;

#pragma unroll 1
    for (int it = 0; it < kPartLaneRows; ++it) {
        const int64_t r0 = wbase + it * 64;
        if (r0 >= n) break;
        // Lanes past the end recompute the last row and skip the store, so the
        // whole wave runs one straight-line body.
        const int64_t r_out = r0 + (threadIdx.x & 63);
        const int64_t r = r_out < n ? r_out : n - 1;
        // Re-read the coefficients through the scalar cache on every pass: the
        // offset is zero but opaque to the compiler, so it cannot hoist hundreds
        // of table values out of the loop into (spilled) registers.
        const float* __restrict__ Ci = C + opaque_zero_s();
        const u32x4* row = reinterpret_cast<const u32x4*>(cv.k + row_index(cv, id, r) * (HD * 2));

        float acc[GT];
#pragma unroll
        for (int j = 0; j < GT; ++j) acc[j] = 0.0f;
        // The row is walked in PIECES pieces (a rolled loop): piece q holds the
        // pairs [q FP, (q+1) FP), i.e. CH 16-byte chunks of the first half of
        // the row and the matching CH chunks of the second half.  Only one
        // piece is live at a time, which keeps wide rows from filling the
        // register file (hd 256 would need 128 registers for the whole row).
        constexpr int FP = F / PIECES;
        constexpr int CH = FP / 8;
        // Pairs in chunks whose coefficients fit the scalar register file.
        constexpr int CP = GT >= 8 ? 1 : 8 / GT;
#pragma unroll 1
        for (int q = 0; q < PIECES; ++q) {
            u32x4 dre[CH], dim[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                dre[i] = row[q * CH + i];
                dim[i] = row[NV / 2 + q * CH + i];
            }
            const uint32_t* wre = reinterpret_cast<const uint32_t*>(dre);
            const uint32_t* wim = reinterpret_cast<const uint32_t*>(dim);
            const float* Cq = Ci + q * FP * GT * 3;
#pragma unroll
            for (int f = 0; f < FP; ++f) {
                if (f % CP == 0) sync_acc<GT>(acc);
                const uint32_t wr = wre[f >> 1], wi = wim[f >> 1];
                const float kre = (f & 1) ? half_hi(wr) : half_lo(wr);
                const float kim = (f & 1) ? half_hi(wi) : half_lo(wi);
                const float mag = __builtin_amdgcn_sqrtf(fmaf(kre, kre, kim * kim));
                const float* c = Cq + f * GT * 3;
#pragma unroll
                for (int j = 0; j < GT; ++j) {
                    acc[j] = fmaf(c[3 * j + 0], kre, acc[j]);
                    acc[j] = fmaf(c[3 * j + 1], kim, acc[j]);
                    acc[j] = fmaf(c[3 * j + 2], mag, acc[j]);
                }
            }
        }
        if (r_out < n) store_scores<GT>(rout + r_out * G, acc, packed);
        if (part) add_moments<GT>(mom, acc, r_out < n);
    }
    if (part) emit_moments<GT>(mom, b.seq[id.seq], id, cv.Hkv, n, G, j0, part);
}

// Waves per SIMD the register allocation must allow (1: no constraint).  At
// hd 128 with four heads the kernel otherwise takes 73 vector + 8 matrix
// accumulator registers (5 waves per SIMD); held to 80 in all it keeps 6
// waves per SIMD resident without spilling and scores 3 % faster.
template <int HD, int GT>
constexpr int kQ8MinWaves = (HD == 128 && GT == 4) ? 6 : 1;

template <int HD, int GT>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(kQ8MinWaves<HD, GT>, 8))) void score_q8_kernel(
    CacheView cv, Batch b, int G, int j0, const int32_t* __restrict__ coef, int coef_words,
    float* __restrict__ raw, PartRec* __restrict__ part) {
    constexpr int F = HD / 2;
    constexpr int NB = HD / 32;
    constexpr int RB = 34 * NB;         // row bytes
    constexpr int W = (RB + 3) / 4;     // 32-bit words covering a row
    constexpr bool kOdd = (NB & 1) != 0; // rows only 2-byte aligned
    const int u = blockIdx.y;
    const UnitId id = unit_id(cv, u);
    const int64_t n = b.seq[id.seq].n;
    if ((int64_t)blockIdx.x * (kScoreThreads / 64) * kPartRows >= n) return;  // whole block
    const int64_t wbase = wave_tile() * kPartRows;
    const CoefGeom cg = coef_geom(TRIA_KV_Q8_0, HD, G);
    const int32_t* __restrict__ T = coef + coef_unit(b, cv, id) * coef_words;
    // The trig digits of this sub-group as matrix-core A operands: word k of
    // head slot h (zero for slots past the sub-group), one table per digit.
    constexpr int HS = GT < 4 ? 4 : GT;  // head slots, a multiple of 4
    __shared__ uint32_t dtab[kCoefDigits][HS][W];
    for (int i = threadIdx.x; i < kCoefDigits * HS * W; i += kScoreThreads) {
        const int dg = i / (HS * W), h = (i / W) % HS, k = i % W;
        dtab[dg][h][k] = h < GT ? (uint32_t)T[cg.digit_off + (dg * G + j0 + h) * W + k] : 0u;
    }
    __syncthreads();
    if (wbase >= n) return;
    const float* __restrict__ SIG = reinterpret_cast<const float*>(T + cg.sig_off) + j0 * NB;
    const float* __restrict__ WT = reinterpret_cast<const float*>(T + cg.w_off) + j0 * F;
    float* rout = raw + b.seq[id.seq].raw_off + ((int64_t)id.l * cv.Hkv + id.g) * n * G + j0;
    const bool packed = (G == GT);
    WaveMoments<GT> mom;

#pragma unroll 1
    for (int it = 0; it < kPartLaneRows; ++it) {
        const int64_t r0 = wbase + it * 64;
        if (r0 >= n) break;
        const int r_out = (int)r0 + (int)(threadIdx.x & 63);  // n < 2^31
        const int64_t r = r_out < n ? r_out : n - 1;
        // see score_f16_kernel: keep the tables in the scalar path
        const int z = opaque_zero_s();
        const uint8_t* rp = cv.k + row_index(cv, id, r) * RB;
        uint32_t wv[W];
        if constexpr (!kOdd) {
            if constexpr (RB % 16 == 0) {
                const u32x4* p4 = reinterpret_cast<const u32x4*>(rp);
#pragma unroll
                for (int i = 0; i < W / 4; ++i) {
                    const u32x4 t = p4[i];
                    wv[4 * i] = t.x; wv[4 * i + 1] = t.y; wv[4 * i + 2] = t.z; wv[4 * i + 3] = t.w;
                }
            } else if constexpr (RB % 8 == 0) {
                const u32x2* p2 = reinterpret_cast<const u32x2*>(rp);
#pragma unroll
                for (int i = 0; i < W / 2; ++i) {
                    const u32x2 t = p2[i];
                    wv[2 * i] = t.x; wv[2 * i + 1] = t.y;
                }
            } else {
                const uint32_t* p1 = reinterpret_cast<const uint32_t*>(rp);
#pragma unroll
                for (int i = 0; i < W; ++i) wv[i] = p1[i];
            }
        } else {
            // Row starts 0 or 2 bytes past a word boundary; read only bytes of this
            // row or the row before it, then realign.
            const uintptr_t a = reinterpret_cast<uintptr_t>(rp);
            const uint32_t sh = (uint32_t)(a & 3u);
            const uint32_t* ap = reinterpret_cast<const uint32_t*>(a - sh);
            uint32_t rw[W];
#pragma unroll
            for (int i = 0; i < W - 1; ++i) rw[i] = ap[i];
            rw[W - 1] = sh ? ap[W - 1] : (uint32_t)(*reinterpret_cast<const uint16_t*>(ap + W - 1));
#pragma unroll
            for (int i = 0; i < W - 1; ++i)
                wv[i] = sh ? __builtin_amdgcn_alignbyte(rw[i + 1], rw[i], 2u) : rw[i];
            wv[W - 1] = sh ? (rw[W - 1] >> 16) : rw[W - 1];
        }

        float dsc[NB];
#pragma unroll
        for (int bk = 0; bk < NB; ++bk) {
            const int o = 34 * bk;
            dsc[bk] = (o & 2) ? half_hi(wv[o >> 2]) : half_lo(wv[o >> 2]);
        }

        float acc[GT];
#pragma unroll
        for (int j = 0; j < GT; ++j) acc[j] = 0.0f;

        // trig part: per block, integer dot product of the stored int8 values with the
        // quantised coefficient digits, then one scale per (head, block).  The
        // products run on the matrix cores as 4x4x4 int8 blocks (16 per
        // instruction): block q of v_mfma_i32_4x4x4i8 is lanes 4q .. 4q + 3, its B
        // operand is word k of those lanes' four rows, its A operand lane 4q + m
        // holds head m's digit of word k, and the result lane 4q + n holds the
        // four heads' sums of its own row n, so every lane keeps its row.
        // (Words never hold quants of two blocks: a block's two scale bytes
        // separate them, and the scale bytes carry zero digits.)  The four
        // digits' sums e_i (|e_i| <= 32 * 127 * 128 < 2^19) form two exact
        // 32-bit integers, e3 * 256 + e2 (weight 2^16) and e1 * 256 + e0, each
        // rounded once to fp32 and accumulated with the (head, block) scale.
        // Digits go two at a time, so two accumulators per head slot are live.
        const uint32_t* __restrict__ dt = &dtab[0][0][0] + z + (threadIdx.x & 3) * W;
#pragma unroll
        for (int bk = 0; bk < NB; ++bk) {
            const int k0 = (34 * bk + 2) >> 2, k1 = (34 * bk + 33) >> 2;
#pragma unroll
            for (int half = 1; half >= 0; --half) {
                sync_acc<GT>(acc);
                i32x4 chi[HS / 4], clo[HS / 4];
#pragma unroll
                for (int c = 0; c < HS / 4; ++c) chi[c] = clo[c] = i32x4{0, 0, 0, 0};
#pragma unroll
                for (int k = k0; k <= k1; ++k) {
#pragma unroll
                    for (int c = 0; c < HS / 4; ++c) {
                        const int ahi = (int)dt[((2 * half + 1) * HS + 4 * c) * W + k];
                        const int alo = (int)dt[((2 * half) * HS + 4 * c) * W + k];
                        chi[c] = __builtin_amdgcn_mfma_i32_4x4x4i8(ahi, (int)wv[k], chi[c], 0, 0, 0);
                        clo[c] = __builtin_amdgcn_mfma_i32_4x4x4i8(alo, (int)wv[k], clo[c], 0, 0, 0);
                    }
                }
                const float wgt = half ? 65536.0f : 1.0f;
#pragma unroll
                for (int j = 0; j < GT; ++j)
                    acc[j] = fmaf((float)(chi[j >> 2][j & 3] * 256 + clo[j >> 2][j & 3]),
                                  dsc[bk] * (wgt * SIG[z + j * NB + bk]), acc[j]);
            }
        }
        // |K_f| term
        constexpr int CPQ = GT >= 8 ? 2 : 16 / GT;
#pragma unroll
        for (int f = 0; f < F; ++f) {
            if (f % CPQ == 0) sync_acc<GT>(acc);
            const int oe = 34 * (f >> 5) + 2 + (f & 31);
            const int oi = 34 * ((f + F) >> 5) + 2 + ((f + F) & 31);
            const float kr = sbyte(wv[oe >> 2], oe & 3) * dsc[f >> 5];
            const float ki = sbyte(wv[oi >> 2], oi & 3) * dsc[(f + F) >> 5];
            const float mag = __builtin_amdgcn_sqrtf(fmaf(kr, kr, ki * ki));
#pragma unroll
            for (int j = 0; j < GT; ++j) acc[j] = fmaf(WT[z + f * GT + j], mag, acc[j]);
        }
        if (r_out < n) store_scores<GT>(rout + (int64_t)r_out * G, acc, packed);
        if (part) add_moments<GT>(mom, acc, r_out < n);
    }
    if (part) emit_moments<GT>(mom, b.seq[id.seq], id, cv.Hkv, n, G, j0, part);
}


// ---------------------------------------------------------------------------
// q8_0 rows with hd % 128 == 0: row-per-lane, the trig products on the matrix
// cores in fp16.
//
// The row's int8 values are exact in fp16, so each stored word (four bytes) is
// fed as four halves to v_mfma_f32_4x4x4f16, blocked like the integer kernel
// above: block q of the instruction is lanes 4q .. 4q + 3, its B operand the
// four halves of one stored word of those lanes' rows, its A operand lane
// 4q + m head m's coefficients of the same four bytes (fp16 hi, then lo, each
// head scaled by a power of two; zero at the block scales), the result lane
// 4q + n the four heads' sums of row n.  Coefficients keep ~22 bits each, the
// products are exact and the sums fp32.  A Re dimension d < hd/2 and its Im
// partner d + hd/2 sit 17 * NB bytes apart, a whole number of words when
// NB % 4 == 0, so words k and k + 17 NB / 4 are taken together: their int8
// values are converted once (to fp32, then packed to fp16 for the matrix
// cores) and serve both the trig products of their two blocks and the |K_f|
// of the pairs they hold.  Per Re block b (and its Im block b + NB/2) the
// products accumulate unscaled and are scaled by the blocks' d and the heads'
// 2^-e once.
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int HD, int GT>
__global__ __launch_bounds__(kScoreThreads) void score_q8_f16_kernel(
    CacheView cv, Batch b, int G, int j0, const int32_t* __restrict__ coef, int coef_words,
    float* __restrict__ raw, PartRec* __restrict__ part) {
    constexpr int F = HD / 2;
    constexpr int NB = HD / 32;
    constexpr int RB = 34 * NB;       // row bytes (a multiple of 8)
    constexpr int W = RB / 4;         // words per row
    constexpr int OFFW = 17 * NB / 4; // Re word k pairs with Im word k + OFFW
    static_assert(NB % 4 == 0, "pairs must be whole words apart");
    const int u = blockIdx.y;
    const UnitId id = unit_id(cv, u);
    const int64_t n = b.seq[id.seq].n;
    if ((int64_t)blockIdx.x * (kScoreThreads / 64) * kPartRows >= n) return;  // whole block
    const int64_t wbase = wave_tile() * kPartRows;
    const CoefGeom cg = coef_geom(TRIA_KV_Q8_0, HD, G);
    const int32_t* __restrict__ T = coef + coef_unit(b, cv, id) * coef_words;
    // A operands of this sub-group: [head slot][word] = {hi halves, lo halves}
    // (zero past the sub-group)
    constexpr int HS = GT < 4 ? 4 : GT;
    __shared__ u32x4 atab[HS][W];
    for (int i = threadIdx.x; i < HS * W; i += kScoreThreads) {
        const int h = i / W, k = i % W;
        u32x4 a = {0u, 0u, 0u, 0u};
        if (h < GT) {
            const int32_t* hi = T + cg.hi_off + ((j0 + h) * W + k) * 2;
            const int32_t* lo = T + cg.lo_off + ((j0 + h) * W + k) * 2;
            a = u32x4{(uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)lo[0], (uint32_t)lo[1]};
        }
        atab[h][k] = a;
    }
    __syncthreads();
    if (wbase >= n) return;
    const float* __restrict__ OSC = reinterpret_cast<const float*>(T + cg.osc_off) + j0;
    const float* __restrict__ WT = reinterpret_cast<const float*>(T + cg.w_off) + j0 * F;
    float* rout = raw + b.seq[id.seq].raw_off + ((int64_t)id.l * cv.Hkv + id.g) * n * G + j0;
    const bool packed = (G == GT);
    WaveMoments<GT> mom;

#pragma unroll 1
    for (int it = 0; it < kPartLaneRows; ++it) {
        const int64_t r0 = wbase + it * 64;
        if (r0 >= n) break;
        const int r_out = (int)r0 + (int)(threadIdx.x & 63);  // n < 2^31
        const int64_t r = r_out < n ? r_out : n - 1;
        const int z = opaque_zero_s();
        const uint8_t* rp = cv.k + row_index(cv, id, r) * RB;
        uint32_t wv[W];
        if constexpr (RB % 16 == 0) {
            const u32x4* p4 = reinterpret_cast<const u32x4*>(rp);
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                const u32x4 t = p4[i];
                wv[4 * i] = t.x; wv[4 * i + 1] = t.y; wv[4 * i + 2] = t.z; wv[4 * i + 3] = t.w;
            }
        } else {
            const u32x2* p2 = reinterpret_cast<const u32x2*>(rp);
#pragma unroll
            for (int i = 0; i < W / 2; ++i) {
                const u32x2 t = p2[i];
                wv[2 * i] = t.x; wv[2 * i + 1] = t.y;
            }
        }
        float dsc[NB];
#pragma unroll
        for (int bk = 0; bk < NB; ++bk) {
            const int o = 34 * bk;
            dsc[bk] = (o & 2) ? half_hi(wv[o >> 2]) : half_lo(wv[o >> 2]);
        }
        float acc[GT];
#pragma unroll
        for (int j = 0; j < GT; ++j) acc[j] = 0.0f;
        const u32x4* __restrict__ at = &atab[0][0] + z + (threadIdx.x & 3) * W;

#pragma unroll
        for (int bk = 0; bk < NB / 2; ++bk) {  // Re block bk with Im block bk + NB/2
            sync_acc<GT>(acc);
            const int k0 = (34 * bk + 2) >> 2, k1 = (34 * bk + 33) >> 2;
            f32x4v cre[HS / 4], cim[HS / 4];
#pragma unroll
            for (int c = 0; c < HS / 4; ++c) cre[c] = cim[c] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = k0; k <= k1; ++k) {
                // the word's int8 values as fp32 (0 at scale bytes, whose coefficients
                // are zero), packed to fp16 for the matrix cores (exact: |q| <= 127)
                float xr[4], xi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int o = 4 * k + e - 34 * bk;
                    const bool quant = o >= 2 && o < 34;
                    xr[e] = quant ? sbyte(wv[k], e) : 0.0f;
                    xi[e] = quant ? sbyte(wv[k + OFFW], e) : 0.0f;
                }
                const half4v bre = __builtin_bit_cast(
                    half4v, u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xr[0], xr[1])),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xr[2], xr[3]))});
                const half4v bim = __builtin_bit_cast(
                    half4v, u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xi[0], xi[1])),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xi[2], xi[3]))});
#pragma unroll
                for (int c = 0; c < HS / 4; ++c) {
                    const u32x4* a = at + (4 * c) * W;
                    const u32x4 ar = a[k], ai = a[k + OFFW];
                    cre[c] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                        __builtin_bit_cast(half4v, u32x2{ar.x, ar.y}), bre, cre[c], 0, 0, 0);
                    cim[c] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                        __builtin_bit_cast(half4v, u32x2{ai.x, ai.y}), bim, cim[c], 0, 0, 0);
                    cre[c] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                        __builtin_bit_cast(half4v, u32x2{ar.z, ar.w}), bre, cre[c], 0, 0, 0);
                    cim[c] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                        __builtin_bit_cast(half4v, u32x2{ai.z, ai.w}), bim, cim[c], 0, 0, 0);
                }
                // |K_f| of the pairs whose Re value is in this word (block bk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int o = 4 * k + e - 34 * bk;
                    if (o < 2 || o >= 34) continue;  // a scale byte
                    const int f = 32 * bk + (o - 2);
                    const float kr = xr[e] * dsc[bk];
                    const float ki = xi[e] * dsc[bk + NB / 2];
                    const float mag = __builtin_amdgcn_sqrtf(fmaf(kr, kr, ki * ki));
#pragma unroll
                    for (int j = 0; j < GT; ++j) acc[j] = fmaf(WT[z + f * GT + j], mag, acc[j]);
                }
                // keep the next words' operand loads from being hoisted above this
                // word's work (they would hold registers the waves need)
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < GT; ++j) {
                const float sr = dsc[bk] * OSC[z + j], si = dsc[bk + NB / 2] * OSC[z + j];
                acc[j] = fmaf(cre[j >> 2][j & 3], sr, acc[j]);
                acc[j] = fmaf(cim[j >> 2][j & 3], si, acc[j]);
            }
        }
        if (r_out < n) store_scores<GT>(rout + (int64_t)r_out * G, acc, packed);
        if (part) add_moments<GT>(mom, acc, r_out < n);
    }
    if (part) emit_moments<GT>(mom, b.seq[id.seq], id, cv.Hkv, n, G, j0, part);
}

// ---------------------------------------------------------------------------
// Matrix-core scorer for fp16 rows (hd % 64 == 0).
//
// One wavefront scores a tile of kPartRows rows in steps of 16.  MFMA operand
// layout (v_mfma_f32_16x16x32_f16, checked on gfx950): lane m + 16 g of the A
// operand holds A[m][8 g + e], lane n + 16 g of the B operand holds
// B[8 g + e][n] (e = 0..7), and lane n + 16 g of the result holds C[4 g + i][n]
// (i = 0..3).  Here m = query head (of a chunk of up to 16), n = row of the
// step, and "k = 8 g + e" is mapped as follows:
//   trig step s (s < hd/32): dimension 32 s + 8 g + e of the row;
//   norm step t (t < F/32):  pair f = 32 t + 8 g + e.
// So lane (n, g) loads 16 bytes at dimension 32 s + 8 g for every s, which
// also gives it both halves of pairs 32 t + 8 g + e (steps t and t + F/32) for
// the norm term.  The A operands of the unit (coefficient hi and lo parts,
// zero for heads past the chunk) are built once per workgroup into LDS.
constexpr int kMfmaThreads = 256;
constexpr int kMfmaSteps = kPartRows / 16;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Coefficient of query head j in the row-per-lane table (sub-group blocks of
// [F][gt][3] = {Re C, Im C, w}).
__device__ __forceinline__ float f16_table_coef(const float* C, int G, int F, int j, int comp, int f) {
    const int j0 = subgroup_start(G, j), gt = subgroup_size(G, j0);
    return C[(j0 * F + f * gt + (j - j0)) * 3 + comp];
}

// Sum over the 16 lanes of a row of the wavefront, returned to all 16.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141, 0xf>(v);  // row_half_mirror
    v += dpp_f32<0x140, 0xf>(v);  // row_mirror
    return v;
}

template <int HD>
__global__ __launch_bounds__(kMfmaThreads) void score_f16_mfma_kernel(
    CacheView cv, Batch b, int G, int c0, int gc, const float* __restrict__ coef, int coef_words,
    float* __restrict__ raw, PartRec* __restrict__ part) {
    constexpr int F = HD / 2;
    constexpr int KS = HD / 32;  // trig steps
    constexpr int NS = F / 32;   // norm steps
    __shared__ u32x4 tab[(KS + NS) * 2 * 64];
    __shared__ int maxbits[16];

    const int u = blockIdx.y;
    const UnitId id = unit_id(cv, u);
    const int64_t n = b.seq[id.seq].n;
    if ((int64_t)blockIdx.x * (kMfmaThreads / 64) * kPartRows >= n) return;  // whole block
    const float* __restrict__ C = coef + coef_unit(b, cv, id) * coef_words;

    // Per-head power-of-two scale: the largest |coefficient| of head m maps into
    // [2^14, 2^15), inside the fp16 range with room for the lo part.
    if (threadIdx.x < 16) maxbits[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < gc * (HD + F); i += kMfmaThreads) {
        const int m = i / (HD + F), d = i - m * (HD + F);
        const int comp = d < F ? 0 : (d < HD ? 1 : 2);
        const int f = d < F ? d : (d < HD ? d - F : d - HD);
        const float a = fabsf(f16_table_coef(C, G, F, c0 + m, comp, f));
        atomicMax(&maxbits[m], __builtin_bit_cast(int, a));  // |x| orders like its bits
    }
    __syncthreads();
    for (int i = threadIdx.x; i < (KS + NS) * 64; i += kMfmaThreads) {
        const int p = i >> 6, ln = i & 63, m = ln & 15, g = ln >> 4;
        const float mx = __builtin_bit_cast(float, maxbits[m & 15]);
        const int ex = (mx > 0.0f && isfinite(mx)) ? 14 - ilogbf(mx) : 0;
        half8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = 0.0f;
            if (m < gc) {
                if (p < KS) {
                    const int d = 32 * p + 8 * g + e;
                    x = f16_table_coef(C, G, F, c0 + m, d < F ? 0 : 1, d < F ? d : d - F);
                } else {
                    x = f16_table_coef(C, G, F, c0 + m, 2, 32 * (p - KS) + 8 * g + e);
                }
                x = ldexpf(x, ex);
            }
            const _Float16 h = (_Float16)x;
            hi[e] = h;
            lo[e] = (_Float16)(x - (float)h);
        }
        tab[(2 * p) * 64 + ln] = __builtin_bit_cast(u32x4, hi);
        tab[(2 * p + 1) * 64 + ln] = __builtin_bit_cast(u32x4, lo);
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, nn = lane & 15, kg = lane >> 4;
    const int64_t tile = (int64_t)blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6);
    const int64_t t0 = tile * kPartRows;
    if (t0 >= n) return;

    // output scale of this lane's heads 4 kg + i (zero past the chunk)
    float osc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * kg + i;
        const float mx = __builtin_bit_cast(float, maxbits[m]);
        const int ex = (mx > 0.0f && isfinite(mx)) ? 14 - ilogbf(mx) : 0;
        osc[i] = m < gc ? ldexpf(1.0f, -ex) : 0.0f;
    }
    float* rout = raw + b.seq[id.seq].raw_off + ((int64_t)id.l * cv.Hkv + id.g) * n * G + c0;
    const bool vec_store = (G % 4 == 0) && (c0 % 4 == 0) && (4 * kg + 3 < gc);

    float shift[4], sd[4], sq[4], cf[4];
    bool have[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        shift[i] = 0.0f; sd[i] = 0.0f; sq[i] = 0.0f; cf[i] = 0.0f; have[i] = false;
    }

    // One step: 16 rows, their K bytes already in B.
    auto step = [&](const u32x4 (&B)[KS], int64_t r0) {
        const int64_t r_out = r0 + nn;
        // the table is re-read from LDS every step (an offset the compiler cannot
        // see through), instead of being hoisted into ~100 registers
        const u32x4* __restrict__ T = tab + lane + opaque_zero_s();
        // three independent accumulation chains (low-half trig, high-half
        // trig, norm term) so consecutive MFMAs do not wait on each other
        f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0, acc2 = acc0;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const half8 bl = __builtin_bit_cast(half8, B[t]);
            const half8 bh = __builtin_bit_cast(half8, B[t + NS]);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, T[(2 * t) * 64]), bl, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, T[(2 * (t + NS)) * 64]), bh, acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, T[(2 * t + 1) * 64]), bl, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, T[(2 * (t + NS) + 1) * 64]), bh, acc1, 0, 0, 0);
            // |K_f| for the lane's 8 pairs, split into fp16 hi + lo (round toward
            // zero, so a magnitude past the fp16 range keeps its hi finite)
            half8 mh, ml;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float k0r = (float)bl[e], k0i = (float)bh[e];
                const float k1r = (float)bl[e + 1], k1i = (float)bh[e + 1];
                const float m0 = __builtin_amdgcn_sqrtf(fmaf(k0r, k0r, k0i * k0i));
                const float m1 = __builtin_amdgcn_sqrtf(fmaf(k1r, k1r, k1i * k1i));
                const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(m0, m1));
                const half2v l = __builtin_bit_cast(
                    half2v, __builtin_amdgcn_cvt_pkrtz(m0 - (float)h[0], m1 - (float)h[1]));
                mh[e] = h[0]; mh[e + 1] = h[1];
                ml[e] = l[0]; ml[e + 1] = l[1];
            }
            const half8 wh = __builtin_bit_cast(half8, T[(2 * (KS + t)) * 64]);
            const half8 wl = __builtin_bit_cast(half8, T[(2 * (KS + t) + 1) * 64]);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh, mh, acc2, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wl, mh, acc2, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh, ml, acc2, 0, 0, 0);
        }

        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = ((acc0[i] + acc1[i]) + acc2[i]) * osc[i];
        const bool row_ok = r_out < n;
        if (row_ok) {
            if (vec_store) {
                typedef float f4e __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(f4e{v[0], v[1], v[2], v[3]},
                                            reinterpret_cast<f4e*>(rout + r_out * G + 4 * kg));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * kg + i < gc) __builtin_nontemporal_store(v[i], rout + r_out * G + 4 * kg + i);
            }
        }
        if (part) {
            bool valid[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) valid[i] = row_ok && (4 * kg + i < gc) && isfinite(v[i]);
            // shift = first finite score of the tile (row order) per head
            if (__ballot(!(have[0] && have[1] && have[2] && have[3]))) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint64_t mk = __ballot(valid[i]);
                    const uint32_t gm = (uint32_t)(mk >> (16 * kg)) & 0xffffu;
                    const int src = 16 * kg + (gm ? __builtin_ctz(gm) : 0);
                    const float sv = __shfl(v[i], src);
                    if (!have[i] && gm) {
                        shift[i] = sv;
                        have[i] = true;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = valid[i] ? v[i] - shift[i] : 0.0f;
                sd[i] += d;
                sq[i] = fmaf(d, d, sq[i]);
                cf[i] += valid[i] ? 1.0f : 0.0f;
            }
        }
    };
    // Rows of the step starting at r0 (rows past the end repeat the last row).
    auto load = [&](u32x4 (&B)[KS], int64_t r0) {
        const int64_t r_out = r0 + nn;
        const int64_t r = r_out < n ? r_out : n - 1;
        const uint8_t* rp = cv.k + row_index(cv, id, r) * (HD * 2) + 16 * kg;
#pragma unroll
        for (int s = 0; s < KS; ++s) B[s] = *reinterpret_cast<const u32x4*>(rp + 64 * s);
    };

#pragma unroll 1
    for (int st = 0; st < kMfmaSteps; ++st) {
        const int64_t r0 = t0 + 16 * st;
        if (r0 >= n) break;
        u32x4 B[KS];
        load(B, r0);
        step(B, r0);
    }
    if (part) {
        PartRec* out = part + (b.seq[id.seq].part_off +
                               ((int64_t)id.l * cv.Hkv + id.g) * part_tiles(n) + tile) * G + c0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float c = row16_sum(cf[i]);
            const float a = row16_sum(sd[i]);
            const float q = row16_sum(sq[i]);
            if (nn == 0 && 4 * kg + i < gc) out[4 * kg + i] = PartRec{c, shift[i], a, q};
        }
    }
}

template <int HD>
hipError_t run_f16_mfma(const CacheView& cv, const Batch& b, int n_units, int64_t max_n, int G,
                        const int32_t* coef, int words, float* raw, PartRec* part, hipStream_t s) {
    const int64_t rows_per_block = (int64_t)(kMfmaThreads / 64) * kPartRows;
    const dim3 grid((unsigned)((max_n + rows_per_block - 1) / rows_per_block), (unsigned)n_units);
    for (int c0 = 0; c0 < G; c0 += 16) {
        const int gc = G - c0 < 16 ? G - c0 : 16;
        hipLaunchKernelGGL((score_f16_mfma_kernel<HD>), grid, dim3(kMfmaThreads), 0, s, cv, b, G, c0,
                           gc, reinterpret_cast<const float*>(coef), words, raw, part);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int HD, int GT>
void run_f16(dim3 grid, hipStream_t s, const CacheView& cv, const Batch& b, int G, int j0,
             const int32_t* coef, int words, float* raw, PartRec* part) {
    hipLaunchKernelGGL((score_f16_kernel<HD, GT>), grid, dim3(kScoreThreads), 0, s, cv, b, G, j0,
                       reinterpret_cast<const float*>(coef), words, raw, part);
}
template <int HD, int GT>
void run_q8(dim3 grid, hipStream_t s, const CacheView& cv, const Batch& b, int G, int j0,
            const int32_t* coef, int words, float* raw, PartRec* part) {
    if constexpr (HD % 128 == 0)
        hipLaunchKernelGGL((score_q8_f16_kernel<HD, GT>), grid, dim3(kScoreThreads), 0, s, cv, b, G,
                           j0, coef, words, raw, part);
    else
        hipLaunchKernelGGL((score_q8_kernel<HD, GT>), grid, dim3(kScoreThreads), 0, s, cv, b, G,
                           j0, coef, words, raw, part);
}

using Runner = void (*)(dim3, hipStream_t, const CacheView&, const Batch&, int, int,
                        const int32_t*, int, float*, PartRec*);

template <int HD>
Runner pick(int k_type, int gt) {
    if (k_type == TRIA_KV_F16) {
        switch (gt) {
            case 1: return run_f16<HD, 1>;
            case 2: return run_f16<HD, 2>;
            case 4: return run_f16<HD, 4>;
            default: return run_f16<HD, 8>;
        }
    }
    switch (gt) {
        case 1: return run_q8<HD, 1>;
        case 2: return run_q8<HD, 2>;
        case 4: return run_q8<HD, 4>;
        default: return run_q8<HD, 8>;
    }
}

Runner pick_runner(int k_type, int hd, int gt) {
    switch (hd) {
        case 32: return pick<32>(k_type, gt);
        case 64: return pick<64>(k_type, gt);
        case 96: return pick<96>(k_type, gt);
        case 128: return pick<128>(k_type, gt);
        case 160: return pick<160>(k_type, gt);
        case 192: return pick<192>(k_type, gt);
        case 224: return pick<224>(k_type, gt);
        case 256: return pick<256>(k_type, gt);
        default: return nullptr;
    }
}

}  // namespace

hipError_t launch_score(const CacheView& cv, const Batch& b, int n_units, int k_type, int G,
                        int hd, const int32_t* coef, float* raw, PartRec* part, hipStream_t s) {
    int64_t max_n = 0;
    for (int i = 0; i < b.n_seq; ++i) max_n = b.seq[i].n > max_n ? b.seq[i].n : max_n;
    if (max_n <= 0 || n_units <= 0) return hipSuccess;
    // one moment tile per wavefront, kPartRows / 64 rows per lane
    const int64_t rows_per_block = (int64_t)(kScoreThreads / 64) * kPartRows;
    const int64_t tiles = (max_n + rows_per_block - 1) / rows_per_block;
    const dim3 grid((unsigned)tiles, (unsigned)n_units);
    const CoefGeom cg = coef_geom(k_type, hd, G);
    if (k_type == TRIA_KV_F16 && hd % 64 == 0) {
        switch (hd) {
            case 64: return run_f16_mfma<64>(cv, b, n_units, max_n, G, coef, cg.words, raw, part, s);
            case 128: return run_f16_mfma<128>(cv, b, n_units, max_n, G, coef, cg.words, raw, part, s);
            case 192: return run_f16_mfma<192>(cv, b, n_units, max_n, G, coef, cg.words, raw, part, s);
            case 256: return run_f16_mfma<256>(cv, b, n_units, max_n, G, coef, cg.words, raw, part, s);
            default: return hipErrorInvalidValue;
        }
    }
    for (int j0 = 0; j0 < G;) {
        const int gt = subgroup_size(G, j0);
        Runner fn = pick_runner(k_type, hd, gt);
        if (!fn) return hipErrorInvalidValue;
        fn(grid, s, cv, b, G, j0, coef, cg.words, raw, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        j0 += gt;
    }
    return hipSuccess;
}

}  // namespace tria
