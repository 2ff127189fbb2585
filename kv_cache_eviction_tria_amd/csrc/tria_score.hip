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
// Mapping: one lane per cached row at a time; a wavefront scores a tile of 256
// rows (four per lane), 1024 rows per workgroup.  Every lane of a wave needs
// the same coefficient at the same time, so the unit's table (built by prep) is read through scalar
// loads into SGPRs and fed to the VALU as the scalar operand; no LDS and no
// cross-lane reduction.  Each lane reads its whole row with wide loads; one
// load instruction touches a cache line per lane and the following loads of
// the row hit the same lines in L1, so K crosses HBM once.  The sqrt of
// |K_f|^2 is shared by all G heads.
//
// q8_0 rows: the trig part is an integer dot product per 32-value block:
// sum_d q_d c_d = sig * sum_d q_d v_d with v the 16-bit quantised coefficient
// split into two base-256 digits, accumulated with packed int8 dot products
// (v_dot4_i32_i8) straight from the stored bytes (the digit tables follow the
// row's byte layout, scale bytes carry zero digits); the block scale d and sig
// are applied once per block.  The |K_f| term dequantises q * d in fp32.
//
// Each wavefront also summarises its rows' scores per head (count, mean,
// squared deviations; fp64) for the selector's z-normalisation, so the raw
// scores are not read an extra time to form the head statistics.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kScoreThreads = 256;

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

template <int GT>
__device__ __forceinline__ void store_scores(float* dst, const float (&acc)[GT], bool packed) {
    if (packed) {
        if constexpr (GT == 1) {
            dst[0] = acc[0];
        } else if constexpr (GT == 2) {
            *reinterpret_cast<float2*>(dst) = make_float2(acc[0], acc[1]);
        } else if constexpr (GT == 4) {
            *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
            *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < GT; ++j) dst[j] = acc[j];
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

template <int HD, int GT>
__global__ __launch_bounds__(kScoreThreads) void score_q8_kernel(
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
    const int64_t wbase = wave_tile() * kPartRows;
    if (wbase >= n) return;
    const CoefGeom cg = coef_geom(TRIA_KV_Q8_0, HD, G);
    const int32_t* __restrict__ T = coef + coef_unit(b, cv, id) * coef_words;
    const int32_t* __restrict__ HI = T + cg.hi_off + j0 * W;
    const int32_t* __restrict__ LO = T + cg.lo_off + j0 * W;
    const float* __restrict__ SIG = reinterpret_cast<const float*>(T + cg.sig_off) + j0 * NB;
    const float* __restrict__ WT = reinterpret_cast<const float*>(T + cg.w_off) + j0 * F;
    float* rout = raw + b.seq[id.seq].raw_off + ((int64_t)id.l * cv.Hkv + id.g) * n * G + j0;
    const bool packed = (G == GT);
    WaveMoments<GT> mom;

#pragma unroll 1
    for (int it = 0; it < kPartLaneRows; ++it) {
        const int64_t r0 = wbase + it * 64;
        if (r0 >= n) break;
        const int64_t r_out = r0 + (threadIdx.x & 63);
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
        // quantised coefficient digits, then one scale per (head, block)
#pragma unroll
        for (int bk = 0; bk < NB; ++bk) {
            sync_acc<GT>(acc);
            const int k0 = (34 * bk + 2) >> 2, k1 = (34 * bk + 33) >> 2;
#pragma unroll
            for (int j = 0; j < GT; ++j) {
                int hi = 0, lo = 0;
#pragma unroll
                for (int k = k0; k <= k1; ++k) {
                    hi = __builtin_amdgcn_sdot4((int)wv[k], HI[z + j * W + k], hi, false);
                    lo = __builtin_amdgcn_sdot4((int)wv[k], LO[z + j * W + k], lo, false);
                }
                acc[j] = fmaf((float)(hi * 256 + lo), dsc[bk] * SIG[z + j * NB + bk], acc[j]);
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
        if (r_out < n) store_scores<GT>(rout + r_out * G, acc, packed);
        if (part) add_moments<GT>(mom, acc, r_out < n);
    }
    if (part) emit_moments<GT>(mom, b.seq[id.seq], id, cv.Hkv, n, G, j0, part);
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
    hipLaunchKernelGGL((score_q8_kernel<HD, GT>), grid, dim3(kScoreThreads), 0, s, cv, b, G, j0,
                       coef, words, raw, part);
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
