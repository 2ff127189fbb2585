// select: GQA aggregation and top-budget selection, one workgroup per unit.
//
// llama.cpp page "TriAttention KV-Cache Eviction (--triattention)":
//   section 5 "Phase C": z-normalise each query head's scores on their own, then
//     the KV head's score is the max over its query heads;
//   section 5 "Phase B" steps 2-3: protect the first `sink` and last `window`
//     rows, sort the rest by score, evict the lowest down to the budget.
// The budget counts the protected rows ("TriAttention Native C++ Worklog":
// compaction logs keep exactly kv_budget rows).
//
// Per unit (1024 threads; thread t owns rows j*1024 + t, j < RPT):
//   1. head statistics: the per-tile moment partials (written by the scorer,
//      or by moments_kernel for caller-provided scores) are merged exactly in
//      fp64 into each head's mean and population variance over the rows with
//      a finite score;
//   2. one read of the raw scores, with the row's G scores in vector loads
//      and eight rows per thread in flight: agg(r) = max_h (s_h - mu_h) /
//      sigma_h in fp32 as ((s_h - mu_hi) - mu_lo) * (1/sigma_h), with mu_h held
//      as a two-float sum and 1/sigma_h rounded once from fp64, so the head's
//      common offset is removed before any rounding of the deviation (-inf if
//      any score is not finite),
//      mapped to an order-preserving 32-bit key (-0 folded into +0), and
//      counted into a 2048-bin histogram that is linear in agg over [-8, 8)
//      (clamped at both ends; the bin is a monotone function of the key);
//   3. the bin holding the k-th largest candidate comes from a suffix scan of
//      the histogram; that bin's keys (a few hundred for the synthetic
//      workloads) are gathered in LDS and the exact k-th largest key T and the
//      number of rows equal to T to take are found by counting.  A bin too
//      large for LDS (e.g. every score equal) falls back to an exact 4-pass
//      8-bit radix select over all candidate keys;
//   4. rows equal to T are taken lowest row first, and the kept rows are
//      written in ascending order: ranks in row order come from wave ballots
//      plus a prefix over the (j, wave) counts.
// Bins live in registers for n <= 128K rows (keys are recomputed from the raw
// scores for the few rows that need them), else keys go to a global scratch
// array.
#include "tria_group.h"

namespace tria {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kWaves = kSelThreads / 64;
constexpr int kBins = 2048;
constexpr float kBinLo = -8.0f;
constexpr float kBinScale = 128.0f;  // bins per unit of agg
constexpr int kListCap = 2048;
// rows per thread whose loads are in flight together (fewer for wide rows)
template <int GV>
constexpr int kBatchRows = GV >= 8 ? 2 : 8;
// Each row's histogram bin stays in registers up to 128 rows per thread
// (n <= 128K); wider units keep their keys in a global scratch array.
template <int RPT>
constexpr bool kBinsInRegs = RPT <= 128;
// Loops over a thread's rows are fully unrolled when its bins live in registers.
template <int RPT>
constexpr int kRowUnroll = kBinsInRegs<RPT> ? RPT : 4;

__device__ __forceinline__ uint32_t order_key(float x) {
    x = x + 0.0f;  // -0 -> +0 so that equal scores compare equal
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Histogram bin of an aggregated score: non-decreasing in x, -inf -> 0.
__device__ __forceinline__ int bin_of(float x) {
    float y = (x - kBinLo) * kBinScale;
    y = fminf(fmaxf(y, 0.0f), (float)(kBins - 1));
    return (int)y;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Exclusive prefix sum over the 1024 threads in thread order; *total = sum.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int s = sh[w];
        before += (w < wid) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// Add 1 to hist[digit] for every active lane; lanes sharing a digit add once.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t digit) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int round = 0; round < 3; ++round) {
        const uint64_t am = __ballot(active);
        if (am == 0) return;
        const int leader = __ffsll((unsigned long long)am) - 1;
        const uint32_t ld = __shfl(digit, leader, 64);
        const bool same = active && digit == ld;
        const uint64_t sm = __ballot(same);
        if (lane == leader) atomicAdd(&hist[ld], (uint32_t)__popcll(sm));
        active = active && !same;
    }
    if (active) atomicAdd(&hist[digit], 1u);
}

__device__ __forceinline__ int lane_rank(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// The G raw scores of row r -> aggregated score (GV: scores per vector load;
// 0 = scalar loads for any G).
template <int GV>
struct RowLoad {
    float4 v[GV == 0 ? 1 : (GV + 3) / 4];
};

// The raw scores are read once per pass (the few rows of the cutoff bin are
// read again): streaming (non-temporal) loads.  On MI355X this made the pass
// about 1 % faster, the gain showing in the compaction that follows.
template <int GV>
__device__ __forceinline__ void load_row(RowLoad<GV>& x, const float* R, int64_t r) {
    if constexpr (GV == 1) {
        x.v[0].x = __builtin_nontemporal_load(R + r);
    } else if constexpr (GV == 2) {
        typedef float f2e __attribute__((ext_vector_type(2)));
        const f2e t = __builtin_nontemporal_load(reinterpret_cast<const f2e*>(R + r * 2));
        x.v[0].x = t.x;
        x.v[0].y = t.y;
    } else if constexpr (GV >= 4) {
#pragma unroll
        for (int i = 0; i < GV / 4; ++i) {
            typedef float f4e __attribute__((ext_vector_type(4)));
            const f4e t = __builtin_nontemporal_load(reinterpret_cast<const f4e*>(R + r * GV) + i);
            x.v[i] = make_float4(t.x, t.y, t.z, t.w);
        }
    }
}

__device__ __forceinline__ float f4_get(const float4& v, int q) {
    return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

__device__ __forceinline__ float uniform_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

template <int GV>
struct Norms {
    HeadNorm h[GV == 0 ? 1 : GV];
    // GV > 0: the group's constants held in scalar registers
    __device__ __forceinline__ void load(const HeadNorm* sh) {
        if constexpr (GV > 0) {
#pragma unroll
            for (int i = 0; i < GV; ++i)
                h[i] = HeadNorm{uniform_f(sh[i].hi), uniform_f(sh[i].lo), uniform_f(sh[i].isg)};
        }
    }
};

template <int GV>
__device__ __forceinline__ float agg_of(const RowLoad<GV>& x, const float* R, int64_t r, int G,
                                        const Norms<GV>& nm, const HeadNorm* sh) {
    float best = -INFINITY;
    bool bad = false;
    if constexpr (GV == 0) {
        for (int h = 0; h < G; ++h) {
            const float s = R[r * G + h];
            if (!isfinite(s)) bad = true;
            const float z = znorm(s, sh[h]);
            best = (h == 0 || z > best) ? z : best;
        }
    } else {
#pragma unroll
        for (int h = 0; h < GV; ++h) {
            const float s = f4_get(x.v[h >> 2], h & 3);
            if (!isfinite(s)) bad = true;
            const float z = znorm(s, nm.h[h]);
            best = (h == 0 || z > best) ? z : best;
        }
    }
    return bad ? -INFINITY : best + 0.0f;
}

// Up to 32K rows the kernel fits 64 registers, so two 1024-thread workgroups
// share a CU and 512 units are selected at once; up to 128K rows the bins take
// up to 64 more registers (one workgroup per CU).
template <int RPT>
constexpr int kSelWavesPerEU = RPT <= 32 ? 8 : 4;

template <int RPT, int GV>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(kSelWavesPerEU<RPT>))) void select_kernel(
    Batch b, int units_per_seq, int G, const float* __restrict__ raw,
    const PartRec* __restrict__ part, int32_t* __restrict__ keep, float* __restrict__ agg_out,
    uint32_t* __restrict__ key_scratch, int32_t* __restrict__ chunk_pb, uint32_t* ticket) {
    constexpr bool kRegKeys = kBinsInRegs<RPT>;
    // the compaction that follows on this stream takes its tasks from ticket[0]
    if (ticket && blockIdx.x == 0 && threadIdx.x == 0) reset_ticket(ticket);
    const int u = blockIdx.x;
    const int seq = u / units_per_seq;
    const int uu = u - seq * units_per_seq;
    // Everything the kernel needs from the sequence's descriptor is taken here,
    // as 32-bit values where they fit (at most 1024 * 256 rows per unit): the
    // descriptor itself is not kept live in scalar registers through the
    // unrolled loops below.
    int n, kept, cand_lo, n_cand;
    const float* __restrict__ R;
    int32_t* __restrict__ KI;
    float* AG;
    uint32_t* KS;
    const PartRec* __restrict__ P;
    int32_t* PB;
    int nb = 0;
    int64_t tiles;
    {
        const SeqDesc& sd = b.seq[seq];
        n = (int)sd.n;
        if (n <= 0) return;
        kept = (int)sd.kept;
        // candidates: rows [s_end, w_start) (all below n)
        cand_lo = (int)sd.s_end;
        n_cand = (int)(sd.w_start - sd.s_end);
        R = raw + sd.raw_off + (int64_t)uu * n * G;
        KI = keep + sd.keep_off + (int64_t)uu * kept;
        AG = agg_out ? agg_out + sd.raw_off / G + (int64_t)uu * n : nullptr;
        KS = kRegKeys ? nullptr : key_scratch + sd.raw_off / G + (int64_t)uu * n;
        tiles = part_tiles(n);
        P = part ? part + (sd.part_off + (int64_t)uu * tiles) * G : nullptr;
        if (chunk_pb) nb = (int)chunk_bounds(kept);
        PB = chunk_pb ? chunk_pb + sd.pb_off + (int64_t)uu * nb : nullptr;
    }

    __shared__ HeadNorm norm_sh[64];
    __shared__ uint32_t hist[kBins + 64];  // + one spare bin per lane, never read
    __shared__ uint32_t list[kListCap];
    __shared__ uint32_t rhist[kWaves][256];
    __shared__ uint32_t tot[256];
    __shared__ int scan_sh[kWaves];
    __shared__ int found_sh[4];
    __shared__ int cnt_sh[RPT * kWaves];

    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    auto row_of = [&](int j) -> int { return j * kSelThreads + t; };

    // 1. head statistics from the tile partials: wavefront w merges heads
    //    w, w + 16, ...  Without partials the scores are used as they are
    //    (identity norms: a shared keep set's group scores).
    for (int h = wid; h < G; h += kWaves) {
        const HeadNorm hn = part ? merge_head_norm(P, tiles, G, h) : HeadNorm{0.0f, 0.0f, 1.0f};
        if (lane == 0) norm_sh[h] = hn;
    }
    for (int i = t; i < kBins + 64; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    Norms<GV> nrm;
    nrm.load(norm_sh);

    // 2. aggregated score -> key, histogram of the candidates
    auto is_cand = [&](int r) -> bool { return (unsigned)(r - cand_lo) < (unsigned)n_cand; };
    // kRegKeys: each row's histogram bin stays in registers (two per word) and
    // the full key is recomputed from the raw scores for the few rows that
    // need it (those in the cutoff bin); otherwise keys go to global scratch.
    uint32_t binw[kRegKeys ? (RPT + 1) / 2 : 1];
#pragma unroll
    for (int i = 0; i < (kRegKeys ? (RPT + 1) / 2 : 1); ++i) binw[i] = 0;
    constexpr int kBatch = kBatchRows<GV>;
    constexpr int kNB = (RPT + kBatch - 1) / kBatch;
    constexpr int kUB = kRegKeys ? kNB : 1;
    // Two copies of this loop: one for units whose every owned row exists (and
    // no aggregate output), with no branch per row (rows that are not
    // candidates count into a spare bin of their lane's own), and one for the
    // rest.  The row count and the candidate range are re-read through empty
    // asm statements and each packed bin word is fixed once written, so that
    // the compiler keeps neither these per-row conditions nor every row's bin
    // in registers of their own for the later phases.
    auto histogram = [&](auto all_rows) {
        constexpr bool kAll = decltype(all_rows)::value;
        int n2 = n, clo = cand_lo;
        asm volatile("" : "+s"(n2), "+s"(clo));
#pragma unroll kUB
        for (int j0 = 0; j0 < RPT; j0 += kBatch) {
            RowLoad<GV> x[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int r = row_of(j0 + q);
                if (j0 + q < RPT && (kAll || r < n2)) load_row<GV>(x[q], R, r);
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int j = j0 + q;
                if (j >= RPT) break;
                const int r = row_of(j);
                if (kAll || r < n2) {
                    const float a = agg_of<GV>(x[q], R, r, G, nrm, norm_sh);
                    if (!kAll && AG) AG[r] = a;
                    const int bn = bin_of(a);
                    const bool cand = (unsigned)(r - clo) < (unsigned)n_cand;
                    if constexpr (kAll) atomicAdd(&hist[cand ? bn : kBins + lane], 1u);
                    else if (cand) atomicAdd(&hist[bn], 1u);
                    if constexpr (kRegKeys) {
                        binw[j >> 1] |= (uint32_t)bn << (16 * (j & 1));
                        if ((j & 1) || j + 1 == RPT) asm volatile("" : "+v"(binw[j >> 1]));
                    } else {
                        KS[r] = order_key(a);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (!AG && n >= RPT * kSelThreads) histogram(std::true_type{});
    else histogram(std::false_type{});
    __syncthreads();
    // the key of row r recomputed exactly as above
    auto key_at = [&](int r) -> uint32_t {
        RowLoad<GV> x;
        load_row<GV>(x, R, r);
        return order_key(agg_of<GV>(x, R, r, G, nrm, norm_sh));
    };
    auto get_key = [&](int j) -> uint32_t {
        const int r = row_of(j);
        if (r >= n) return 0u;
        if constexpr (kRegKeys) return key_at(r);
        else return KS[r];
    };
    auto bin_j = [&](int j) -> int {
        if constexpr (kRegKeys) return (int)((binw[j >> 1] >> (16 * (j & 1))) & 0xffffu);
        else return bin_of(key_value(get_key(j)));
    };

    // 3. threshold: the k-th largest candidate key T; krem rows equal to T are taken
    const int k_take = kept - (n - n_cand);
    const bool radix = k_take > 0 && k_take < n_cand;
    const bool take_all = k_take >= n_cand;
    uint32_t T = 0;
    int krem = 0, bstar = -1;
    bool rank_ties = false;
    constexpr int kMW = (RPT + 31) / 32;
    uint32_t cutw[kMW];
#pragma unroll
    for (int q = 0; q < kMW; ++q) cutw[q] = 0;
    if (radix) {
        // bins from the top: thread t holds bins kBins-1-2t and kBins-2-2t
        const int b0 = kBins - 1 - 2 * t, b1 = b0 - 1;
        const int c0 = t < kBins / 2 ? (int)hist[b0] : 0;
        const int c1 = t < kBins / 2 ? (int)hist[b1] : 0;
        int total;
        const int above = block_excl_scan(c0 + c1, scan_sh, &total);
        const int k = (int)k_take;
        if (t < kBins / 2) {
            if (above < k && above + c0 >= k) {
                found_sh[0] = b0;
                found_sh[1] = k - above;
            } else if (above + c0 < k && above + c0 + c1 >= k) {
                found_sh[0] = b1;
                found_sh[1] = k - above - c0;
            }
        }
        if (t == 0) found_sh[2] = 0;
        __syncthreads();
        bstar = found_sh[0];
        const int kb = found_sh[1];
        const int cb = (int)hist[bstar];
        // the candidates in the cutoff bin, one bit per owned row
#pragma unroll kRowUnroll<RPT>
        for (int j = 0; j < RPT; ++j)
            if (is_cand(row_of(j)) && bin_j(j) == bstar) cutw[j >> 5] |= 1u << (j & 31);
        if (cb <= kListCap) {
            // the bin's keys into LDS, then the kb-th largest by counting
            for (int w = 0; w < kMW; ++w)
                for (uint32_t m = cutw[w]; m; m &= m - 1)
                    list[atomicAdd(&found_sh[2], 1)] = get_key(w * 32 + __ffs(m) - 1);
            __syncthreads();
            for (int i = t; i < cb; i += kSelThreads) {
                const uint32_t ki = list[i];
                int g = 0, e = 0;
                for (int q = 0; q < cb; ++q) {
                    const uint32_t kq = list[q];
                    g += kq > ki;
                    e += kq == ki;
                }
                if (g < kb && kb <= g + e) {  // every thread holding T writes the same values
                    found_sh[0] = (int)ki;
                    found_sh[1] = kb - g;
                    found_sh[3] = e;
                }
            }
            __syncthreads();
            T = (uint32_t)found_sh[0];
            krem = found_sh[1];
            rank_ties = found_sh[3] > krem;
            __syncthreads();
        } else {
            // exact radix select over every candidate key
            uint32_t prefix = 0, mask = 0;
            krem = k;
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                for (int i = lane; i < 256; i += 64) rhist[wid][i] = 0;
                __syncthreads();
                // (rare: a cutoff bin too large for LDS) keys recomputed per pass
#pragma unroll 1
                for (int j = 0; j < RPT; ++j) {
                    const int r = row_of(j);
                    const bool c = is_cand(r);
                    const uint32_t kk = c ? get_key(j) : 0u;
                    const bool act = c && ((kk & mask) == prefix);
                    hist_add(rhist[wid], act, (kk >> shift) & 255u);
                }
                __syncthreads();
                if (t < 256) {
                    uint32_t s = 0;
#pragma unroll
                    for (int w = 0; w < kWaves; ++w) s += rhist[w][t];
                    tot[t] = s;
                }
                __syncthreads();
                if (wid == 0) {
                    // lane l holds bins 4l..4l+3; count of keys in bins above this lane's
                    const uint32_t e0 = tot[4 * lane], e1 = tot[4 * lane + 1],
                                   e2 = tot[4 * lane + 2], e3 = tot[4 * lane + 3];
                    const uint32_t mine = e0 + e1 + e2 + e3;
                    uint32_t incl = mine;  // inclusive suffix sum over lanes >= lane
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const uint32_t y = __shfl_down(incl, o, 64);
                        if (lane + o < 64) incl += y;
                    }
                    uint32_t ab = incl - mine;
                    const uint32_t cs[4] = {e0, e1, e2, e3};
#pragma unroll
                    for (int q = 3; q >= 0; --q) {
                        if (ab < (uint32_t)krem && ab + cs[q] >= (uint32_t)krem) {
                            found_sh[0] = 4 * lane + q;
                            found_sh[1] = krem - (int)ab;
                        }
                        ab += cs[q];
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)found_sh[0] << shift;
                mask |= 255u << shift;
                krem = found_sh[1];
                __syncthreads();
            }
            T = prefix;
            rank_ties = true;
        }
    }

    // 4. ties at T go to the lowest rows; then write kept rows in order.
    // Row order is (j, wave, lane); ranks = prefix over the (j, wave) counts
    // plus the lane's rank within its wave's ballot.
    // Row j * 1024 + t of this thread is bit j % 32 of word j / 32 of a flag
    // array.  The words are walked with fixed indices and the bits with a loop
    // counter, so each ballot's lane mask is formed right before its use
    // (formed all at once, 32 masks of 64 bits spill the scalar registers).
    auto ordered_ranks = [&](const uint32_t(&bits)[kMW], auto use_rank) {
#pragma unroll
        for (int w = 0; w < kMW; ++w) {
            const uint32_t bw = bits[w];
            const int jn = RPT - 32 * w < 32 ? RPT - 32 * w : 32;
#pragma unroll 4
            for (int jj = 0; jj < jn; ++jj) {
                const uint64_t m = __ballot((bw >> jj) & 1u);
                if (lane == 0) cnt_sh[(32 * w + jj) * kWaves + wid] = __popcll(m);
            }
        }
        __syncthreads();
        constexpr int kPer = (RPT * kWaves + kSelThreads - 1) / kSelThreads;
        int loc[kPer], sum = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = kPer * t + q;
            loc[q] = sum;
            sum += e < RPT * kWaves ? cnt_sh[e] : 0;
        }
        int total;
        const int base = block_excl_scan(sum, scan_sh, &total);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = kPer * t + q;
            if (e < RPT * kWaves) cnt_sh[e] = base + loc[q];
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kMW; ++w) {
            const uint32_t bw = bits[w];
            const int jn = RPT - 32 * w < 32 ? RPT - 32 * w : 32;
#pragma unroll 4
            for (int jj = 0; jj < jn; ++jj) {
                const bool f = ((bw >> jj) & 1u) != 0;
                const uint64_t m = __ballot(f);
                if (f) use_rank(w, jj, cnt_sh[(32 * w + jj) * kWaves + wid] + lane_rank(m));
            }
        }
        __syncthreads();
    };
    // keep decision bits, one per owned row; tie bits for rows equal to T
    uint32_t kbits[kMW], tiew[kMW];
#pragma unroll
    for (int q = 0; q < kMW; ++q) kbits[q] = tiew[q] = 0;
    auto set_keep = [&](int j) { kbits[j >> 5] |= 1u << (j & 31); };
#pragma unroll kRowUnroll<RPT>
    for (int j = 0; j < RPT; ++j) {
        const int r = row_of(j);
        if (r >= n) continue;
        // bins are monotone in the key: above the cutoff bin means above T
        if (!is_cand(r) || take_all || (radix && bin_j(j) > bstar)) set_keep(j);
    }
    if (radix) {
        // rows of the cutoff bin compare their keys with T
        for (int w = 0; w < kMW; ++w)
            for (uint32_t m = cutw[w]; m; m &= m - 1) {
                const int j = w * 32 + __ffs(m) - 1;
                const uint32_t kk = get_key(j);
                if (kk > T || (kk == T && !rank_ties)) kbits[w] |= 1u << (j & 31);
                else if (kk == T) tiew[w] |= 1u << (j & 31);
            }
    }
    if (rank_ties) {
        ordered_ranks(tiew, [&](int w, int jj, int rank) {
            if (rank < krem) kbits[w] |= 1u << jj;
        });
    }
    ordered_ranks(kbits, [&](int w, int jj, int rank) {
        if (rank < kept) KI[rank] = (int32_t)row_of(32 * w + jj);
    });
    // The scan's prefix at (j, wave) is the number of kept rows below row
    // 64 (16 j + wave): write it at the compaction's chunk boundaries.
    if (PB) {
        for (int e = t; e < nb; e += kSelThreads) PB[e] = e < RPT * kWaves ? cnt_sh[e] : kept;
    }
}

// Moment partials of caller-provided raw scores (the scorer writes them
// itself during a whole pass): one wavefront per tile of kPartRows rows.
constexpr int kMomThreads = 256;
__global__ __launch_bounds__(kMomThreads) void moments_kernel(Batch b, int units_per_seq, int G,
                                                              const float* __restrict__ raw,
                                                              PartRec* __restrict__ part) {
    const int u = blockIdx.y;
    const int seq = u / units_per_seq;
    const int uu = u - seq * units_per_seq;
    const SeqDesc sd = b.seq[seq];
    const int64_t n = sd.n;
    const int64_t tile = (int64_t)blockIdx.x * (kMomThreads / 64) + (threadIdx.x >> 6);
    if (tile * kPartRows >= n) return;  // whole wavefront past the end
    const float* __restrict__ R = raw + sd.raw_off + (int64_t)uu * n * G;
    PartRec* out = part + (sd.part_off + (int64_t)uu * part_tiles(n) + tile) * G;
    for (int h0 = 0; h0 < G; h0 += 4) {
        WaveMoments<4> mom;
        for (int i = 0; i < kPartLaneRows; ++i) {
            const int64_t r = tile * kPartRows + i * 64 + (threadIdx.x & 63);
            float s[4];
            bool v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s[q] = (r < n && h0 + q < G) ? R[r * G + h0 + q] : 0.0f;
                v[q] = r < n && h0 + q < G && isfinite(s[q]);
            }
            mom.add(s, v);
        }
        mom.emit(out + h0, G - h0 < 4 ? G - h0 : 4);
    }
}

template <int RPT, int GV>
void run_sel(int grid, hipStream_t s, const Batch& b, int ups, int G, const float* raw,
             const PartRec* part, int32_t* keep, float* agg, uint32_t* ks, int32_t* pb,
             uint32_t* ticket) {
    hipLaunchKernelGGL((select_kernel<RPT, GV>), dim3(grid), dim3(kSelThreads), 0, s, b, ups, G,
                       raw, part, keep, agg, ks, pb, ticket);
}

using SelRunner = void (*)(int, hipStream_t, const Batch&, int, int, const float*,
                           const PartRec*, int32_t*, float*, uint32_t*, int32_t*, uint32_t*);

template <int RPT>
SelRunner pick_gv(int G) {
    switch (G) {
        case 1: return run_sel<RPT, 1>;
        case 2: return run_sel<RPT, 2>;
        case 4: return run_sel<RPT, 4>;
        case 8: return run_sel<RPT, 8>;
        default: return run_sel<RPT, 0>;
    }
}

}  // namespace

// Rows a key-scratch array must hold for a batch (0 when keys stay in registers).
// Unit uu of sequence i uses rows raw_off/G + uu*n .. + n of the array, so the
// size is the largest such end (the batch may describe a group of layers whose
// offsets start past zero).
int64_t select_key_scratch_rows(const Batch& b, int units_per_seq, int G) {
    int64_t max_n = 0, end = 0;
    for (int i = 0; i < b.n_seq; ++i) {
        const SeqDesc& sd = b.seq[i];
        max_n = sd.n > max_n ? sd.n : max_n;
        const int64_t e = sd.raw_off / G + (int64_t)units_per_seq * sd.n;
        end = e > end ? e : end;
    }
    return max_n > 128 * kSelThreads ? end : 0;
}

hipError_t launch_moments(const Batch& b, int units_per_seq, int G, const float* raw,
                          PartRec* part, hipStream_t s) {
    int64_t max_n = 0;
    for (int i = 0; i < b.n_seq; ++i) max_n = b.seq[i].n > max_n ? b.seq[i].n : max_n;
    if (max_n <= 0) return hipSuccess;
    const int64_t rows_per_block = (int64_t)(kMomThreads / 64) * kPartRows;
    const dim3 grid((unsigned)((max_n + rows_per_block - 1) / rows_per_block),
                    (unsigned)(units_per_seq * b.n_seq));
    hipLaunchKernelGGL(moments_kernel, grid, dim3(kMomThreads), 0, s, b, units_per_seq, G, raw,
                       part);
    return hipGetLastError();
}

hipError_t launch_select_impl(const Batch& b, int units_per_seq, int G, const float* raw,
                              const PartRec* part, int32_t* keep, float* agg,
                              uint32_t* key_scratch, int32_t* chunk_pb, uint32_t* ticket,
                              hipStream_t s) {
    int64_t max_n = 0;
    for (int i = 0; i < b.n_seq; ++i) max_n = b.seq[i].n > max_n ? b.seq[i].n : max_n;
    if (max_n <= 0) return hipSuccess;
    const int grid = units_per_seq * b.n_seq;
    const int64_t rpt = (max_n + kSelThreads - 1) / kSelThreads;
    SelRunner fn;
    if (rpt <= 1) fn = pick_gv<1>(G);
    else if (rpt <= 2) fn = pick_gv<2>(G);
    else if (rpt <= 4) fn = pick_gv<4>(G);
    else if (rpt <= 8) fn = pick_gv<8>(G);
    else if (rpt <= 16) fn = pick_gv<16>(G);
    else if (rpt <= 32) fn = pick_gv<32>(G);
    else if (rpt <= 64) fn = pick_gv<64>(G);
    else if (rpt <= 128) fn = pick_gv<128>(G);
    else if (rpt <= 256) fn = pick_gv<256>(G);
    else return hipErrorInvalidValue;
    fn(grid, s, b, units_per_seq, G, raw, part, keep, agg, key_scratch, chunk_pb, ticket);
    return hipGetLastError();
}

}  // namespace tria
