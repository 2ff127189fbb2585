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
// Per unit (1024 threads; thread t owns rows j*1024 + t, j < RPT, so every
// load of the raw scores is coalesced):
//   1. moments of every head over the rows with a finite score (fp64 sums of
//      values shifted by the head's first score, against cancellation);
//   2. agg(r) = max_h (s_h - mu_h)/sigma_h in fp64, rounded once to fp32,
//      -inf if any of the row's scores is not finite; mapped to an
//      order-preserving 32-bit key (-0 folded into +0);
//   3. exact k-th-largest key among the candidates by four 8-bit radix passes
//      over LDS histograms (one per wave; lanes that share a digit add once);
//   4. ties at the threshold go to the lowest row indices, and the kept rows
//      are written in ascending order: ranks in row order come from wave
//      ballots plus a prefix over the (j, wave) counts.
// Keys live in registers for n <= 8K rows, in LDS for n <= 32K, else in a
// global scratch array.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kWaves = kSelThreads / 64;
constexpr int kHeadChunk = 4;

__device__ __forceinline__ uint32_t order_key(float x) {
    x = x + 0.0f;  // -0 -> +0 so that equal scores compare equal
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
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

template <int RPT, int KM>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    Batch b, int units_per_seq, int G, const float* __restrict__ raw, int32_t* __restrict__ keep,
    float* __restrict__ agg_out, uint32_t* __restrict__ key_scratch) {
    const int u = blockIdx.x;
    const int seq = u / units_per_seq;
    const int uu = u - seq * units_per_seq;
    const SeqDesc sd = b.seq[seq];
    const int64_t n = sd.n;
    if (n <= 0) return;
    const float* __restrict__ R = raw + sd.raw_off + (int64_t)uu * n * G;
    int32_t* __restrict__ KI = keep + sd.keep_off + (int64_t)uu * sd.kept;
    float* AG = agg_out ? agg_out + (int64_t)uu * n : nullptr;
    // KM: where the keys live -- 0 registers, 1 LDS, 2 global scratch
    constexpr bool kGmemKeys = KM == 2;
    uint32_t* KS = kGmemKeys ? key_scratch + sd.raw_off / G + (int64_t)uu * n : nullptr;
    __shared__ uint32_t key_lds[KM == 1 ? RPT * kSelThreads : 1];

    __shared__ double red[kWaves][kHeadChunk][2];
    __shared__ int redc[kWaves][kHeadChunk];
    __shared__ double mu_sh[64], isg_sh[64];
    __shared__ uint32_t hist[kWaves][256];
    __shared__ uint32_t tot[256];
    __shared__ int scan_sh[kWaves];
    __shared__ int found_sh[2];
    __shared__ int cnt_sh[RPT * kWaves];

    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    auto row_of = [&](int j) -> int64_t { return (int64_t)j * kSelThreads + t; };
    // loops over owned rows are fully unrolled when keys live in registers

    // 1. moments per head (rows strided by 1024 for coalesced reads)
    for (int h0 = 0; h0 < G; h0 += kHeadChunk) {
        double shift[kHeadChunk], sum[kHeadChunk], sq[kHeadChunk];
        int cnt[kHeadChunk];
#pragma unroll
        for (int q = 0; q < kHeadChunk; ++q) {
            const float s0 = (h0 + q < G) ? R[h0 + q] : 0.0f;
            shift[q] = isfinite(s0) ? (double)s0 : 0.0;
            sum[q] = 0.0;
            sq[q] = 0.0;
            cnt[q] = 0;
        }
        for (int64_t r = t; r < n; r += kSelThreads) {
#pragma unroll
            for (int q = 0; q < kHeadChunk; ++q) {
                if (h0 + q < G) {
                    const float s = R[r * G + h0 + q];
                    if (isfinite(s)) {
                        const double d = (double)s - shift[q];
                        sum[q] += d;
                        sq[q] = fma(d, d, sq[q]);
                        cnt[q] += 1;
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kHeadChunk; ++q) {
            const double a = wave_sum(sum[q]), c = wave_sum(sq[q]);
            const int k = wave_sum_i(cnt[q]);
            if (lane == 0) {
                red[wid][q][0] = a;
                red[wid][q][1] = c;
                redc[wid][q] = k;
            }
        }
        __syncthreads();
        if (t < kHeadChunk && h0 + t < G) {
            double a = 0.0, c = 0.0;
            long long k = 0;
            for (int w = 0; w < kWaves; ++w) {
                a += red[w][t][0];
                c += red[w][t][1];
                k += redc[w][t];
            }
            double mu = 0.0, isg = 0.0;
            if (k > 0) {
                const float s0 = R[h0 + t];
                const double m = a / (double)k;
                double var = c / (double)k - m * m;
                var = var > 0.0 ? var : 0.0;
                mu = (isfinite(s0) ? (double)s0 : 0.0) + m;
                const double sg = sqrt(var);
                isg = sg > 0.0 ? 1.0 / sg : 0.0;
            }
            mu_sh[h0 + t] = mu;
            isg_sh[h0 + t] = isg;
        }
        __syncthreads();
    }

    // 2. aggregated score -> order-preserving key
    const int64_t cand_lo = sd.s_end, cand_hi = sd.w_start;
    uint32_t key[KM == 0 ? RPT : 1];
#pragma unroll (KM == 0 ? RPT : 4)
    for (int j = 0; j < RPT; ++j) {
        const int64_t r = row_of(j);
        if (r < n) {
            double best = -INFINITY;
            bool bad = false;
            for (int h = 0; h < G; ++h) {
                const float s = R[r * G + h];
                if (!isfinite(s)) bad = true;
                const double z = ((double)s - mu_sh[h]) * isg_sh[h];
                best = (h == 0 || z > best) ? z : best;
            }
            const float a = bad ? -INFINITY : (float)best;
            if (AG) AG[r] = a;
            const uint32_t kk = order_key(a);
            if constexpr (KM == 2) KS[r] = kk;
            else if constexpr (KM == 1) key_lds[j * kSelThreads + t] = kk;
            else key[j] = kk;
        } else {
            if constexpr (KM == 1) key_lds[j * kSelThreads + t] = 0;
            else if constexpr (KM == 0) key[j] = 0;
        }
    }
    auto get_key = [&](int j) -> uint32_t {
        if constexpr (KM == 2) return KS[row_of(j)];
        else if constexpr (KM == 1) return key_lds[j * kSelThreads + t];
        else return key[j];
    };
    auto is_cand = [&](int64_t r) -> bool { return r >= cand_lo && r < cand_hi; };

    // 3. threshold: the k-th largest candidate key
    const int64_t n_cand = cand_hi - cand_lo;
    const int64_t k_take = sd.kept - (n - n_cand);
    const bool take_none = k_take <= 0;
    const bool take_all = k_take >= n_cand;
    uint32_t prefix = 0, mask = 0;
    int krem = (int)k_take;
    if (!take_none && !take_all) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int i = lane; i < 256; i += 64) hist[wid][i] = 0;
            __syncthreads();
#pragma unroll (KM == 0 ? RPT : 4)
            for (int j = 0; j < RPT; ++j) {
                const int64_t r = row_of(j);
                const uint32_t kk = get_key(j);
                const bool act = r < n && is_cand(r) && ((kk & mask) == prefix);
                hist_add(hist[wid], act, (kk >> shift) & 255u);
            }
            __syncthreads();
            if (t < 256) {
                uint32_t s = 0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) s += hist[w][t];
                tot[t] = s;
            }
            __syncthreads();
            if (wid == 0) {
                // lane l holds bins 4l..4l+3; count of keys in bins above this lane's
                const uint32_t c0 = tot[4 * lane], c1 = tot[4 * lane + 1], c2 = tot[4 * lane + 2],
                               c3 = tot[4 * lane + 3];
                const uint32_t mine = c0 + c1 + c2 + c3;
                uint32_t incl = mine;  // inclusive suffix sum over lanes >= lane
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t y = __shfl_down(incl, o, 64);
                    if (lane + o < 64) incl += y;
                }
                uint32_t above = incl - mine;
                const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
                for (int q = 3; q >= 0; --q) {
                    if (above < (uint32_t)krem && above + cs[q] >= (uint32_t)krem) {
                        found_sh[0] = 4 * lane + q;
                        found_sh[1] = krem - (int)above;
                    }
                    above += cs[q];
                }
            }
            __syncthreads();
            prefix |= (uint32_t)found_sh[0] << shift;
            mask |= 255u << shift;
            krem = found_sh[1];
            __syncthreads();
        }
    }
    const uint32_t T = prefix;

    // 4. ties at T go to the lowest rows; then write kept rows in order.
    // Row order is (j, wave, lane); ranks = prefix over the (j, wave) counts
    // plus the lane's rank within its wave's ballot.
    const bool radix = !take_none && !take_all;
    auto ordered_ranks = [&](auto flag_of, auto use_rank) {
#pragma unroll (KM == 0 ? RPT : 4)
        for (int j = 0; j < RPT; ++j) {
            const uint64_t m = __ballot(flag_of(j));
            if (lane == 0) cnt_sh[j * kWaves + wid] = __popcll(m);
        }
        __syncthreads();
        int loc[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * t + q;
            loc[q] = sum;
            sum += e < RPT * kWaves ? cnt_sh[e] : 0;
        }
        int total;
        const int base = block_excl_scan(sum, scan_sh, &total);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * t + q;
            if (e < RPT * kWaves) cnt_sh[e] = base + loc[q];
        }
        __syncthreads();
#pragma unroll (KM == 0 ? RPT : 4)
        for (int j = 0; j < RPT; ++j) {
            const bool f = flag_of(j);
            const uint64_t m = __ballot(f);
            if (f) use_rank(j, cnt_sh[j * kWaves + wid] + lane_rank(m));
        }
        __syncthreads();
    };
    // keep decision bits, one per owned row
    uint32_t kbits[(RPT + 31) / 32];
#pragma unroll
    for (int q = 0; q < (RPT + 31) / 32; ++q) kbits[q] = 0;
    auto set_keep = [&](int j) { kbits[j >> 5] |= 1u << (j & 31); };
#pragma unroll (KM == 0 ? RPT : 4)
    for (int j = 0; j < RPT; ++j) {
        const int64_t r = row_of(j);
        if (r >= n) continue;
        if (!is_cand(r) || take_all) {
            set_keep(j);
        } else if (radix && get_key(j) > T) {
            set_keep(j);
        }
    }
    if (radix) {
        ordered_ranks(
            [&](int j) {
                const int64_t r = row_of(j);
                return r < n && is_cand(r) && get_key(j) == T;
            },
            [&](int j, int rank) {
                if (rank < krem) set_keep(j);
            });
    }
    ordered_ranks([&](int j) { return ((kbits[j >> 5] >> (j & 31)) & 1u) != 0; },
                  [&](int j, int rank) {
                      if (rank < sd.kept) KI[rank] = (int32_t)row_of(j);
                  });
}

template <int RPT, int KM>
void run_sel(int grid, hipStream_t s, const Batch& b, int ups, int G, const float* raw,
             int32_t* keep, float* agg, uint32_t* ks) {
    hipLaunchKernelGGL((select_kernel<RPT, KM>), dim3(grid), dim3(kSelThreads), 0, s, b, ups, G,
                       raw, keep, agg, ks);
}

}  // namespace

// Rows a key-scratch array must hold for a batch (0 when keys stay on chip).
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
    return max_n > 32 * kSelThreads ? end : 0;
}

hipError_t launch_select_impl(const Batch& b, int units_per_seq, int G, const float* raw,
                              int32_t* keep, float* agg, uint32_t* key_scratch, hipStream_t s) {
    int64_t max_n = 0;
    for (int i = 0; i < b.n_seq; ++i) max_n = b.seq[i].n > max_n ? b.seq[i].n : max_n;
    if (max_n <= 0) return hipSuccess;
    const int grid = units_per_seq * b.n_seq;
    const int64_t rpt = (max_n + kSelThreads - 1) / kSelThreads;
    if (rpt <= 1) run_sel<1, 0>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 2) run_sel<2, 0>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 4) run_sel<4, 0>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 8) run_sel<8, 0>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 16) run_sel<16, 1>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 32) run_sel<32, 1>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 64) run_sel<64, 2>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 128) run_sel<128, 2>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else if (rpt <= 256) run_sel<256, 2>(grid, s, b, units_per_seq, G, raw, keep, agg, key_scratch);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tria
