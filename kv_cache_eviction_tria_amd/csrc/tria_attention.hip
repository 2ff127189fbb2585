// Decode attention over the cache that an eviction pass leaves: one decode
// step's scaled dot-product attention of each KV head's G query heads over
// the unit's n cached rows ("TriAttention Native C++ Worklog", "What was
// implemented": decode continues on the compacted cache; the llama.cpp page's
// section 4 GQA grouping, query head g*G + j on KV head g).  Row order does not
// matter to softmax, so ordered and hole-filled caches are read alike.
//
//   s_j(r) = scale * q_j . k_r,  out_j = sum_r softmax_r(s_j)(r) * v_r.
//
// Split over row ranges (flash-decoding): workgroup (split, unit) walks its
// range in 64-row tiles, wavefront w taking tiles w, w + 4, ...  Per tile:
//   1. lane = row: s_j for the row (K decoded to fp32; q_j read through scalar
//      loads -- every lane needs the same query value at the same time);
//   2. online softmax: tile max and sum per head by wavefront reductions,
//      the running output rescaled, the tile's probabilities staged in LDS;
//   3. lane = dims: out_j[d] += p_j(r) v_r[d] over the tile's rows (each V row
//      read as one coalesced sweep of the wavefront).
// The four wavefronts merge in LDS; a second kernel merges the splits.
// fp32 throughout.  HBM-bound: every K and V row is read once.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kAttMaxG = 8;  // heads per launch (groups of 8 for larger G)

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_add_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float half_of(uint32_t w, int hi) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? (w >> 16) : (w & 0xffffu)));
}

// Element e of a stored row as fp32 (fp16: 2 bytes each; q8_0: 34-byte blocks
// of an fp16 scale and 32 int8).
__device__ __forceinline__ float row_elem(const uint8_t* row, int k_type, int e) {
    if (k_type == TRIA_KV_F16) {
        return (float)*reinterpret_cast<const _Float16*>(row + 2 * e);
    }
    const uint8_t* blk = row + 34 * (e >> 5);
    const float d = (float)*reinterpret_cast<const _Float16*>(blk);
    return d * (float)(int8_t)blk[2 + (e & 31)];
}

// q_j . k for one row of an fp16 key: 16-byte pieces (rows are 2*HD bytes,
// 16-byte aligned), each converted and used at once.
template <int HD, int GT>
__device__ __forceinline__ void dot_f16(const uint8_t* row, const float* __restrict__ Q, int z,
                                        float (&s)[GT]) {
    const u32x4* r4 = reinterpret_cast<const u32x4*>(row);
#pragma unroll
    for (int j = 0; j < GT; ++j) s[j] = 0.0f;
#pragma unroll 2
    for (int c = 0; c < HD / 8; ++c) {
        const u32x4 x = r4[c];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float kv = half_of(w[i >> 1], i & 1);
#pragma unroll
            for (int j = 0; j < GT; ++j) s[j] = fmaf(Q[z + j * HD + 8 * c + i], kv, s[j]);
        }
    }
}

// q_j . k for one row of a q8_0 key (34 * HD/32 bytes, so rows are 8-byte
// aligned when HD/32 % 4 == 0, 4-byte aligned when it is even): the whole row
// is read with 8- or 4-byte loads, else 2 bytes at a time; per block, the int8
// values times q, then the scale.
template <int HD, int GT>
__device__ __forceinline__ void dot_q8(const uint8_t* row, const float* __restrict__ Q, int z,
                                       float (&s)[GT]) {
    constexpr int NB = HD / 32;
#pragma unroll
    for (int j = 0; j < GT; ++j) s[j] = 0.0f;
    if constexpr (NB % 2 == 0) {
        constexpr int W = 34 * NB / 4;
        uint32_t wv[W];
        if constexpr (NB % 4 == 0) {
            const u32x2* r2 = reinterpret_cast<const u32x2*>(row);
#pragma unroll
            for (int i = 0; i < W / 2; ++i) {
                const u32x2 t = r2[i];
                wv[2 * i] = t.x;
                wv[2 * i + 1] = t.y;
            }
        } else {
            const uint32_t* r1 = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
            for (int i = 0; i < W; ++i) wv[i] = r1[i];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int o = 34 * b;
            const float d = half_of(wv[o >> 2], (o & 2) != 0);
            float t[GT];
#pragma unroll
            for (int j = 0; j < GT; ++j) t[j] = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int ob = o + 2 + i;
                const float kv = (float)(int8_t)(wv[ob >> 2] >> (8 * (ob & 3)));
#pragma unroll
                for (int j = 0; j < GT; ++j) t[j] = fmaf(Q[z + j * HD + 32 * b + i], kv, t[j]);
            }
#pragma unroll
            for (int j = 0; j < GT; ++j) s[j] = fmaf(d, t[j], s[j]);
        }
    } else {
#pragma unroll 1
        for (int b = 0; b < NB; ++b) {
            const uint16_t* h = reinterpret_cast<const uint16_t*>(row + 34 * b);
            const float d = (float)__builtin_bit_cast(_Float16, h[0]);
            float t[GT];
#pragma unroll
            for (int j = 0; j < GT; ++j) t[j] = 0.0f;
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2) {
                const uint16_t x = h[1 + i2];
                const float a = (float)(int8_t)(x & 0xff), c = (float)(int8_t)(x >> 8);
#pragma unroll
                for (int j = 0; j < GT; ++j) {
                    t[j] = fmaf(Q[z + j * HD + 32 * b + 2 * i2], a, t[j]);
                    t[j] = fmaf(Q[z + j * HD + 32 * b + 2 * i2 + 1], c, t[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < GT; ++j) s[j] = fmaf(d, t[j], s[j]);
        }
    }
}

__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// Per (unit, split, head): running max m, sum l and the unnormalised output.
struct AttPart {
    float m, l;
};

// V rows read as 16-byte pieces (8 fp16 values): LPR lanes cover a row, so a
// wavefront reads 64 / LPR rows per instruction.  HD in {32, 64, 128, 256}.
template <int HD>
constexpr bool kVecV = HD == 32 || HD == 64 || HD == 128 || HD == 256;

// grid (splits, units); q: [seq][L][Hq][HD] fp32; parts: [unit][split][G]
// records, pacc: [unit][split][G][HD].  Heads j0 .. j0+GT-1 of each group.
// VEC: fp16 V read in 16-byte pieces (see kVecV); else element by element.
template <int HD, int GT, bool VEC>
__global__ __launch_bounds__(kAttThreads) void attention_split_kernel(
    CacheView cv, Batch b, int G, int j0, int k_type, int v_type, const float* __restrict__ q,
    float scale, int rows_per_split, AttPart* __restrict__ parts, float* __restrict__ pacc) {
    constexpr int LPR = VEC ? HD / 8 : 64;         // lanes per V row
    constexpr int RPI = 64 / LPR;                  // V rows per wavefront instruction
    constexpr int NACC = VEC ? 8 : (HD + 63) / 64;  // output dims per lane
    __shared__ float p_sh[kAttWaves][GT][64];
    __shared__ float m_sh[kAttWaves][GT], l_sh[kAttWaves][GT];
    __shared__ float acc_sh[kAttWaves][GT][HD];
    const int u = blockIdx.y, split = blockIdx.x, n_split = gridDim.x;
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const int64_t n = sd.n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int dg = lane % LPR, ro = lane / LPR;  // VEC: dims 8 dg .. 8 dg + 7 of rows = ro mod RPI
    const int64_t r_lo = (int64_t)split * rows_per_split;
    const int64_t r_hi = r_lo + rows_per_split < n ? r_lo + rows_per_split : n;
    const int Hq = cv.Hkv * G;
    const float* Qu = q + (((int64_t)id.seq * cv.L + id.l) * Hq + (int64_t)id.g * G + j0) * HD;

    float m[GT], l[GT], acc[GT][NACC];
#pragma unroll
    for (int j = 0; j < GT; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[j][i] = 0.0f;
    }
    const int kb = cv.kb, vb = cv.vb;
    for (int64_t t0 = r_lo + (int64_t)wave * 64; t0 < r_hi; t0 += kAttWaves * 64) {
        // 1. scores, lane = row
        const int64_t r = t0 + lane;
        const bool valid = r < r_hi;
        float s[GT];
        {
            const int64_t rr = valid ? r : t0;
            const uint8_t* row = cv.k + row_index(cv, id, rr) * kb;
            const int z = opaque_zero();
            if (k_type == TRIA_KV_F16) dot_f16<HD, GT>(row, Qu, z, s);
            else dot_q8<HD, GT>(row, Qu, z, s);
        }
        // 2. online softmax over the tile
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            const float sj = valid ? s[j] * scale : -INFINITY;
            const float tmax = wave_max_f32(sj);
            const float mn = fmaxf(m[j], tmax);
            const float alpha = m[j] == -INFINITY ? 0.0f : __expf(m[j] - mn);
            const float p = valid ? __expf(sj - mn) : 0.0f;
            l[j] = l[j] * alpha + wave_add_f32(p);
            m[j] = mn;
#pragma unroll
            for (int i = 0; i < NACC; ++i) acc[j][i] *= alpha;
            p_sh[wave][j][lane] = p;
        }
        // 3. accumulate the tile's V rows (LDS writes of this wave are visible to
        //    its own later reads: one wavefront, in order)
        const int nt = (int)(r_hi - t0 < 64 ? r_hi - t0 : 64);
        if constexpr (VEC) {
            // unrolled so that several V loads of a tile are in flight together
            // (two per pass, as the compiler left the loop, ran at 5.0 TB/s
            // against 6.1 with four; eight per pass cost G = 8 a wave per SIMD)
            constexpr int kVUnroll = GT <= 4 ? 4 : 2;
#pragma unroll kVUnroll
            for (int rr = ro; rr < nt; rr += RPI) {
                const uint8_t* vrow = cv.v + row_index(cv, id, t0 + rr) * vb;
                // V is read once per step: streaming (non-temporal) loads
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vrow) + dg);
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                float vv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) vv[i] = half_of(w[i >> 1], i & 1);
#pragma unroll
                for (int j = 0; j < GT; ++j) {
                    const float p = p_sh[wave][j][rr];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(p, vv[i], acc[j][i]);
                }
            }
        } else {
            for (int rr = 0; rr < nt; ++rr) {
                const uint8_t* vrow = cv.v + row_index(cv, id, t0 + rr) * vb;
                float vv[NACC];
#pragma unroll
                for (int i = 0; i < NACC; ++i) {
                    const int e = lane + 64 * i;
                    vv[i] = e < HD ? row_elem(vrow, v_type, e) : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < GT; ++j) {
                    const float p = p_sh[wave][j][rr];
#pragma unroll
                    for (int i = 0; i < NACC; ++i) acc[j][i] = fmaf(p, vv[i], acc[j][i]);
                }
            }
        }
    }
    // VEC: add the RPI row groups' partial sums (lanes dg, dg + LPR, ...)
    if constexpr (VEC) {
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
            for (int j = 0; j < GT; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[j][i] += __shfl_xor(acc[j][i], o, 64);
        }
    }
    // merge the four wavefronts
#pragma unroll
    for (int j = 0; j < GT; ++j) {
        if (lane == 0) {
            m_sh[wave][j] = m[j];
            l_sh[wave][j] = l[j];
        }
        if constexpr (VEC) {
            if (ro == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc_sh[wave][j][8 * dg + i] = acc[j][i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < NACC; ++i) {
                const int e = lane + 64 * i;
                if (e < HD) acc_sh[wave][j][e] = acc[j][i];
            }
        }
    }
    __syncthreads();
    const int64_t rec = ((int64_t)u * n_split + split) * G + j0;
    for (int x = threadIdx.x; x < GT * HD; x += kAttThreads) {
        const int j = x / HD, e = x - j * HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, m_sh[w][j]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) {
            const float f = m_sh[w][j] == -INFINITY ? 0.0f : __expf(m_sh[w][j] - M);
            L += l_sh[w][j] * f;
            A += acc_sh[w][j][e] * f;
        }
        pacc[(rec + j) * HD + e] = A;
        if (e == 0) parts[rec + j] = AttPart{M, L};
    }
}

// One block per (unit, head): merges the splits; no rows at all gives zeros.
template <int HD>
__global__ __launch_bounds__(kAttThreads) void attention_combine_kernel(
    CacheView cv, int G, int n_split, const AttPart* __restrict__ parts,
    const float* __restrict__ pacc, float* __restrict__ out) {
    const int u = blockIdx.x / G, j = blockIdx.x - (blockIdx.x / G) * G;
    const UnitId id = unit_id(cv, u);
    const int Hq = cv.Hkv * G;
    float* O = out + (((int64_t)id.seq * cv.L + id.l) * Hq + (int64_t)id.g * G + j) * HD;
    const int64_t rec0 = (int64_t)u * n_split * G + j;
    float M = -INFINITY;
    for (int sp = 0; sp < n_split; ++sp) M = fmaxf(M, parts[rec0 + (int64_t)sp * G].m);
    for (int e = threadIdx.x; e < HD; e += kAttThreads) {
        float L = 0.0f, A = 0.0f;
        for (int sp = 0; sp < n_split; ++sp) {
            const AttPart pt = parts[rec0 + (int64_t)sp * G];
            const float f = pt.m == -INFINITY ? 0.0f : __expf(pt.m - M);
            L += pt.l * f;
            A += pacc[(rec0 + (int64_t)sp * G) * HD + e] * f;
        }
        O[e] = L > 0.0f ? A / L : 0.0f;
    }
}

template <int HD, int GT>
void run_split(dim3 grid, hipStream_t s, const CacheView& cv, const Batch& b, int G, int j0,
               int kt, int vt, const float* q, float scale, int rps, AttPart* parts,
               float* pacc) {
    if (kVecV<HD> && vt == TRIA_KV_F16)
        hipLaunchKernelGGL((attention_split_kernel<HD, GT, kVecV<HD>>), grid, dim3(kAttThreads), 0,
                           s, cv, b, G, j0, kt, vt, q, scale, rps, parts, pacc);
    else
        hipLaunchKernelGGL((attention_split_kernel<HD, GT, false>), grid, dim3(kAttThreads), 0, s,
                           cv, b, G, j0, kt, vt, q, scale, rps, parts, pacc);
}

template <int HD>
hipError_t launch_hd(const CacheView& cv, const Batch& b, int n_units, int G, int kt, int vt,
                     const float* q, float scale, int n_split, int rps, AttPart* parts,
                     float* pacc, float* out, hipStream_t s) {
    const dim3 grid((unsigned)n_split, (unsigned)n_units);
    for (int j0 = 0; j0 < G;) {
        const int left = G - j0;
        const int gt = left >= 8 ? 8 : (left >= 4 ? 4 : (left >= 2 ? 2 : 1));
        switch (gt) {
            case 8: run_split<HD, 8>(grid, s, cv, b, G, j0, kt, vt, q, scale, rps, parts, pacc); break;
            case 4: run_split<HD, 4>(grid, s, cv, b, G, j0, kt, vt, q, scale, rps, parts, pacc); break;
            case 2: run_split<HD, 2>(grid, s, cv, b, G, j0, kt, vt, q, scale, rps, parts, pacc); break;
            default: run_split<HD, 1>(grid, s, cv, b, G, j0, kt, vt, q, scale, rps, parts, pacc); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        j0 += gt;
    }
    hipLaunchKernelGGL((attention_combine_kernel<HD>), dim3((unsigned)(n_units * G)),
                       dim3(kAttThreads), 0, s, cv, G, n_split, parts, pacc, out);
    return hipGetLastError();
}

}  // namespace

// Row ranges per unit: enough workgroups to fill the device several times,
// each range a multiple of 64 rows.
void attention_splits(const Batch& b, int n_units, int* n_split, int* rows_per_split) {
    int64_t max_n = 0;
    for (int i = 0; i < b.n_seq; ++i) max_n = b.seq[i].n > max_n ? b.seq[i].n : max_n;
    int ns = (int)((4096 + n_units - 1) / (n_units > 0 ? n_units : 1));
    const int64_t tiles = (max_n + 63) / 64;
    if (ns > tiles) ns = (int)(tiles > 0 ? tiles : 1);
    if (ns < 1) ns = 1;
    if (ns > 256) ns = 256;
    const int64_t per = ((tiles + ns - 1) / ns) * 64;
    *n_split = (int)((max_n + per - 1) / (per > 0 ? per : 1));
    if (*n_split < 1) *n_split = 1;
    *rows_per_split = (int)(per > 0 ? per : 64);
}

hipError_t launch_attention(const CacheView& cv, const Batch& b, int n_units, int G, int hd,
                            int k_type, int v_type, const float* q, float scale, int n_split,
                            int rows_per_split, void* parts, float* pacc, float* out,
                            hipStream_t s) {
    AttPart* P = static_cast<AttPart*>(parts);
    switch (hd) {
        case 32: return launch_hd<32>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 64: return launch_hd<64>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 96: return launch_hd<96>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 128: return launch_hd<128>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 160: return launch_hd<160>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 192: return launch_hd<192>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 224: return launch_hd<224>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        case 256: return launch_hd<256>(cv, b, n_units, G, k_type, v_type, q, scale, n_split, rows_per_split, P, pacc, out, s);
        default: return hipErrorInvalidValue;
    }
}

size_t attention_part_bytes() { return sizeof(AttPart); }

}  // namespace tria
