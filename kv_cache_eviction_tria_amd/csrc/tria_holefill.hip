// Hole-filling compaction: a variant of the order-preserving gather that
// moves far fewer rows in steady state (llama.cpp page "TriAttention KV-Cache
// Eviction (--triattention)", section 5 "Phase B" step 4 asks only that the
// kept rows end up packed in place with no gaps; the cache's cells carry
// their positions).
//
// With K kept rows of a unit of n rows (kept indices ascending):
//   run   = the trailing run of kept rows n-run .. n-1 (it holds the window);
//   lim   = K - run;
//   holes = rows below lim that are not kept, ascending;
//   tails = kept rows at or above lim outside the run, ascending (as many);
//   phase A: hole i <- tail i (no two moves touch the same row, and no move
//            reads a row another one writes: any order, any workgroup);
//   phase B: the run moves down by n - K rows to lim .. K-1, in order.
// Kept rows below lim (the sinks among them) stay where they are, so the
// selection's rules -- sinks are the first rows, the window the last ones --
// keep holding on the compacted cache, and the kept set of every later pass
// is the order-preserving pass's whenever no two candidates tie at the
// cutoff (ties go to the lower row, and rows are no longer in position
// order).  Phase B overwrites tails, so it runs after phase A (next launch).
//
// Both phases index the kept rows directly: the run length and the first tail
// by binary search, the i-th hole as i + e with e the first kept index whose
// rank-free gap idx[e] - e exceeds i.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kHoleThreads = 256;
constexpr int kHoleItems = 8;  // pieces per thread and array for a 64-row chunk
constexpr int kHoleBlocksPerUnit = 8;  // phase A workgroups per unit, at most

struct RunPlan {
    int run, lim, t0, m;  // trailing run, K - run, first tail, tail count
};

__device__ __forceinline__ RunPlan plan_of(const int32_t* __restrict__ idx, int K, int n) {
    RunPlan p;
    // run: the largest j with idx[K-j] == n-j for all j <= run (monotone)
    int lo = 0, hi = K;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (idx[K - mid] == n - mid) lo = mid;
        else hi = mid - 1;
    }
    p.run = lo;
    p.lim = K - p.run;
    // t0: first e < lim with idx[e] >= lim
    lo = 0;
    hi = p.lim;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] < p.lim) lo = mid + 1;
        else hi = mid;
    }
    p.t0 = lo;
    p.m = p.lim - p.t0;
    return p;
}

// Row i of the holes below lim: i + e, e the first index in [0, t0] with
// idx[e] - e > i (idx[t0] counts as beyond every hole).
__device__ __forceinline__ int hole_of(const int32_t* __restrict__ idx, int t0, int i) {
    int lo = 0, hi = t0;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] - mid > i) hi = mid;
        else lo = mid + 1;
    }
    return i + lo;
}

template <int PW>
struct PieceT;
template <>
struct PieceT<16> { using T = u32x4; };
template <>
struct PieceT<8> { using T = u32x2; };
template <>
struct PieceT<4> { using T = uint32_t; };
template <>
struct PieceT<2> { using T = uint16_t; };

template <typename T>
__device__ __forceinline__ void use(const T& x) {
    asm volatile("" ::"v"(x));  // the load that fills x has completed
}

// Phase A copy: the rows listed in src_row/dst_row (at most 64; src < 0: no
// move), every piece loaded and stored by the same thread (no move reads a row
// another one writes), pieces dealt row-major so that threads touch
// consecutive bytes.
// Moved bytes are read once and written once: loads carry the non-temporal
// (streaming) hint, and so do stores of 16-byte pieces (fp16 rows); narrower
// pieces (q8_0 rows straddle cache lines) keep the normal store policy, as in
// the ordered compaction.
template <int PW>
__device__ __forceinline__ void copy_direct(uint8_t* base, int rb, const int64_t* src,
                                            const int64_t* dst) {
    using T = typename PieceT<PW>::T;
    const int ppr = rb / PW;
    for (int i = threadIdx.x; i < kChunkRows * ppr; i += kHoleThreads) {
        const int r = i / ppr;
        if (src[r] >= 0) {
            const int off = (i - r * ppr) * PW;
            const T x = __builtin_nontemporal_load(reinterpret_cast<const T*>(base + src[r] * rb + off));
            T* d = reinterpret_cast<T*>(base + dst[r] * rb + off);
            if constexpr (PW == 16) __builtin_nontemporal_store(x, d);
            else *d = x;
        }
    }
}

// Phase B move of `rows` rows (rows * ppr <= kHoleThreads * kHoleItems): every
// piece is loaded into registers, the block synchronises, then stores.
template <int PW>
struct RowsMove {
    using T = typename PieceT<PW>::T;
    T buf[kHoleItems];
    __device__ __forceinline__ void load(const uint8_t* base, int rb, const int64_t* src,
                                         int rows) {
        const int ppr = rb / PW;
#pragma unroll
        for (int k = 0; k < kHoleItems; ++k) {
            const int i = (int)threadIdx.x + k * kHoleThreads;
            const int r = i / ppr;
            if (r < rows && src[r] >= 0)
                buf[k] = __builtin_nontemporal_load(
                    reinterpret_cast<const T*>(base + src[r] * rb + (i - r * ppr) * PW));
        }
    }
    __device__ __forceinline__ void wait() {
#pragma unroll
        for (int k = 0; k < kHoleItems; ++k) use(buf[k]);
    }
    __device__ __forceinline__ void store(uint8_t* base, int rb, const int64_t* src,
                                          const int64_t* dst, int rows) const {
        const int ppr = rb / PW;
#pragma unroll
        for (int k = 0; k < kHoleItems; ++k) {
            const int i = (int)threadIdx.x + k * kHoleThreads;
            const int r = i / ppr;
            if (r < rows && src[r] >= 0) {
                T* q = reinterpret_cast<T*>(base + dst[r] * rb + (i - r * ppr) * PW);
                if constexpr (PW == 16) __builtin_nontemporal_store(buf[k], q);
                else *q = buf[k];
            }
        }
    }
};

// Phase A: grid (kHoleBlocksPerUnit, units); block q takes chunks q, q + Q, ...
// of the unit's tail -> hole moves.
template <int PK, int PV>
__global__ __launch_bounds__(kHoleThreads) void holefill_tails_kernel(CacheView cv, Batch b,
                                                                      const int32_t* __restrict__ keep) {
    __shared__ int64_t src_row[kChunkRows];
    __shared__ int64_t dst_row[kChunkRows];
    const int u = blockIdx.y;
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const int K = (int)sd.kept, n = (int)sd.n;
    if (K <= 0 || K >= n) return;
    const int uu = id.l * cv.Hkv + id.g;
    const int32_t* idx = keep + sd.keep_off + (int64_t)uu * K;
    const RunPlan pl = plan_of(idx, K, n);
    const int t = threadIdx.x;
    for (int c0 = blockIdx.x * kChunkRows; c0 < pl.m; c0 += gridDim.x * kChunkRows) {
        if (t < kChunkRows) {
            int64_t sr = -1, dr = -1;
            const int i = c0 + t;
            if (i < pl.m) {
                const int src = idx[pl.t0 + i];
                const int dst = hole_of(idx, pl.t0, i);
                if (src >= pl.lim && src < n && dst >= 0 && dst < pl.lim) {
                    sr = row_index(cv, id, src);
                    dr = row_index(cv, id, dst);
                }
            }
            src_row[t] = sr;
            dst_row[t] = dr;
        }
        __syncthreads();
        copy_direct<PK>(cv.k, cv.kb, src_row, dst_row);
        copy_direct<PV>(cv.v, cv.vb, src_row, dst_row);
        if (t < kChunkRows && src_row[t] >= 0)
            reinterpret_cast<uint32_t*>(cv.pos)[dst_row[t]] =
                reinterpret_cast<const uint32_t*>(cv.pos)[src_row[t]];
        __syncthreads();  // the tables are rewritten for the next chunk
    }
}

// Phase B: one block per unit; the trailing run moves down by n - K rows,
// `rows` rows at a time in ascending order (a chunk's stores land only on
// rows that earlier chunks, or its own loads, have already read).
template <int PK, int PV>
__global__ __launch_bounds__(kHoleThreads) void holefill_run_kernel(CacheView cv, Batch b,
                                                                    const int32_t* __restrict__ keep,
                                                                    int rows) {
    __shared__ int64_t src_row[kChunkRows];
    __shared__ int64_t dst_row[kChunkRows];
    const int u = blockIdx.x;
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const int K = (int)sd.kept, n = (int)sd.n;
    if (K <= 0 || K >= n) return;
    const int uu = id.l * cv.Hkv + id.g;
    const int32_t* idx = keep + sd.keep_off + (int64_t)uu * K;
    const RunPlan pl = plan_of(idx, K, n);
    const int t = threadIdx.x;
    for (int c0 = 0; c0 < pl.run; c0 += rows) {
        if (t < rows) {
            int64_t sr = -1, dr = -1;
            const int j = c0 + t;
            if (j < pl.run) {
                sr = row_index(cv, id, n - pl.run + j);
                dr = row_index(cv, id, pl.lim + j);
            }
            src_row[t] = sr;
            dst_row[t] = dr;
        }
        __syncthreads();
        RowsMove<PK> mk;
        RowsMove<PV> mv;
        mk.load(cv.k, cv.kb, src_row, rows);
        mv.load(cv.v, cv.vb, src_row, rows);
        const int64_t ps = t < rows ? src_row[t] : -1;
        uint32_t p = 0;
        if (ps >= 0) p = reinterpret_cast<const uint32_t*>(cv.pos)[ps];
        mk.wait();
        mv.wait();
        use(p);
        __syncthreads();  // every source of the chunk has been read
        mk.store(cv.k, cv.kb, src_row, dst_row, rows);
        mv.store(cv.v, cv.vb, src_row, dst_row, rows);
        if (ps >= 0) reinterpret_cast<uint32_t*>(cv.pos)[dst_row[t]] = p;
        __syncthreads();  // stores issued before the tables are rewritten
    }
}

int piece_of(int rb) {
    int pw = 16;
    while (pw > 2 && rb % pw != 0) pw >>= 1;
    return pw;
}

template <int PK, int PV>
hipError_t launch_pv(const CacheView& cv, const Batch& b, int n_units, const int32_t* keep,
                     hipStream_t s) {
    // phase B chunk: as many rows (<= 64) as fit kHoleItems pieces per thread
    const int ppr = cv.kb / PK > cv.vb / PV ? cv.kb / PK : cv.vb / PV;
    int rows = kHoleThreads * kHoleItems / ppr;
    rows = rows > kChunkRows ? kChunkRows : rows;
    if (rows < 1) return hipErrorInvalidValue;
    // Phase A moves at most n - kept rows per unit (one per evicted row below
    // the run), so it needs no more blocks than 64-row chunks of that bound;
    // surplus blocks would only repeat the plan's binary searches and exit.
    int64_t most = 0;
    for (int i = 0; i < b.n_seq; ++i) {
        const int64_t e = b.seq[i].n - b.seq[i].kept;
        most = e > most ? e : most;
    }
    int64_t qa = (most + kChunkRows - 1) / kChunkRows;
    qa = qa < 1 ? 1 : (qa > kHoleBlocksPerUnit ? kHoleBlocksPerUnit : qa);
    hipLaunchKernelGGL((holefill_tails_kernel<PK, PV>), dim3((unsigned)qa, n_units),
                       dim3(kHoleThreads), 0, s, cv, b, keep);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((holefill_run_kernel<PK, PV>), dim3(n_units), dim3(kHoleThreads), 0, s, cv,
                       b, keep, rows);
    return hipGetLastError();
}

template <int PK>
hipError_t launch_pk(int pv, const CacheView& cv, const Batch& b, int n_units,
                     const int32_t* keep, hipStream_t s) {
    switch (pv) {
        case 16: return launch_pv<PK, 16>(cv, b, n_units, keep, s);
        case 8: return launch_pv<PK, 8>(cv, b, n_units, keep, s);
        case 4: return launch_pv<PK, 4>(cv, b, n_units, keep, s);
        default: return launch_pv<PK, 2>(cv, b, n_units, keep, s);
    }
}

}  // namespace

hipError_t launch_holefill(const CacheView& cv, const Batch& b, int n_units, const int32_t* keep,
                           hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    const int pk = piece_of(cv.kb), pv = piece_of(cv.vb);
    switch (pk) {
        case 16: return launch_pk<16>(pv, cv, b, n_units, keep, s);
        case 8: return launch_pk<8>(pv, cv, b, n_units, keep, s);
        case 4: return launch_pk<4>(pv, cv, b, n_units, keep, s);
        default: return launch_pk<2>(pv, cv, b, n_units, keep, s);
    }
}

}  // namespace tria
