// compact: in-place, order-preserving gather of the kept rows.
//
// llama.cpp page "TriAttention KV-Cache Eviction (--triattention)", section 5
// "Phase B" step 4: compact the cache in place, no gaps.  "TriAttention
// Native C++ Worklog", section "What was implemented": one GPU gather/repack
// instead of many small device copies; the result must be an exact gather of
// the kept rows (the worklog's post- vs pre-compaction checks).
//
//   row d <- row keep_idx[d], d < kept, for K, V and positions.
//
// In place without a second buffer.  keep_idx is ascending with
// keep_idx[d] >= d, so a row is overwritten only by a destination at or below
// it, and the only hazard is a write landing on a row that a smaller
// destination still has to read.
//
// The destinations of a unit are cut into chunks of CR rows (256, 128 or 64:
// the widest whose pieces fit one workgroup's registers); a task moves one
// chunk of one unit (K, V and positions).  A task
//   1. loads the source rows of its chunk into registers,
//   2. once they have arrived, publishes that (flag[unit][chunk] = epoch),
//   3. waits until every earlier chunk that reads a row of its own
//      destination range has published, and
//   4. stores.
// The chunks that read rows [CR c, CR c + CR) are exactly those holding the
// ranks P(CR c) .. P(CR c + CR)-1, P(x) = number of kept rows below x (the
// selector writes P every 64 rows); a later chunk never reads them, because its
// sources lie above its own destinations.  So every read sees the original
// row and no task waits on anything but loads that are already in flight.
//
// Tasks are handed out in increasing order from a ticket counter (a few at a
// time), ordered by chunk, then unit, and numbered densely: only the chunks a
// unit has are tasks (sequences of a batch keep different row counts).  So
// the chunks of a unit are taken in order and a task only waits on smaller
// tasks, all of which are held by workgroups that are already running.  The
// smallest unfinished task never waits, whatever subset of the grid is
// resident (other kernels may share the GPU).  Each wait is also bounded: a workgroup that gives up records an
// error (see tria_device_status) and stores anyway.  The counter is reset by
// the kernel that runs before the compaction on the same stream (the
// selector, or the prefix-count kernel for caller-provided indices).
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kMaxFlowThreads = 1024;
constexpr int kSpinLimit = 1 << 18;  // polls (each a memory round trip plus a short sleep)
// Pieces per thread and array; the launch uses 256, 512 or 1024 threads so
// that a chunk of either array needs at most this many.
constexpr int kItems = 8;
// Piece code of an array moved in 4-byte words (HalfMove below).
constexpr int kWords = 1;

template <int PW>
struct Piece;
template <>
struct Piece<16> { using T = u32x4; };
template <>
struct Piece<8> { using T = u32x2; };
template <>
struct Piece<4> { using T = uint32_t; };
template <>
struct Piece<2> { using T = uint16_t; };

template <typename T>
__device__ __forceinline__ void hold(const T& x) {
    // A use of the register: the compiler waits for the load that fills it.
    asm volatile("" ::"v"(x));
}

// Item k of this thread is piece i = t + blockDim k of the chunk in row-major
// order: row i / ppr, byte (i % ppr) * PW.  Rows and offsets advance by a
// fixed step per item, so no division per item.
struct ItemWalk {
    int r, off, dr, doff, ppr_bytes;
    __device__ __forceinline__ ItemWalk(int ppr, int pw) {
        const int i = (int)threadIdx.x, nt = (int)blockDim.x;
        r = i / ppr;
        off = (i - r * ppr) * pw;
        dr = nt / ppr;
        doff = (nt - dr * ppr) * pw;
        ppr_bytes = ppr * pw;
    }
    __device__ __forceinline__ void next() {
        r += dr;
        off += doff;
        if (off >= ppr_bytes) {
            off -= ppr_bytes;
            ++r;
        }
    }
};

// One array's part of a task: the pieces of the chunk's rows, dealt to the
// threads in row-major order (consecutive threads move consecutive pieces).
//
// A moved byte is read once and written once, so the loads carry the
// non-temporal (streaming) cache hint, and so do the stores of 16-byte pieces
// (rows of fp16 values).  Narrower pieces (rows of q8_0 blocks: 136-byte rows
// straddle 128-byte lines) keep the normal store policy; on MI355X the hint
// made those stores slower and the others faster.  The hint changes no
// ordering: a read never needs a value written by the same pass.
template <int PW, int CR>
struct ArrayMove {
    using T = typename Piece<PW>::T;
    T buf[kItems];

    __device__ __forceinline__ void load(const uint8_t* base, int rb, const int64_t* src) {
        ItemWalk w(rb / PW, PW);
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            if (w.r < CR) {
                const int64_t s = src[w.r];
                if (s >= 0)
                    buf[k] = __builtin_nontemporal_load(reinterpret_cast<const T*>(base + s * rb + w.off));
            }
            w.next();
        }
    }
    __device__ __forceinline__ void wait() {
#pragma unroll
        for (int k = 0; k < kItems; ++k) hold(buf[k]);
    }
    __device__ __forceinline__ void store(uint8_t* base, int rb, const int64_t* src,
                                          const int64_t* dst) const {
        ItemWalk w(rb / PW, PW);
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            if (w.r < CR && src[w.r] >= 0) {
                T* p = reinterpret_cast<T*>(base + dst[w.r] * rb + w.off);
                if constexpr (PW == 16)
                    __builtin_nontemporal_store(buf[k], p);
                else
                    *p = buf[k];
            }
            w.next();
        }
    }
};

// An array whose row width is 2 modulo 4 (q8_0 rows at head_dim 32, 96, 160,
// 224) has rows on 2-byte boundaries only.  Where its 2-byte pieces would not
// fit 256-row chunks (rows over 64 bytes), it is moved in aligned 4-byte
// destination words instead (piece code kWords): each 16-row group of the chunk
// (contiguous in memory in both layouts) is one byte span, and lane l of the
// group's wavefront(s) takes the span's words l, l + 64 W, ... (W wavefronts
// per group).  A word's two halves may belong to two rows (a row boundary in
// the middle of the word) and come from two source rows; each half is read
// with the aligned 4-byte load that holds it (one load when both halves lie in
// one aligned source word), and the word is stored whole when both halves
// move, else as the one 2-byte half that does.  Every load holds a byte of a
// moved source row and every store writes only bytes of moved destination rows
// of this chunk, so neighbouring spans (other chunks, other units) are never
// written.  Needs all kMaxFlowThreads threads.
template <int CR>
struct HalfMove {
    static constexpr int kGroups = CR / kBlockRows;
    static constexpr int kWavesPerGroup = (kMaxFlowThreads / 64) / kGroups;
    static constexpr int kStep = 64 * kWavesPerGroup;  // words between a lane's items
    static constexpr int kItems = 8;
    static_assert(kGroups * kWavesPerGroup == kMaxFlowThreads / 64, "whole wavefronts per group");
    uint32_t lo[kItems], hi[kItems];
    // per item one byte: 1 half 0 moves, 2 half 1 moves, 4 half 0 is lo's upper
    // half, 8 half 1 is the upper half (of lo if 16, else of hi)
    uint64_t sel;

    // Byte offset of this wavefront's span (its group's first row), -1 when no
    // row of the group moves; the group's first row within the chunk.
    __device__ __forceinline__ static int64_t span_start(const int64_t* grp, int rb, int* g0) {
        const int g = (int)(threadIdx.x >> 6) / kWavesPerGroup;
        *g0 = g * kBlockRows;
        return grp[g] < 0 ? -1 : grp[g] * rb;
    }
    __device__ __forceinline__ static int first_word() {
        return ((int)(threadIdx.x >> 6) % kWavesPerGroup) * 64 + (int)(threadIdx.x & 63);
    }
    __device__ __forceinline__ void load(const uint8_t* base, int rb, const int64_t* src,
                                         const int64_t* grp) {
        sel = 0;
#pragma unroll
        for (int k = 0; k < kItems; ++k) lo[k] = hi[k] = 0u;
        int g0;
        const int64_t G = span_start(grp, rb, &g0);
        if (G < 0) return;
        const int span = kBlockRows * rb;
        // span byte p of half 0 of the lane's first word (p >= -2) as row r and
        // byte off (p = -2: r = -1, off = rb - 2); later words are 4 kStep bytes on
        const int p0 = 4 * first_word() - (int)(G & 3);
        int r = p0 < 0 ? -1 : p0 / rb;
        int off = p0 - r * rb;
        const int dr = (4 * kStep) / rb, doff = (4 * kStep) - dr * rb;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int p = p0 + 4 * kStep * k;
            if (p >= span) break;
            const int64_t s0 = r >= 0 ? src[g0 + r] : -1;
            int r1 = r, off1 = off + 2;
            if (off1 == rb) {
                ++r1;
                off1 = 0;
            }
            const int64_t s1 = p + 2 >= span ? -1 : (r1 == r ? s0 : src[g0 + r1]);
            const int64_t a0 = s0 >= 0 ? s0 * rb + off : -1;  // source bytes, -1: not moved
            const int64_t a1 = s1 >= 0 ? s1 * rb + off1 : -1;
            const bool m0 = a0 >= 0, m1 = a1 >= 0;
            const bool one = m0 && m1 && r1 == r && (a0 & 3) == 0;  // one source word
            if (m0)
                lo[k] = __builtin_nontemporal_load(
                    reinterpret_cast<const uint32_t*>(base + (a0 & ~(int64_t)3)));
            if (m1 && !one)
                hi[k] = __builtin_nontemporal_load(
                    reinterpret_cast<const uint32_t*>(base + (a1 & ~(int64_t)3)));
            const uint64_t bits = (m0 ? 1u : 0u) | (m1 ? 2u : 0u) | ((a0 & 2) ? 4u : 0u) |
                                  ((a1 & 2) ? 8u : 0u) | (one ? 16u : 0u);
            sel |= bits << (8 * k);
            r += dr;
            off += doff;
            if (off >= rb) {
                off -= rb;
                ++r;
            }
        }
    }
    __device__ __forceinline__ void wait() {
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            hold(lo[k]);
            hold(hi[k]);
        }
    }
    __device__ __forceinline__ void store(uint8_t* base, int rb, const int64_t* grp) const {
        int g0;
        const int64_t G = span_start(grp, rb, &g0);
        if (G < 0) return;
        const int64_t w0 = (G & ~(int64_t)3) + 4 * (int64_t)first_word();
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const uint32_t bits = (uint32_t)(sel >> (8 * k)) & 0xffu;
            if ((bits & 3u) == 0u) continue;
            const uint32_t h0 = (bits & 4u) ? (lo[k] >> 16) : (lo[k] & 0xffffu);
            const uint32_t x1 = (bits & 16u) ? lo[k] : hi[k];
            const uint32_t h1 = (bits & 8u) ? (x1 >> 16) : (x1 & 0xffffu);
            uint8_t* w = base + w0 + 4 * (int64_t)kStep * k;
            if ((bits & 3u) == 3u)
                *reinterpret_cast<uint32_t*>(w) = h0 | (h1 << 16);
            else if (bits & 1u)
                *reinterpret_cast<uint16_t*>(w) = (uint16_t)h0;
            else
                *reinterpret_cast<uint16_t*>(w + 2) = (uint16_t)h1;
        }
    }
};

// The mover of one array: pieces of PW bytes, or 4-byte words (PW == kWords).
template <int PW, int CR>
struct MoverOf { using T = ArrayMove<PW, CR>; };
template <int CR>
struct MoverOf<kWords, CR> { using T = HalfMove<CR>; };

template <int PW, int CR>
__device__ __forceinline__ void move_load(ArrayMove<PW, CR>& m, const uint8_t* base, int rb,
                                          const int64_t* src, const int64_t*) {
    m.load(base, rb, src);
}
template <int CR>
__device__ __forceinline__ void move_load(HalfMove<CR>& m, const uint8_t* base, int rb,
                                          const int64_t* src, const int64_t* grp) {
    m.load(base, rb, src, grp);
}
template <int PW, int CR>
__device__ __forceinline__ void move_store(const ArrayMove<PW, CR>& m, uint8_t* base, int rb,
                                           const int64_t* src, const int64_t* dst, const int64_t*) {
    m.store(base, rb, src, dst);
}
template <int CR>
__device__ __forceinline__ void move_store(const HalfMove<CR>& m, uint8_t* base, int rb,
                                           const int64_t*, const int64_t*, const int64_t* grp) {
    m.store(base, rb, grp);
}

// Destination chunks of CR rows per unit (a multiple of kChunkRows).
template <int CR>
__host__ __device__ inline int64_t flow_chunks(int64_t kept) { return (kept + CR - 1) / CR; }

// Chunks of CR rows a unit of the sequence moves (0 when nothing is evicted).
__host__ __device__ inline int seq_chunks(const SeqDesc& sd, int cr) {
    return (sd.kept > 0 && sd.kept < sd.n) ? (int)((sd.kept + cr - 1) / cr) : 0;
}

// Dense task numbering.  With the sequences sorted by chunk count v_0 >= v_1
// >= ... (ties by index) and P = units per sequence, chunk level c holds the
// sequences with v_i > c, P units each, and tasks run level by level.  Segment
// k covers levels [v_{k+1}, v_k), where sorted sequences 0 .. k are present;
// it starts at task P ((k + 1) v_{k+1} + sum_{i > k} v_i).
struct TaskPlan {
    uint32_t t0[kMaxSeq];  // first task of segment k (non-increasing in k)
    int c0[kMaxSeq];       // first level of segment k
    int seq[kMaxSeq];      // sorted position -> sequence
    int segs;              // sequences with at least one chunk
};

// A value every lane holds alike, as a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// Called by every thread of the workgroup; the first wavefront (one lane per
// sequence, n_seq <= 64) does the work.  The caller synchronises before use.
static_assert(kMaxSeq <= 64, "one lane of a wavefront per sequence");
template <int CR>
__device__ void build_plan(const Batch& b, TaskPlan& tp, int* sorted_v) {
    const int i = threadIdx.x;
    if (i < 64) {
        const int v = i < b.n_seq ? seq_chunks(b.seq[i], CR) : -1;
        int rank = 0, segs = 0;  // rank: position in the sorted order
        for (int j = 0; j < b.n_seq; ++j) {
            const int vj = __shfl(v, j);
            rank += (vj > v) || (vj == v && j < i);
            segs += vj > 0;
        }
        if (i < b.n_seq) {
            sorted_v[rank] = v;
            tp.seq[rank] = i;
        }
        if (i == 0) tp.segs = segs;
    }
    __syncthreads();
    if (i < tp.segs) {
        int64_t tail = 0;  // sum of v over sorted positions > i
        for (int j = i + 1; j < tp.segs; ++j) tail += sorted_v[j];
        const int v1 = i + 1 < tp.segs ? sorted_v[i + 1] : 0;
        tp.t0[i] = (uint32_t)((int64_t)(i + 1) * v1 + tail);  // in units of P
        tp.c0[i] = v1;
    }
}

template <int PK, int PV, int CR>
__global__ __launch_bounds__(kMaxFlowThreads) void compact_flow_kernel(
    CacheView cv, Batch b, const int32_t* __restrict__ keep, const int32_t* __restrict__ pb,
    uint32_t* flags, int max_chunks, uint32_t n_tasks, int ticket_tasks, uint32_t* ticket,
    int* err) {
    constexpr int kPerP = CR / kChunkRows;  // prefix-count entries per chunk
    __shared__ int64_t src_row[CR];  // physical source row, -1 if the row stays
    __shared__ int64_t dst_row[CR];
    constexpr bool kHalf = PK == kWords || PV == kWords;
    // physical first row of each 16-row group (-1 past the kept rows)
    __shared__ int64_t grp_row[kHalf ? CR / kBlockRows : 1];
    __shared__ uint32_t first_sh;
    __shared__ TaskPlan tp;
    __shared__ int sorted_v[kMaxSeq];
    const int t = threadIdx.x;
    const int per_seq = cv.L * cv.Hkv;
    const uint32_t epoch = uniform(ticket[1]);  // set by the kernel before this one
    build_plan<CR>(b, tp, sorted_v);
    while (true) {
        if (t == 0) first_sh = atomicAdd(ticket, (uint32_t)ticket_tasks);
        __syncthreads();  // also publishes the plan on the first round
        const uint32_t first = uniform(first_sh);
        __syncthreads();
        if (first >= n_tasks) break;
        const uint32_t last = n_tasks - first > (uint32_t)ticket_tasks ? first + ticket_tasks : n_tasks;
        for (uint32_t task = first; task < last; ++task) {
            // segment: the smallest k with P t0[k] <= task (t0[segs - 1] == 0); the
            // plan is uniform, so the decode stays in scalar registers
            int lo = 0, hi = uniform(tp.segs) - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((uint64_t)uniform(tp.t0[mid]) * per_seq <= task) hi = mid;
                else lo = mid + 1;
            }
            const uint32_t rel = task - uniform(tp.t0[lo]) * (uint32_t)per_seq;
            const uint32_t level = (uint32_t)(lo + 1) * (uint32_t)per_seq;  // tasks per level
            const int c = uniform(tp.c0[lo]) + (int)(rel / level);
            const uint32_t r = rel % level;
            const int u = uniform(tp.seq[r / per_seq]) * per_seq + (int)(r % per_seq);
            const UnitId id = unit_id(cv, u);
            const SeqDesc& sd = b.seq[id.seq];
            const int kept = (int)sd.kept, n = (int)sd.n;
            // never taken (only the chunks a unit moves are tasks); kept as guards,
            // which also hold the kernel to fewer registers
            if (kept <= 0 || kept >= n) continue;
            if (c >= (int)flow_chunks<CR>(kept)) continue;
            const int uu = id.l * cv.Hkv + id.g;
            const int32_t* idx = keep + sd.keep_off + (int64_t)uu * kept;
            uint32_t* F = flags + (int64_t)u * max_chunks;
            const int d0 = c * CR;

            // 1. the chunk's sources, then its loads
            if (t < CR) {
                int64_t sr = -1, dr = -1;
                const int d = d0 + t;
                if (d < kept) {
                    const int s = idx[d];
                    if (s > d && s < n) {
                        sr = row_index(cv, id, s);
                        dr = row_index(cv, id, d);
                    }
                }
                src_row[t] = sr;
                dst_row[t] = dr;
            }
            if (kHalf && t < CR / kBlockRows) {
                const int d = d0 + kBlockRows * t;
                grp_row[t] = d < kept ? row_index(cv, id, d) : -1;
            }
            __syncthreads();
            typename MoverOf<PK, CR>::T mk;
            typename MoverOf<PV, CR>::T mv;
            uint32_t pos = 0;
            move_load(mk, cv.k, cv.kb, src_row, grp_row);
            move_load(mv, cv.v, cv.vb, src_row, grp_row);
            const int64_t ps = t < CR ? src_row[t] : -1;
            if (ps >= 0) pos = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cv.pos) + ps);
            mk.wait();
            mv.wait();
            hold(pos);
            __syncthreads();  // every source of this chunk has been read

            // 2. publish, 3. wait for the earlier chunks that read this chunk's rows
            if (t == 0) (void)__hip_atomic_exchange(&F[c], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (t < 64) {
                const int32_t* P = pb + sd.pb_off + (int64_t)uu * chunk_bounds(kept);
                const int nb = (int)chunk_count(kept);
                const int p0 = P[kPerP * c], p1 = P[min(kPerP * c + kPerP, nb)];
                const int lo = p0 / CR;
                const int hi = min(c - 1, (p1 - 1) / CR);
                if (p1 > p0) {
                    for (int base = lo; base <= hi; base += 64) {
                        const int cc = base + t;
                        int spins = 0;
                        while (true) {
                            const bool ready =
                                cc > hi ||
                                __hip_atomic_load(&F[cc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                                    epoch;
                            if (__ballot(!ready) == 0) break;
                            if (++spins > kSpinLimit) {
                                if (t == 0) atomicOr(err, 1);
                                break;
                            }
                            __builtin_amdgcn_s_sleep(2);
                        }
                    }
                }
            }
            __syncthreads();

            // 4. stores
            move_store(mk, cv.k, cv.kb, src_row, dst_row, grp_row);
            move_store(mv, cv.v, cv.vb, src_row, dst_row, grp_row);
            if (ps >= 0) __builtin_nontemporal_store(pos, reinterpret_cast<uint32_t*>(cv.pos) + dst_row[t]);
            __syncthreads();  // the row tables are rewritten by the next task
        }
    }
}

// P(64 e) for caller-provided kept indices: lower bound of 64 e in the
// ascending indices, one thread per (unit, boundary).
__global__ __launch_bounds__(256) void chunk_bounds_kernel(CacheView cv, Batch b,
                                                           const int32_t* __restrict__ keep,
                                                           int32_t* __restrict__ pb, int n_units,
                                                           int max_bounds, uint32_t* ticket) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i == 0) reset_ticket(ticket);  // for the compaction that follows on this stream
    if (i >= (int64_t)n_units * max_bounds) return;
    const int u = (int)(i / max_bounds), e = (int)(i - (int64_t)u * max_bounds);
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const int64_t kept = sd.kept;
    if (e >= chunk_bounds(kept)) return;
    const int uu = id.l * cv.Hkv + id.g;
    const int32_t* idx = keep + sd.keep_off + (int64_t)uu * kept;
    const int64_t x = (int64_t)e * kChunkRows;
    int64_t lo = 0, hi = kept;  // first position with idx >= x
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (idx[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    pb[sd.pb_off + (int64_t)uu * chunk_bounds(kept) + e] = (int32_t)lo;
}

int piece_width(int rb) {
    int pw = 16;
    while (pw > 2 && rb % pw != 0) pw >>= 1;
    return pw;
}

using FlowKernel = void (*)(CacheView, Batch, const int32_t*, const int32_t*, uint32_t*, int,
                            uint32_t, int, uint32_t*, int*);

template <int PK, int CR>
FlowKernel flow_for_v(int pv) {
    switch (pv) {
        case 16: return compact_flow_kernel<PK, 16, CR>;
        case 8: return compact_flow_kernel<PK, 8, CR>;
        case 4: return compact_flow_kernel<PK, 4, CR>;
        case 2: return compact_flow_kernel<PK, 2, CR>;
        default: return compact_flow_kernel<PK, kWords, CR>;
    }
}

template <int CR>
FlowKernel flow_kernel(int pk, int pv) {
    switch (pk) {
        case 16: return flow_for_v<16, CR>(pv);
        case 8: return flow_for_v<8, CR>(pv);
        case 4: return flow_for_v<4, CR>(pv);
        case 2: return flow_for_v<2, CR>(pv);
        default: return flow_for_v<kWords, CR>(pv);
    }
}

// Workgroups of a kernel that are resident at once on the whole device.
int resident_groups(FlowKernel k, int threads) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k),
                                                     threads, 0) != hipSuccess)
        return 0;
    return cus * per_cu;
}

// Tasks taken per ticket: two while a workgroup has few tasks (the last
// tickets balance the workgroups' ends), more when it has hundreds (a batch
// of sequences): each ticket is a round trip to one counter.
int ticket_size(int64_t tasks, int grid) {
    int64_t tt = tasks / ((int64_t)grid * 16);
    return (int)(tt < 2 ? 2 : (tt > 16 ? 16 : tt));
}

// 64-row chunks of the largest kept count (flags are sized for these; a launch
// with wider chunks uses fewer of them).
int64_t max_chunks_of(const Batch& b) {
    int64_t m = 0;
    for (int i = 0; i < b.n_seq; ++i) {
        const int64_t c = chunk_count(b.seq[i].kept);
        m = c > m ? c : m;
    }
    return m;
}

}  // namespace

int64_t compact_flag_words(const Batch& b, int n_units) {
    return max_chunks_of(b) * n_units;
}

hipError_t launch_compact(const CacheView& cv, const Batch& b, int n_units, const int32_t* keep,
                          const int32_t* pb, int32_t* pb_scratch, CompactState& st,
                          uint32_t* ticket, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    const int64_t max_chunks = max_chunks_of(b);
    if (max_chunks <= 0) return hipSuccess;
    if (max_chunks * n_units > st.flag_words) return hipErrorInvalidValue;
    if (!pb) {
        int64_t max_bounds = 0;
        for (int i = 0; i < b.n_seq; ++i) {
            const int64_t e = chunk_bounds(b.seq[i].kept);
            max_bounds = e > max_bounds ? e : max_bounds;
        }
        const int64_t threads = max_bounds * n_units;
        hipLaunchKernelGGL(chunk_bounds_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, s, cv, b, keep, pb_scratch, n_units, (int)max_bounds, ticket);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        pb = pb_scratch;
    }
    // the piece width of each array; rows of 2-byte pieces that would not fit
    // 256-row chunks move in 4-byte words
    auto code = [](int64_t rb) {
        const int pw = piece_width((int)rb);
        return pw == 2 && 4 * kChunkRows * (rb / 2) > (int64_t)kMaxFlowThreads * kItems ? kWords
                                                                                      : pw;
    };
    const int pk = code(cv.kb), pv = code(cv.vb);
    // the widest chunk (256, 128 or 64 rows) whose pieces fit kItems per thread
    // of a kMaxFlowThreads workgroup: fewer barriers and flag waits per byte and
    // more bytes in flight per workgroup.  In 4-byte words a 16-row group spans
    // at most 4 rb + 1 words, and its (kMaxFlowThreads / 64) / (rows / 16)
    // wavefronts take kItems per lane.
    auto fits = [&](int64_t rows) {
        for (int a = 0; a < 2; ++a) {
            const int64_t rb = a ? cv.vb : cv.kb;
            const int pw = a ? pv : pk;
            const int64_t waves = (kMaxFlowThreads / 64) / (rows / kBlockRows);
            if (pw == kWords ? 4 * rb + 1 > (int64_t)kItems * 64 * waves
                             : rows * (rb / pw) > (int64_t)kMaxFlowThreads * kItems)
                return false;
        }
        return true;
    };
    const int cr = fits(4 * kChunkRows) ? 4 * kChunkRows
                 : (fits(2 * kChunkRows) ? 2 * kChunkRows : kChunkRows);
    if (!fits(cr)) return hipErrorInvalidValue;
    const FlowKernel k = cr == 4 * kChunkRows   ? flow_kernel<4 * kChunkRows>(pk, pv)
                       : cr == 2 * kChunkRows ? flow_kernel<2 * kChunkRows>(pk, pv)
                                              : flow_kernel<kChunkRows>(pk, pv);
    // threads such that each array's chunk is at most kItems pieces per thread
    // (all of them for 4-byte words)
    int64_t ppr = 0;
    if (pk != kWords) ppr = cv.kb / pk;
    if (pv != kWords && cv.vb / pv > ppr) ppr = cv.vb / pv;
    const int64_t pieces = (int64_t)cr * ppr;
    int threads = 256;
    while ((int64_t)threads * kItems < pieces) threads *= 2;
    if (pk == kWords || pv == kWords) threads = kMaxFlowThreads;
    if (threads > kMaxFlowThreads) return hipErrorInvalidValue;
    int64_t chunks = 0, sum_chunks = 0;  // chunks of cr rows: the largest count, the sum
    for (int i = 0; i < b.n_seq; ++i) {
        const int64_t c = seq_chunks(b.seq[i], cr);
        chunks = c > chunks ? c : chunks;
        sum_chunks += c;
    }
    const int64_t per_seq = (int64_t)cv.L * cv.Hkv;
    if (per_seq * b.n_seq != n_units) return hipErrorInvalidValue;
    const int64_t tasks = sum_chunks * per_seq;
    if (tasks == 0) return hipSuccess;  // nothing evicted anywhere
    if (tasks >= (int64_t)1 << 31) return hipErrorInvalidValue;
    // as many workgroups as fit at once (residency is not required), or the cap
    int grid = resident_groups(k, threads);
    if (grid <= 0) return hipErrorInvalidValue;
    if (st.max_groups > 0 && st.max_groups < grid) grid = st.max_groups;
    const int tt = ticket_size(tasks, grid);
    const int64_t need = (tasks + tt - 1) / tt;
    if (need < grid) grid = (int)need;
    hipLaunchKernelGGL(k, dim3(grid), dim3(threads), 0, s, cv, b, keep, pb, st.flags,
                       (int)chunks, (uint32_t)tasks, tt, ticket, st.err);
    return hipGetLastError();
}

}  // namespace tria
