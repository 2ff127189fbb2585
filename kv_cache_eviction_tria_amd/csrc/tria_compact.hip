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
// In place and race-free without a second buffer: keep_idx[d] >= d, so a row
// is only ever overwritten by a destination at or below it.  Each workgroup
// owns one independent byte column ("slice") of one array of one unit and
// walks the destination rows in increasing chunks.  A chunk's stores are
// issued only after a workgroup barrier that every thread reaches after its
// loads of that chunk's sources have returned.  Every source of a later chunk
// lies at or above that chunk's first destination, i.e. above everything an
// earlier chunk writes, so the loads of the next chunk are issued before the
// current chunk's stores (a one-chunk read-ahead, indices two chunks ahead):
// each chunk costs one overlapped memory round trip instead of two serial
// ones.  Rows whose source is the row itself are skipped, so a leading kept
// run costs nothing but its index read.  Slices of <= 128 bytes spread one
// unit over several workgroups; each thread of a slice moves one fixed column.
#include "tria_internal.h"

namespace tria {

namespace {

#ifndef TRIA_COMPACT_THREADS
#define TRIA_COMPACT_THREADS 256
#endif
constexpr int kCompactThreads = TRIA_COMPACT_THREADS;
constexpr int kMaxSlices = 16;
// Kept indices staged in LDS up to this size (keeps >= 2 workgroups per CU).
constexpr size_t kMaxIdxLds = 64 * 1024;

struct Slice {
    int32_t arr;    // 0 = K, 1 = V, 2 = positions
    int32_t off;    // byte offset of the slice in the row
    int32_t cw;     // bytes moved per item: 2, 4, 8 or 16
    int32_t lg;     // log2 of the items per row (a power of two, <= 64)
};

struct SliceSet {
    int32_t n;
    Slice s[kMaxSlices];
};

template <int CW>
struct Chunk;
template <>
struct Chunk<2> { using T = uint16_t; };
template <>
struct Chunk<4> { using T = uint32_t; };
template <>
struct Chunk<8> { using T = u32x2; };
template <>
struct Chunk<16> { using T = u32x4; };

template <typename T>
__device__ __forceinline__ void wait_loaded(const T& x) {
    // A use of the register: the compiler waits for the load that fills it.
    asm volatile("" ::"v"(x));
}

// Byte offset of logical row r of the unit from the unit's base pointer.
// Contiguous: rows are consecutive.  Paged: via the block table (64-bit).
template <bool PAGED>
struct RowAddr {
    uint8_t* base;
    int rb;
    const int32_t* bt;  // paged: this sequence's block-table row
    int64_t blk_stride; // paged: bytes per physical block of this layer
    __device__ __forceinline__ uint8_t* operator()(int32_t r) const {
        if constexpr (!PAGED) {
            return base + (uint32_t)r * (uint32_t)rb;
        } else {
            const int64_t blk = bt[r >> 4];
            return base + blk * blk_stride + (uint32_t)(r & 15) * (uint32_t)rb;
        }
    }
};

template <int CW, int IPT, bool PAGED, typename IdxT>
__device__ __forceinline__ void compact_slice(const RowAddr<PAGED>& ra, int off, int lg,
                                              IdxT idx, int32_t kept, int32_t n) {
    using T = typename Chunk<CW>::T;
    const int col = threadIdx.x & ((1 << lg) - 1);
    const int rr0 = threadIdx.x >> lg;
    const int rstep = kCompactThreads >> lg;  // rows between a thread's items
    const int rpc = IPT * rstep;              // rows per chunk
    const int32_t nchunks = (kept + rpc - 1) / rpc;
    const int coff = off + col * CW;

    auto load_idx = [&](int32_t c, int32_t (&src)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int32_t d = c * rpc + rr0 + i * rstep;
            src[i] = d < kept ? idx[d] : -1;
        }
    };
    auto moves = [&](int32_t c, int i, int32_t sr) {
        const int32_t d = c * rpc + rr0 + i * rstep;
        return sr > d && sr < n;
    };
    auto load_data = [&](int32_t c, const int32_t (&src)[IPT], T (&buf)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i)
            if (moves(c, i, src[i]))
                buf[i] = __builtin_nontemporal_load(reinterpret_cast<const T*>(ra(src[i]) + coff));
    };
    auto store_data = [&](int32_t c, const int32_t (&src)[IPT], const T (&buf)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i)
            if (moves(c, i, src[i])) {
                const int32_t d = c * rpc + rr0 + i * rstep;
                __builtin_nontemporal_store(buf[i], reinterpret_cast<T*>(ra(d) + coff));
            }
    };
    auto finish_loads = [&](T (&buf)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) wait_loaded(buf[i]);
        __syncthreads();  // every source of this chunk has been read
    };

    int32_t sA[IPT], sB[IPT];
    T bA[IPT], bB[IPT];
    load_idx(0, sA);
    load_data(0, sA, bA);
    load_idx(1, sB);
    for (int32_t c = 0; c < nchunks; c += 2) {
        load_data(c + 1, sB, bB);  // read-ahead: sources of c+1 lie above chunk c's rows
        finish_loads(bA);
        store_data(c, sA, bA);
        load_idx(c + 2, sA);
        if (c + 1 >= nchunks) break;
        load_data(c + 2, sA, bA);
        finish_loads(bB);
        store_data(c + 1, sB, bB);
        load_idx(c + 3, sB);
    }
}

// Buffer-resource loads/stores: an offset at or past the resource size is
// dropped by the hardware (loads return 0), so items that do not move get an
// out-of-range offset instead of a branch.  Straight-line code lets the
// compiler wait for exactly the loads a chunk needs (not for the read-ahead).
constexpr uint32_t kOOB = 0x80000000u;

template <int CW>
struct BufIO;
template <>
struct BufIO<16> {
    using T = u32x4;
    static __device__ __forceinline__ T ld(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
    }
    static __device__ __forceinline__ void st(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, o, 0, 0);
    }
};
template <>
struct BufIO<8> {
    using T = u32x2;
    static __device__ __forceinline__ T ld(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
    }
    static __device__ __forceinline__ void st(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, o, 0, 0);
    }
};
template <>
struct BufIO<4> {
    using T = uint32_t;
    static __device__ __forceinline__ T ld(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
    }
    static __device__ __forceinline__ void st(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, o, 0, 0);
    }
};
template <>
struct BufIO<2> {
    using T = unsigned short;
    static __device__ __forceinline__ T ld(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
    }
    static __device__ __forceinline__ void st(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, o, 0, 0);
    }
};

// Contiguous cache: the unit's rows are one buffer of cap * rb bytes.
template <int CW, int IPT, typename IdxT>
__device__ __forceinline__ void compact_slice_buf(__amdgpu_buffer_rsrc_t rs, int rb, int off,
                                                  int lg, IdxT idx, int32_t kept, int32_t n) {
    using IO = BufIO<CW>;
    using T = typename IO::T;
    const int col = threadIdx.x & ((1 << lg) - 1);
    const int rr0 = threadIdx.x >> lg;
    const int rstep = kCompactThreads >> lg;
    const int rpc = IPT * rstep;
    const int32_t nchunks = (kept + rpc - 1) / rpc;
    const uint32_t coff = (uint32_t)(off + col * CW);

    // byte offsets of this thread's sources (OOB if the row does not move)
    auto src_offs = [&](int32_t c, uint32_t (&so)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int32_t d = c * rpc + rr0 + i * rstep;
            const int32_t v = idx[d < kept ? d : kept - 1];  // branch-free read
            const int32_t sr = d < kept ? v : -1;
            so[i] = (sr > d && sr < n) ? (uint32_t)sr * (uint32_t)rb + coff : kOOB;
        }
    };
    // A buffer's data and offset registers stay live from its stores until it
    // is reloaded (the empty asm uses below): otherwise the register allocator
    // reuses them right after the stores for temporaries, and protecting the
    // in-flight store data makes the compiler wait for everything issued
    // before those stores -- including the read-ahead loads.
    auto load = [&](int32_t c, uint32_t (&so)[IPT], T (&buf)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            asm volatile("" ::"v"(buf[i]));
            asm volatile("" ::"v"(so[i]));
        }
        src_offs(c, so);
#pragma unroll
        for (int i = 0; i < IPT; ++i) buf[i] = IO::ld(rs, so[i]);
    };
    auto drain_store = [&](int32_t c, uint32_t (&so)[IPT], T (&buf)[IPT]) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) wait_loaded(buf[i]);
        __syncthreads();  // every source of chunk c has been read
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int32_t d = c * rpc + rr0 + i * rstep;
            so[i] = so[i] == kOOB ? kOOB : (uint32_t)d * (uint32_t)rb + coff;
            IO::st(buf[i], rs, so[i]);
        }
    };

    // Four buffers, two chunks of read-ahead: chunk c+2 is loaded into the
    // buffer whose stores (chunk c-2) were issued two steps earlier.
    uint32_t o0[IPT] = {}, o1[IPT] = {}, o2[IPT] = {}, o3[IPT] = {};
    T b0[IPT] = {}, b1[IPT] = {}, b2[IPT] = {}, b3[IPT] = {};
    load(0, o0, b0);
    load(1, o1, b1);
    for (int32_t c = 0; c < nchunks; c += 4) {
        load(c + 2, o2, b2);
        drain_store(c, o0, b0);
        if (c + 1 >= nchunks) break;
        load(c + 3, o3, b3);
        drain_store(c + 1, o1, b1);
        if (c + 2 >= nchunks) break;
        load(c + 4, o0, b0);
        drain_store(c + 2, o2, b2);
        if (c + 3 >= nchunks) break;
        load(c + 5, o1, b1);
        drain_store(c + 3, o3, b3);
    }
}

template <bool PAGED, bool IDX_LDS>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CacheView cv, Batch b,
                                                                   SliceSet ss,
                                                                   const int32_t* __restrict__ keep,
                                                                   int n_units) {
    extern __shared__ int32_t idx_sh[];
    // Workgroups are dealt to the 8 XCDs round-robin by id; give all slices of a
    // unit ids that are equal mod 8 and adjacent, so they share one L2 and run
    // together (the halves of a row are then fetched from HBM once).
    const int w = blockIdx.x;
    const int q = w >> 3;
    const int u = (q / ss.n) * 8 + (w & 7);
    if (u >= n_units) return;
    const Slice sl = ss.s[q % ss.n];
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const int32_t kept = (int32_t)sd.kept, n = (int32_t)sd.n;
    if (kept <= 0 || kept >= n) return;  // nothing evicted: no row moves
    const int32_t* idx = keep + sd.keep_off + ((int64_t)id.l * cv.Hkv + id.g) * kept;
    uint8_t* arr = sl.arr == 0 ? cv.k : (sl.arr == 1 ? cv.v : reinterpret_cast<uint8_t*>(cv.pos));
    RowAddr<PAGED> ra;
    ra.rb = sl.arr == 0 ? cv.kb : (sl.arr == 1 ? cv.vb : 4);
    if constexpr (!PAGED) {
        ra.base = arr + ((int64_t)id.l * cv.Hkv + id.g) * cv.cap * ra.rb;
        ra.bt = nullptr;
        ra.blk_stride = 0;
    } else {
        ra.base = arr + ((int64_t)id.l * cv.n_blocks * cv.Hkv + id.g) * kBlockRows * ra.rb;
        ra.bt = cv.bt + (int64_t)id.seq * cv.max_blocks;
        ra.blk_stride = (int64_t)cv.Hkv * kBlockRows * ra.rb;
    }
    auto run = [&](auto ix) {
        if constexpr (!PAGED) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                ra.base, (short)0, (int)(cv.cap * ra.rb), 0x00020000);
            switch (sl.cw) {
                case 16: compact_slice_buf<16, 4>(rs, ra.rb, sl.off, sl.lg, ix, kept, n); break;
                case 8: compact_slice_buf<8, 8>(rs, ra.rb, sl.off, sl.lg, ix, kept, n); break;
                case 4: compact_slice_buf<4, 8>(rs, ra.rb, sl.off, sl.lg, ix, kept, n); break;
                default: compact_slice_buf<2, 8>(rs, ra.rb, sl.off, sl.lg, ix, kept, n); break;
            }
            return;
        }
        switch (sl.cw) {
            case 16: compact_slice<16, 8, PAGED>(ra, sl.off, sl.lg, ix, kept, n); break;
            case 8: compact_slice<8, 8, PAGED>(ra, sl.off, sl.lg, ix, kept, n); break;
            case 4: compact_slice<4, 16, PAGED>(ra, sl.off, sl.lg, ix, kept, n); break;
            default: compact_slice<2, 16, PAGED>(ra, sl.off, sl.lg, ix, kept, n); break;
        }
    };
    if constexpr (IDX_LDS) {
        // Stage the unit's kept indices once (coalesced), so that no chunk waits
        // on a dependent index load from memory.
        for (int32_t i = threadIdx.x; i < kept; i += kCompactThreads) idx_sh[i] = idx[i];
        __syncthreads();
        run(static_cast<const int32_t*>(idx_sh));
    } else {
        run(idx);
    }
}

// Split a row of rb bytes into slices of a power-of-two number of items of the
// widest aligned chunk, at most 128 bytes per slice.
#ifndef TRIA_SLICE_BYTES
#define TRIA_SLICE_BYTES 128
#endif
void add_slices(SliceSet& ss, int arr, int rb) {
    int cw = 16;
    while (cw > 2 && (rb % cw) != 0) cw >>= 1;
    int items = rb / cw, off = 0;
    const int max_items = TRIA_SLICE_BYTES / cw > 0 ? TRIA_SLICE_BYTES / cw : 1;
    while (items > 0 && ss.n < kMaxSlices) {
        int take = max_items;
        while (take > items) take >>= 1;
        int lg = 0;
        while ((1 << lg) < take) ++lg;
        ss.s[ss.n++] = Slice{arr, off, cw, lg};
        off += take * cw;
        items -= take;
    }
}

}  // namespace

hipError_t launch_compact(const CacheView& cv, const Batch& b, int n_units,
                          const int32_t* keep, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    SliceSet ss;
    ss.n = 0;
    add_slices(ss, 0, cv.kb);
    add_slices(ss, 1, cv.vb);
    add_slices(ss, 2, 4);
    int64_t max_kept = 0;
    for (int i = 0; i < b.n_seq; ++i) max_kept = b.seq[i].kept > max_kept ? b.seq[i].kept : max_kept;
    const size_t lds = (size_t)max_kept * sizeof(int32_t);
    const dim3 grid(ss.n * ((n_units + 7) / 8) * 8), blk(kCompactThreads);
    if (lds <= kMaxIdxLds) {
        if (cv.bt)
            hipLaunchKernelGGL((compact_kernel<true, true>), grid, blk, lds, s, cv, b, ss, keep, n_units);
        else
            hipLaunchKernelGGL((compact_kernel<false, true>), grid, blk, lds, s, cv, b, ss, keep, n_units);
    } else {
        if (cv.bt)
            hipLaunchKernelGGL((compact_kernel<true, false>), grid, blk, 0, s, cv, b, ss, keep, n_units);
        else
            hipLaunchKernelGGL((compact_kernel<false, false>), grid, blk, 0, s, cv, b, ss, keep, n_units);
    }
    return hipGetLastError();
}

}  // namespace tria
