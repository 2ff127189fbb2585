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
// walks the destination rows in increasing chunks: it loads every source of a
// chunk into registers, passes a workgroup barrier, then stores the chunk.
// The sources of later chunks lie at or above their own destinations, i.e.
// above everything this chunk writes, so no later load can see a clobbered
// row, and no other workgroup touches this slice.  Rows whose source is the
// row itself are skipped, so a leading kept run costs nothing but its index
// read.  Slices of <= 128 bytes spread one unit over several workgroups.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kCompactThreads = 256;
constexpr int kItemsPerThread = 8;
constexpr int kMaxSlices = 16;

struct Slice {
    int32_t arr;    // 0 = K, 1 = V, 2 = positions
    int32_t off;    // byte offset of the slice in the row
    int32_t bytes;  // slice width
    int32_t cw;     // bytes moved per item: 2, 4, 8 or 16
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

template <int CW>
__device__ __forceinline__ void compact_slice(uint8_t* base, int rb, int off, int bytes,
                                              const CacheView& cv, const UnitId& id,
                                              const int32_t* __restrict__ idx, int64_t kept,
                                              int64_t n) {
    using T = typename Chunk<CW>::T;
    const int ipr = bytes / CW;  // items per row
    const int rows_per_chunk = (kCompactThreads * kItemsPerThread) / ipr;
    for (int64_t c0 = 0; c0 < kept; c0 += rows_per_chunk) {
        T buf[kItemsPerThread];
        T* dst[kItemsPerThread];
        bool mv[kItemsPerThread];
#pragma unroll
        for (int i = 0; i < kItemsPerThread; ++i) {
            const int item = threadIdx.x + i * kCompactThreads;
            const int rr = item / ipr;
            const int col = item - rr * ipr;
            const int64_t d = c0 + rr;
            mv[i] = false;
            dst[i] = nullptr;
            if (rr < rows_per_chunk && d < kept) {
                const int64_t src = idx[d];
                if (src > d && src < n) {
                    mv[i] = true;
                    const T* sp = reinterpret_cast<const T*>(base + row_index(cv, id, src) * rb + off) + col;
                    buf[i] = __builtin_nontemporal_load(sp);
                    dst[i] = reinterpret_cast<T*>(base + row_index(cv, id, d) * rb + off) + col;
                }
            }
        }
        __syncthreads();  // every source of this chunk has been read
#pragma unroll
        for (int i = 0; i < kItemsPerThread; ++i)
            if (mv[i]) __builtin_nontemporal_store(buf[i], dst[i]);
    }
}

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CacheView cv, Batch b,
                                                                   SliceSet ss,
                                                                   const int32_t* __restrict__ keep) {
    const int u = blockIdx.y;
    const Slice sl = ss.s[blockIdx.x];
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const int64_t kept = sd.kept, n = sd.n;
    if (kept <= 0 || kept >= n) return;  // nothing evicted: no row moves
    const int32_t* idx = keep + sd.keep_off + ((int64_t)id.l * cv.Hkv + id.g) * kept;
    uint8_t* base = sl.arr == 0 ? cv.k : (sl.arr == 1 ? cv.v : reinterpret_cast<uint8_t*>(cv.pos));
    const int rb = sl.arr == 0 ? cv.kb : (sl.arr == 1 ? cv.vb : 4);
    switch (sl.cw) {
        case 16: compact_slice<16>(base, rb, sl.off, sl.bytes, cv, id, idx, kept, n); break;
        case 8: compact_slice<8>(base, rb, sl.off, sl.bytes, cv, id, idx, kept, n); break;
        case 4: compact_slice<4>(base, rb, sl.off, sl.bytes, cv, id, idx, kept, n); break;
        default: compact_slice<2>(base, rb, sl.off, sl.bytes, cv, id, idx, kept, n); break;
    }
}

void add_slices(SliceSet& ss, int arr, int rb) {
    int cw = 16;
    while (cw > 2 && (rb % cw) != 0) cw >>= 1;
    int ns = (rb + 64) / 128;  // ~128-byte slices
    if (ns < 1) ns = 1;
    const int items = rb / cw;
    const int per = (items + ns - 1) / ns;
    for (int i = 0, off = 0; off < rb && ss.n < kMaxSlices; ++i) {
        const int bytes = (rb - off) < per * cw ? (rb - off) : per * cw;
        ss.s[ss.n++] = Slice{arr, off, bytes, cw};
        off += bytes;
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
    hipLaunchKernelGGL(compact_kernel, dim3(ss.n, n_units), dim3(kCompactThreads), 0, s, cv, b, ss,
                       keep);
    return hipGetLastError();
}

}  // namespace tria
