// Calibration statistics on the GPU (llama.cpp page "TriAttention KV-Cache
// Eviction (--triattention)", section 2, "Generating a .tria file": the
// generator hooks each layer's pre-RoPE query tensor during forward passes and
// accumulates per-head statistics; section 5, "Phase C", names the per-head
// q_mean / q_abs arrays the scorer uploads).  Per layer, query head h and
// frequency pair f, with q_f = q[f] + i q[f + hd/2] (NEOX halves):
//   sums over tokens of Re q_f, Im q_f and |q_f|  (fp64)
// and, at the end,
//   q_mean = sums / T,  q_abs = sum|q_f| / T,  w = q_abs - |q_mean|
// (w: the norm-term weight; zero when every token's pair points the same way).
//
// Streaming: tria_calib_add takes one layer's query rows of one batch in one
// launch.  The layer keeps kCalSlots fp64 accumulators per (pair, sum); the
// tokens are cut into chunks of 32, and workgroup (column, y) covers 256
// (head, pair) slots of chunks y, y + S, y + 2S, ... (S = min(chunks,
// kCalSlots), and fewer when one call adds many layers, so that a launch
// holds about kCalTargetBlocks workgroups: each slot's read-modify-write and
// the finish's read of it are then spread over more tokens): four consecutive
// pairs per lane (one 16-byte load of the real
// halves and one of the imaginary halves per token; consecutive lanes read
// consecutive bytes), the tokens dealt over its four wavefronts and their sums
// combined in LDS in a fixed order, then added into accumulator slot y -- which
// no other workgroup of the launch touches, and adds on one stream run in
// order.  tria_calib_finish adds a layer's slots in slot order (the slots any
// call used).  So every sum is formed in an order fixed by the call sequence,
// never by scheduling.  The
// pair magnitude is formed in fp32 (the inputs are at most fp32), the sums in
// fp64.
#include <new>

#include "tria_internal.h"

namespace {

constexpr int kCalThreads = 256;
constexpr int kCalTok = 32;    // tokens per chunk
constexpr int kCalSlots = 64;  // accumulator slots per layer (workgroup rows of a launch)
constexpr int kCalMaxLayers = 128;  // layers finished per launch
constexpr int64_t kCalTargetBlocks = 4608;  // workgroups a many-layer add aims for

template <typename QT>
__device__ __forceinline__ float q_load(const QT* p);
template <>
__device__ __forceinline__ float q_load<float>(const float* p) {
    return *p;
}
template <>
__device__ __forceinline__ float q_load<_Float16>(const _Float16* p) {
    return (float)*p;
}
template <>
__device__ __forceinline__ float q_load<uint16_t>(const uint16_t* p) {
    return __uint_as_float((uint32_t)*p << 16);  // bfloat16: the top half of a float
}

// Four consecutive values of a row as floats (one 16-byte load for fp32,
// 8 bytes for the 16-bit types).  Every query value is read once: streaming
// (non-temporal) loads, 10 % faster per sample on MI355X.
template <typename QT>
__device__ __forceinline__ float4 q_load4(const QT* p);
template <>
__device__ __forceinline__ float4 q_load4<float>(const float* p) {
    typedef float f4e __attribute__((ext_vector_type(4)));
    const f4e t = __builtin_nontemporal_load(reinterpret_cast<const f4e*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
template <>
__device__ __forceinline__ float4 q_load4<_Float16>(const _Float16* p) {
    typedef unsigned int u2e __attribute__((ext_vector_type(2)));
    const u2e u = __builtin_nontemporal_load(reinterpret_cast<const u2e*>(p));
    return make_float4((float)__builtin_bit_cast(_Float16, (uint16_t)(u.x & 0xffffu)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x >> 16)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y & 0xffffu)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y >> 16)));
}
template <>
__device__ __forceinline__ float4 q_load4<uint16_t>(const uint16_t* p) {
    typedef unsigned int u2e __attribute__((ext_vector_type(2)));
    const u2e u = __builtin_nontemporal_load(reinterpret_cast<const u2e*>(p));
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

constexpr int kCalWaves = kCalThreads / 64;

// grid (pair blocks of 256, S accumulator slots).  Lane j of every wavefront
// takes pairs 4j .. 4j+3 of the block's 256 (F % 4 == 0: never across a head)
// and wavefront w the tokens t0 + w, t0 + w + 4, ... of the block's chunks
// (y, y + S, ...); the four wavefronts' sums are added in LDS in a fixed order
// and then into slot y: slot[(y * HF + pair) * 3 + {re, im, abs}].
template <typename QT>
__global__ __launch_bounds__(kCalThreads) void calib_partial4_kernel(
    const QT* __restrict__ q, int64_t T, int64_t stride, int F, int hd, int HF,
    double* __restrict__ slot, int64_t q_layer, int64_t slot_layer) {
    __shared__ double sums[kCalWaves][12][64];
    q += (int64_t)blockIdx.z * q_layer;  // layer z of the call
    slot += (int64_t)blockIdx.z * slot_layer;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p0 = blockIdx.x * 256 + 4 * lane;
    const bool in = p0 < HF;
    const int h = p0 / F, f = p0 - h * F;
    const QT* base = q + (int64_t)h * hd + f;
    double sr[4] = {0.0, 0.0, 0.0, 0.0}, si[4] = {0.0, 0.0, 0.0, 0.0}, sa[4] = {0.0, 0.0, 0.0, 0.0};
    for (int64_t t0 = (int64_t)blockIdx.y * kCalTok; in && t0 < T;
         t0 += (int64_t)gridDim.y * kCalTok) {
        const int64_t t1 = t0 + kCalTok < T ? t0 + kCalTok : T;
        for (int64_t t = t0 + wave; t < t1; t += kCalWaves) {
            const float4 re = q_load4<QT>(base + t * stride);
            const float4 im = q_load4<QT>(base + t * stride + F);
            const float r[4] = {re.x, re.y, re.z, re.w}, m[4] = {im.x, im.y, im.z, im.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sr[k] += (double)r[k];
                si[k] += (double)m[k];
                sa[k] += (double)__builtin_amdgcn_sqrtf(fmaf(r[k], r[k], m[k] * m[k]));
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        sums[wave][3 * k][lane] = sr[k];
        sums[wave][3 * k + 1][lane] = si[k];
        sums[wave][3 * k + 2][lane] = sa[k];
    }
    __syncthreads();
    if (wave == 0 && in) {
        double* out = slot + ((int64_t)blockIdx.y * HF + p0) * 3;
#pragma unroll
        for (int j = 0; j < 12; ++j) {
            double s = sums[0][j][lane];
#pragma unroll
            for (int w = 1; w < kCalWaves; ++w) s += sums[w][j][lane];
            out[j] += s;
        }
    }
}

// Any F: one pair per thread, chunks y, y + S, ... into slot y.
template <typename QT>
__global__ __launch_bounds__(kCalThreads) void calib_partial_kernel(
    const QT* __restrict__ q, int64_t T, int64_t stride, int F, int hd, int HF,
    double* __restrict__ slot, int64_t q_layer, int64_t slot_layer) {
    q += (int64_t)blockIdx.z * q_layer;  // layer z of the call
    slot += (int64_t)blockIdx.z * slot_layer;
    const int i = blockIdx.x * kCalThreads + threadIdx.x;
    if (i >= HF) return;
    const int h = i / F, f = i - h * F;
    const QT* base = q + (int64_t)h * hd + f;
    double sr = 0.0, si = 0.0, sa = 0.0;
    for (int64_t t0 = (int64_t)blockIdx.y * kCalTok; t0 < T; t0 += (int64_t)gridDim.y * kCalTok) {
        const int64_t t1 = t0 + kCalTok < T ? t0 + kCalTok : T;
        for (int64_t t = t0; t < t1; ++t) {
            const float re = q_load<QT>(base + t * stride);
            const float im = q_load<QT>(base + t * stride + F);
            sr += (double)re;
            si += (double)im;
            sa += (double)__builtin_amdgcn_sqrtf(fmaf(re, re, im * im));
        }
    }
    double* out = slot + ((int64_t)blockIdx.y * HF + i) * 3;
    out[0] += sr;
    out[1] += si;
    out[2] += sa;
}

// Token counts of up to kCalMaxLayers layers, passed by value.
struct CalCounts {
    int64_t n[kCalMaxLayers];
    int slots[kCalMaxLayers];  // accumulator slots in use
};

// Outputs of layers l0 .. l0 + gridDim.y - 1 from their sums (zeros for a
// layer with no tokens).
__global__ __launch_bounds__(kCalThreads) void calib_finish_kernel(const double* __restrict__ acc,
                                                                   int HF, int l0, CalCounts cnt,
                                                                   float* q_re, float* q_im,
                                                                   float* q_abs, float* w) {
    const int i = blockIdx.x * kCalThreads + threadIdx.x;
    if (i >= HF) return;
    const int l = l0 + (int)blockIdx.y;
    const int64_t count = cnt.n[blockIdx.y];
    const int64_t o = (int64_t)l * HF + i;
    // the layer's slots, in slot order
    const double* a = acc + ((int64_t)l * kCalSlots * HF + i) * 3;
    double sr = 0.0, si = 0.0, sa = 0.0;
    for (int y = 0; y < cnt.slots[blockIdx.y]; ++y) {
        sr += a[(int64_t)y * HF * 3];
        si += a[(int64_t)y * HF * 3 + 1];
        sa += a[(int64_t)y * HF * 3 + 2];
    }
    const double inv = count > 0 ? 1.0 / (double)count : 0.0;
    const double mr = sr * inv, mi = si * inv, ma = sa * inv;
    q_re[o] = (float)mr;
    q_im[o] = (float)mi;
    if (q_abs) q_abs[o] = (float)ma;
    w[o] = (float)(ma - sqrt(mr * mr + mi * mi));
}

}  // namespace

struct tria_calib {
    int L, Hq, hd, F, HF;
    double* acc = nullptr;      // [L][kCalSlots][HF][3]
    int64_t* count = nullptr;   // host [L]
    int* slots = nullptr;       // host [L]: accumulator slots any add has used
};

extern "C" {

int tria_calib_create(tria_calib** out, int32_t n_layers, int32_t n_q_heads, int32_t head_dim) {
    if (!out) return TRIA_E_INVAL;
    *out = nullptr;
    if (n_layers < 1 || n_q_heads < 1) return TRIA_E_INVAL;
    if (head_dim < 2 || head_dim % 2 != 0 || head_dim > 1024) return TRIA_E_UNSUPPORTED;
    tria_calib* c = new (std::nothrow) tria_calib();
    if (!c) return TRIA_E_NOMEM;
    c->L = n_layers;
    c->Hq = n_q_heads;
    c->hd = head_dim;
    c->F = head_dim / 2;
    c->HF = n_q_heads * c->F;
    c->count = static_cast<int64_t*>(calloc((size_t)n_layers, sizeof(int64_t)));
    c->slots = static_cast<int*>(calloc((size_t)n_layers, sizeof(int)));
    const size_t bytes = (size_t)n_layers * kCalSlots * c->HF * 3 * sizeof(double);
    hipError_t e = c->count && c->slots ? hipMalloc(reinterpret_cast<void**>(&c->acc), bytes) : hipErrorOutOfMemory;
    if (e == hipSuccess) e = hipMemset(c->acc, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();  // zeroed before any stream's add
    if (e != hipSuccess) {
        tria_calib_free(c);
        return e == hipErrorOutOfMemory ? TRIA_E_NOMEM : TRIA_E_HIP;
    }
    *out = c;
    return TRIA_OK;
}

void tria_calib_free(tria_calib* c) {
    if (!c) return;
    if (c->acc) (void)hipFree(c->acc);
    free(c->count);
    free(c->slots);
    delete c;
}

int tria_calib_add_layers(tria_calib* c, int32_t layer0, int32_t n_layers, const void* q,
                          int32_t q_type, int64_t n_tokens, int64_t row_stride,
                          int64_t layer_stride, hipStream_t stream) {
    if (!c || !q || layer0 < 0 || n_layers < 1 || n_layers > c->L - layer0 || n_tokens < 0)
        return TRIA_E_INVAL;
    if (row_stride < (int64_t)c->Hq * c->hd) return TRIA_E_INVAL;
    if (n_tokens > INT64_MAX / row_stride) return TRIA_E_INVAL;  // rows past any address
    if (n_layers > 1 && layer_stride < n_tokens * row_stride) return TRIA_E_INVAL;
    if (n_layers > 65535) return TRIA_E_UNSUPPORTED;
    if (q_type != TRIA_Q_F32 && q_type != TRIA_Q_F16 && q_type != TRIA_Q_BF16)
        return TRIA_E_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(q) % (q_type == TRIA_Q_F32 ? 4 : 2) != 0) return TRIA_E_INVAL;
    if (n_tokens == 0) return TRIA_OK;
    const int64_t chunks = (n_tokens + kCalTok - 1) / kCalTok;
    double* slot = c->acc + (int64_t)layer0 * kCalSlots * c->HF * 3;
    const int64_t slot_layer = (int64_t)kCalSlots * c->HF * 3;
    const int64_t q_layer = n_layers > 1 ? layer_stride : 0;
    const bool vec = c->F % 4 == 0;
    // 16-byte (8-byte) loads need the rows aligned: the base and both strides
    const size_t esz = q_type == TRIA_Q_F32 ? 4 : 2;
    const bool aligned = (reinterpret_cast<uintptr_t>(q) % (4 * esz)) == 0 && row_stride % 4 == 0 &&
                         q_layer % 4 == 0;
    const int64_t cols = vec && aligned ? (c->HF + 255) / 256 : (c->HF + kCalThreads - 1) / kCalThreads;
    int64_t want = (kCalTargetBlocks + cols * n_layers - 1) / (cols * n_layers);
    want = want < kCalSlots ? want : kCalSlots;
    const unsigned S = (unsigned)(chunks < want ? chunks : want);
    // vector path: 256 pairs per block; scalar path: one pair per thread; one
    // grid layer per query layer
    const dim3 grid((unsigned)cols, S, (unsigned)n_layers);
    if (q_type == TRIA_Q_F32) {
        auto k = vec && aligned ? calib_partial4_kernel<float> : calib_partial_kernel<float>;
        hipLaunchKernelGGL(k, grid, dim3(kCalThreads), 0, stream, static_cast<const float*>(q),
                           n_tokens, row_stride, c->F, c->hd, c->HF, slot, q_layer, slot_layer);
    } else if (q_type == TRIA_Q_F16) {
        auto k = vec && aligned ? calib_partial4_kernel<_Float16> : calib_partial_kernel<_Float16>;
        hipLaunchKernelGGL(k, grid, dim3(kCalThreads), 0, stream, static_cast<const _Float16*>(q),
                           n_tokens, row_stride, c->F, c->hd, c->HF, slot, q_layer, slot_layer);
    } else {
        auto k = vec && aligned ? calib_partial4_kernel<uint16_t> : calib_partial_kernel<uint16_t>;
        hipLaunchKernelGGL(k, grid, dim3(kCalThreads), 0, stream, static_cast<const uint16_t*>(q),
                           n_tokens, row_stride, c->F, c->hd, c->HF, slot, q_layer, slot_layer);
    }
    if (hipGetLastError() != hipSuccess) return TRIA_E_HIP;
    for (int i = 0; i < n_layers; ++i) {
        c->count[layer0 + i] += n_tokens;
        if ((int)S > c->slots[layer0 + i]) c->slots[layer0 + i] = (int)S;
    }
    return TRIA_OK;
}

int tria_calib_add(tria_calib* c, int32_t layer, const void* q, int32_t q_type, int64_t n_tokens,
                   int64_t row_stride, hipStream_t stream) {
    return tria_calib_add_layers(c, layer, 1, q, q_type, n_tokens, row_stride, 0, stream);
}

int64_t tria_calib_tokens(const tria_calib* c, int32_t layer) {
    if (!c || layer < 0 || layer >= c->L) return TRIA_E_INVAL;
    return c->count[layer];
}

int tria_calib_finish(tria_calib* c, float* q_re, float* q_im, float* q_abs, float* norm_w,
                      hipStream_t stream) {
    if (!c || !q_re || !q_im || !norm_w) return TRIA_E_INVAL;
    const unsigned blocks = (unsigned)((c->HF + kCalThreads - 1) / kCalThreads);
    for (int l0 = 0; l0 < c->L; l0 += kCalMaxLayers) {
        const int nl = c->L - l0 < kCalMaxLayers ? c->L - l0 : kCalMaxLayers;
        CalCounts cnt;
        for (int j = 0; j < kCalMaxLayers; ++j) {
            cnt.n[j] = j < nl ? c->count[l0 + j] : 0;
            cnt.slots[j] = j < nl ? c->slots[l0 + j] : 0;
        }
        hipLaunchKernelGGL(calib_finish_kernel, dim3(blocks, (unsigned)nl), dim3(kCalThreads), 0,
                           stream, c->acc, c->HF, l0, cnt, q_re, q_im, q_abs, norm_w);
        if (hipGetLastError() != hipSuccess) return TRIA_E_HIP;
    }
    return TRIA_OK;
}

}  // extern "C"
