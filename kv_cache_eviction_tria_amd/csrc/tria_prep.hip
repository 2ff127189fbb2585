// prep: per-unit coefficient table of the score.
//
// The score's trigonometric part is sum_f Re(C_{j,f} conj(K_f)) with
// C_{j,f} = qbar_{j,f} * A_f and A_f the mean over the offset set D of
// exp(i omega_f (p + delta)) ("TriAttention Native C++ Worklog", section
// "Phase 9: final root cause - native scorer used the wrong formulation":
// the phase is applied on the query side only).  p is the absolute position
// stored with the unit's newest row (same worklog, section "2026-04-18:
// later-compaction absolute-position bug isolated and fixed"), read here on
// the device so that no host round trip is needed.
//
// A_f factors exactly as exp(i omega_f p) * M_f with M_f the mean of
// exp(i omega_f delta), which the host computes once in fp64; this kernel
// evaluates the remaining phase in fp64 (omega_0 p reaches ~1e5 rad, beyond
// what fp32 can resolve) and rounds the products to the table format the
// score kernel reads from scalar registers.
#include "tria_internal.h"

namespace tria {

namespace {

constexpr int kPrepThreads = 256;
// |v| <= 127 * (2^24 + 2^16 + 2^8 + 1) has four balanced base-256 digits in [-128, 127]
constexpr int64_t kDigitMax = 2139062143;
constexpr int kPrepHeadDims = 2048;  // trig coefficients of a batch of heads in LDS

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    CacheView cv, Batch b, int k_type, int G, int hd, const float* __restrict__ q_re,
    const float* __restrict__ q_im, const float* __restrict__ norm_w,
    const double* __restrict__ omega, const double* __restrict__ m_re,
    const double* __restrict__ m_im, int32_t* __restrict__ coef) {
    const int u = blockIdx.x;
    const UnitId id = unit_id(cv, u);
    const SeqDesc& sd = b.seq[id.seq];
    const CoefGeom cg = coef_geom(k_type, hd, G);
    const int F = cg.F;
    int32_t* out = coef + coef_unit(b, cv, id) * cg.words;
    float* outf = reinterpret_cast<float*>(out);
    if (sd.n <= 0) return;

    __shared__ double a_re[128], a_im[128];
    // a batch of heads' trig coefficients, head jj at [jj * hd]: [Re C_0..F-1, Im C_0..F-1]
    __shared__ double c_all[kPrepHeadDims];
    __shared__ float sig_sh[kPrepHeadDims / 32];

    const int64_t p = cv.pos[row_index(cv, id, sd.n - 1)];
    for (int f = threadIdx.x; f < F; f += kPrepThreads) {
        double s, c;
        sincos(omega[f] * (double)p, &s, &c);
        a_re[f] = c * m_re[f] - s * m_im[f];
        a_im[f] = c * m_im[f] + s * m_re[f];
    }
    __syncthreads();

    const int Hq = cv.Hkv * G;
    const int64_t stat0 = ((int64_t)(b.coef_l0 + id.l) * Hq + (int64_t)id.g * G) * F;

    if (k_type == TRIA_KV_F16) {
        for (int i = threadIdx.x; i < F * G; i += kPrepThreads) {
            const int j = i / F, f = i - j * F;
            const int j0 = subgroup_start(G, j), gt = subgroup_size(G, j0);
            const int o = (j0 * F + f * gt + (j - j0)) * 3;
            const int64_t s = stat0 + (int64_t)j * F + f;
            const double qr = q_re[s], qi = q_im[s];
            outf[o + 0] = (float)(qr * a_re[f] - qi * a_im[f]);
            outf[o + 1] = (float)(qr * a_im[f] + qi * a_re[f]);
            outf[o + 2] = norm_w[s];
        }
        return;
    }

    if (cg.q8_f16) {
        // q8_0, hd % 128 == 0: each head's trig coefficients scaled by 2^e (its
        // largest magnitude into [2^14, 2^15), inside the fp16 range with room
        // below) and split into fp16 hi + lo, about 22 significant bits of every
        // coefficient whatever its size against the others; osc = 2^-e undoes
        // the scale.  Coefficients are placed at the byte positions of the
        // stored row (zero at the block scales), four per stored word.
        const int W = cg.W, RB = 34 * cg.NB;
        __shared__ int ex_sh[64];
        // each head's largest |coefficient| (NaN left out), one (head, pair) per
        // thread: non-negative doubles order as their bit patterns
        __shared__ unsigned long long mx_sh[64];
        for (int j = threadIdx.x; j < G; j += kPrepThreads) mx_sh[j] = 0ull;
        __syncthreads();
        for (int i = threadIdx.x; i < F * G; i += kPrepThreads) {
            const int j = i / F, f = i - j * F;
            const int64_t s = stat0 + (int64_t)j * F + f;
            const double qr = q_re[s], qi = q_im[s];
            const double v = fmax(fabs(qr * a_re[f] - qi * a_im[f]), fabs(qr * a_im[f] + qi * a_re[f]));
            if (v > 0.0) atomicMax(&mx_sh[j], (unsigned long long)__double_as_longlong(v));
        }
        __syncthreads();
        for (int j = threadIdx.x; j < G; j += kPrepThreads) {
            const double m = __longlong_as_double((long long)mx_sh[j]);
            int ex = 0;
            if (m > 0.0 && isfinite(m)) ex = 14 - ilogb(m);
            ex = ex > 100 ? 100 : (ex < -100 ? -100 : ex);
            ex_sh[j] = ex;
            outf[cg.osc_off + j] = ldexpf(1.0f, -ex);
        }
        for (int i = threadIdx.x; i < F * G; i += kPrepThreads) {
            const int j = i / F, f = i - j * F;
            const int j0 = subgroup_start(G, j), gt = subgroup_size(G, j0);
            outf[cg.w_off + j0 * F + f * gt + (j - j0)] = norm_w[stat0 + (int64_t)j * F + f];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < G * W; i += kPrepThreads) {
            const int j = i / W, k = i - j * W;
            const int64_t s0 = stat0 + (int64_t)j * F;
            uint32_t hw[2] = {0u, 0u}, lw[2] = {0u, 0u};
            for (int b4 = 0; b4 < 4; ++b4) {
                const int byte = 4 * k + b4;
                if (byte >= RB) continue;
                const int blk = byte / 34, o = byte - 34 * blk;
                if (o < 2) continue;  // scale bytes: zero coefficients
                const int d = 32 * blk + (o - 2);
                const int f = d < F ? d : d - F;
                const double qr = q_re[s0 + f], qi = q_im[s0 + f];
                const double c = d < F ? qr * a_re[f] - qi * a_im[f] : qr * a_im[f] + qi * a_re[f];
                const float x = (float)ldexp(c, ex_sh[j]);
                const _Float16 h = (_Float16)x;
                const _Float16 l = (_Float16)(x - (float)h);
                hw[b4 >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, h) << (16 * (b4 & 1));
                lw[b4 >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, l) << (16 * (b4 & 1));
            }
            out[cg.hi_off + (j * W + k) * 2 + 0] = (int32_t)hw[0];
            out[cg.hi_off + (j * W + k) * 2 + 1] = (int32_t)hw[1];
            out[cg.lo_off + (j * W + k) * 2 + 0] = (int32_t)lw[0];
            out[cg.lo_off + (j * W + k) * 2 + 1] = (int32_t)lw[1];
        }
        return;
    }

    // q8_0: trig coefficients quantised per (head, 32-dim block) to 32-bit integers
    // v = round(c / sig), sig = (block max) / kDigitMax, split into four balanced
    // base-256 digits so that the score kernel can accumulate sum_d q_d * v_d
    // with int8 products.  The error of a coefficient is at most sig / 2, about
    // 2^-32 of the block maximum: a coefficient 1e4 times smaller than its
    // block's largest still keeps about 18 significant bits (16-bit integers
    // kept 2 or 3, too few when the keys are large on exactly those dimensions).
    // The heads are taken kPrepHeadDims / hd at a time, each phase over all of
    // them at once.
    const int NB = cg.NB, W = cg.W, RB = 34 * NB;
    const int HB = kPrepHeadDims / hd;  // heads per batch (hd <= 256: at least 8)
    for (int jb = 0; jb < G; jb += HB) {
        const int nh = G - jb < HB ? G - jb : HB;
        for (int i = threadIdx.x; i < nh * F; i += kPrepThreads) {
            const int jj = i / F, f = i - jj * F, j = jb + jj;
            const int64_t s0 = stat0 + (int64_t)j * F;
            const int j0 = subgroup_start(G, j), gt = subgroup_size(G, j0);
            const double qr = q_re[s0 + f], qi = q_im[s0 + f];
            c_all[jj * hd + f] = qr * a_re[f] - qi * a_im[f];
            c_all[jj * hd + f + F] = qr * a_im[f] + qi * a_re[f];
            outf[cg.w_off + j0 * F + f * gt + (j - j0)] = norm_w[s0 + f];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nh * NB; i += kPrepThreads) {
            const int jj = i / NB, blk = i - jj * NB;
            double m = 0.0;
            for (int t = 0; t < 32; ++t) m = fmax(m, fabs(c_all[jj * hd + 32 * blk + t]));
            const float sg = (float)(m / (double)kDigitMax);
            sig_sh[jj * NB + blk] = sg;
            outf[cg.sig_off + (jb + jj) * NB + blk] = sg;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nh * W; i += kPrepThreads) {
            const int jj = i / W, k = i - jj * W, j = jb + jj;
            uint32_t dw[kCoefDigits] = {};
            for (int b4 = 0; b4 < 4; ++b4) {
                const int byte = 4 * k + b4;
                if (byte >= RB) continue;
                const int blk = byte / 34, o = byte - 34 * blk;
                if (o < 2) continue;  // scale bytes get zero digits
                const float sg = sig_sh[jj * NB + blk];
                int64_t v = 0;
                if (sg > 0.0f) {
                    const double t = c_all[jj * hd + 32 * blk + (o - 2)] / (double)sg;
                    v = llrint(t);
                    v = v > kDigitMax ? kDigitMax : (v < -kDigitMax ? -kDigitMax : v);
                }
                for (int dg = 0; dg < kCoefDigits; ++dg) {
                    const int64_t d = ((v + 128) & 255) - 128;  // balanced digit
                    dw[dg] |= (uint32_t)(d & 255) << (8 * b4);
                    v = (v - d) / 256;
                }
            }
            for (int dg = 0; dg < kCoefDigits; ++dg)
                out[cg.digit_off + (dg * G + j) * W + k] = (int32_t)dw[dg];
        }
        __syncthreads();  // the batch's tables are rewritten by the next one
    }
}

}  // namespace

hipError_t launch_prep(const CacheView& cv, const Batch& b, int n_units, int k_type, int G,
                       int hd, const float* q_re, const float* q_im, const float* w,
                       const double* omega, const double* m_re, const double* m_im,
                       int32_t* coef, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel, dim3(n_units), dim3(kPrepThreads), 0, s, cv, b, k_type, G, hd,
                       q_re, q_im, w, omega, m_re, m_im, coef);
    return hipGetLastError();
}

}  // namespace tria
