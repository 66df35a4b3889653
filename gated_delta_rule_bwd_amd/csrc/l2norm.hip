// l2norm.hip -- gfx950 kernels of the per-(token, head) L2 normalisation of q and k that sits
// between the short convolution and the gated delta rule (meTile, "Training kernels and
// gradients", section "Recurrent delta attention": the normalisation is a step of its own,
// outside the recurrence), and of its backward:
//   n = sqrt(sum_i x_i^2 + eps),  y = x / n,  dx = dy / n - x (x . dy) / n^3.
//
// A group of LPR lanes owns one row of W floats (chunks of V = 4 floats when every row start is
// 16-byte aligned, else V = 1; a lane holds two chunks, up to 16 floats for the widest rows).
// The row sums are a butterfly over the group, so every lane of it ends with the same bits.
// HBM-bound: each row is read and written once.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int BLOCK = 256;

template <int V>
__device__ __forceinline__ void ldc(const float *p, float *x) {
    if constexpr (V == 4) {
        const float4 t = *reinterpret_cast<const float4 *>(p);
        x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else {
        x[0] = *p;
    }
}
// outputs are written once and never re-read here: nontemporal stores leave L2 to the inputs
typedef float f4v __attribute__((ext_vector_type(4)));
template <int V>
__device__ __forceinline__ void stc(float *p, const float *x) {
    if constexpr (V == 4) __builtin_nontemporal_store(f4v{x[0], x[1], x[2], x[3]}, reinterpret_cast<f4v *>(p));
    else __builtin_nontemporal_store(x[0], p);
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int V, int LPR, bool BWD>
__global__ void __launch_bounds__(BLOCK) l2norm_kernel(const NormArgs a) {
    constexpr int NCMAX = 16 / V;              // chunks per lane
    constexpr int RPB = BLOCK / LPR;           // rows per block and pass
    const int nch = a.W / V;
    const int nc = (nch + LPR - 1) / LPR;      // chunks this row needs per lane (<= NCMAX)
    const int sub = threadIdx.x % LPR;
    const int64_t rows = (int64_t)a.n_seqs * a.T * a.H;
    // the loop bound is uniform over the block, so every lane of a group takes part in the
    // shuffles; lanes past the last row work on a clamped row and store nothing
    for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < rows; r0 += (int64_t)gridDim.x * RPB) {
        const int64_t r = r0 + threadIdx.x / LPR;
        const bool live = r < rows;
        const int64_t rc = live ? r : rows - 1;
        const int64_t h = rc % a.H, t = (rc / a.H) % a.T, s = rc / ((int64_t)a.H * a.T);
        const float *xr = a.x + s * a.sx.seq + t * a.sx.tok + h * a.sx.head;
        float x[NCMAX * V], g[NCMAX * V];
        float ss = 0.f, xg = 0.f;
#pragma unroll
        for (int j = 0; j < NCMAX; ++j) {
            if (j < nc) {                       // uniform over the launch
                const int c = sub + j * LPR;
                const bool ok = c < nch;
                const int cc = ok ? c : nch - 1;
                ldc<V>(xr + (int64_t)cc * V, x + j * V);
                if constexpr (BWD) {
                    const float *gr = a.dy + s * a.sdy.seq + t * a.sdy.tok + h * a.sdy.head;
                    ldc<V>(gr + (int64_t)cc * V, g + j * V);
                }
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    x[j * V + e] = ok ? x[j * V + e] : 0.f;
                    ss = fmaf(x[j * V + e], x[j * V + e], ss);
                    if constexpr (BWD) {
                        g[j * V + e] = ok ? g[j * V + e] : 0.f;
                        xg = fmaf(x[j * V + e], g[j * V + e], xg);
                    }
                }
            }
        }
        ss = group_sum<LPR>(ss);
        if constexpr (BWD) xg = group_sum<LPR>(xg);
        const float n = sqrtf(ss + a.eps);
        float *orow = a.out + s * a.so.seq + t * a.so.tok + h * a.so.head;
        if constexpr (BWD) {
            const float inv = 1.f / n;
            const float coef = xg * (inv * inv * inv);
#pragma unroll
            for (int j = 0; j < NCMAX; ++j) {
                if (j < nc) {
#pragma unroll
                    for (int e = 0; e < V; ++e) x[j * V + e] = fmaf(g[j * V + e], inv, -x[j * V + e] * coef);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NCMAX; ++j) {
                if (j < nc) {
#pragma unroll
                    for (int e = 0; e < V; ++e) x[j * V + e] = x[j * V + e] / n;
                }
            }
        }
        if (live) {
#pragma unroll
            for (int j = 0; j < NCMAX; ++j) {
                const int c = sub + j * LPR;
                if (j < nc && c < nch) stc<V>(orow + (int64_t)c * V, x + j * V);
            }
        }
    }
}

template <int V, bool BWD>
hipError_t launch_v(const NormArgs &a, hipStream_t st) {
    const int64_t rows = (int64_t)a.n_seqs * a.T * a.H;
    if (rows <= 0) return hipSuccess;
    const int nch = a.W / V;
    // the fewest lanes (a power of two, at most 64) that hold the row in two chunks each: two
    // loads in flight per lane and tensor measured faster than one (more rows per wave) or
    // four (fewer waves)
    int lpr = 1;
    while (lpr < 64 && 2 * lpr < nch) lpr <<= 1;
    if ((nch + lpr - 1) / lpr > 16 / V) return hipErrorInvalidValue;
    const int64_t rpb = BLOCK / lpr;
    int64_t blocks = (rows + rpb - 1) / rpb;
    if (blocks > 65535) blocks = 65535;
    void *params[] = {const_cast<NormArgs *>(&a)};
    const void *fn = nullptr;
    switch (lpr) {
#define GDN_L(l) case l: fn = (const void *)l2norm_kernel<V, l, BWD>; break;
        GDN_L(1) GDN_L(2) GDN_L(4) GDN_L(8) GDN_L(16) GDN_L(32) GDN_L(64)
#undef GDN_L
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(BLOCK), params, 0, st);
}

bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool st4(const gdn_strides &s) { return s.seq % 4 == 0 && s.tok % 4 == 0 && s.head % 4 == 0; }

}  // namespace

hipError_t launch_l2norm(const NormArgs &a, bool bwd, hipStream_t st) {
    const bool vec = a.W % 4 == 0 && al16(a.x) && al16(a.out) && st4(a.sx) && st4(a.so) &&
                     (!bwd || (al16(a.dy) && st4(a.sdy)));
    if (bwd) return vec ? launch_v<4, true>(a, st) : launch_v<1, true>(a, st);
    return vec ? launch_v<4, false>(a, st) : launch_v<1, false>(a, st);
}

}  // namespace gdn
