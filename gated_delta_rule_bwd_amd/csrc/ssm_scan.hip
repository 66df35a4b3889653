// ssm_scan.hip -- gfx950 kernels of the selective state-space scan (Mamba-1: one decay per
// state; Mamba-2: one per head) and of its backward, the reverse recurrence (page "S1-24:
// chunked attention", the SSM_SCAN_BACK commit notes and the n_group fold).  Per sequence s,
// head h (group g = h / (H / G)), head element i and state n, with step d = softplus(dt) (or dt):
//   a = exp(d A[h, n]),  s[i, n] = a s[i, n] + d x[i] B[g, n],  y[i] = sum_n s[i, n] C[g, n].
//
// Layout of the work: a row is one (s, h, i); 16 lanes own a row, each lane NPL = N / 16
// consecutive state columns; a workgroup is 16 rows (4 per wave), which must lie in one group.
// The forward keeps the row's state in registers, writes y through a 16-lane DPP sum and saves
// the state before every 8-token window.  The backward walks the windows in reverse: it
// replays a window from its saved state into registers, then walks its tokens backwards with
// the state gradient gs in registers.  Row sums (dx, the decay term of ddt) are 16-lane DPP
// sums; the column sums of a token (dC = sum_i gy s, dB = sum_i gs d x over the 16 rows) are
// reduce-scattered over the four row groups of a wave with permlane swaps, summed over the four
// waves in LDS at the window's end and written as the segment's partial; a combine kernel adds
// the segments of each group (and the rows of each head for ddt) in a fixed order.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int WIN = 8;           // tokens per saved state / replay window
constexpr int ROWS = 16;         // rows per workgroup (one segment)

__device__ __forceinline__ int as_i(float v) { return __builtin_bit_cast(int, v); }
__device__ __forceinline__ float as_f(int v) { return __builtin_bit_cast(float, v); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}

template <int NPL>
__device__ __forceinline__ void ldv(const float *p, float (&v)[NPL]) {
    if constexpr (NPL == 1) {
        v[0] = *p;
    } else if constexpr (NPL == 2) {
        const float2 t = *reinterpret_cast<const float2 *>(p);
        v[0] = t.x; v[1] = t.y;
    } else {
#pragma unroll
        for (int q = 0; q < NPL / 4; ++q) {
            const float4 t = reinterpret_cast<const float4 *>(p)[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    }
}
template <int NPL>
__device__ __forceinline__ void stv(float *p, const float (&v)[NPL]) {
    if constexpr (NPL == 1) {
        *p = v[0];
    } else if constexpr (NPL == 2) {
        *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int q = 0; q < NPL / 4; ++q)
            reinterpret_cast<float4 *>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

// exp for the per-token decay: the hardware exp2 of x log2(e).  Its relative error is about
// |x| 2^-24 from rounding x log2(e), the same order as the rounding of the product d A itself.
__device__ __forceinline__ float dexp(float x) { return __expf(x); }

struct Row {
    int64_t r, s, h, i, g;
};
__device__ __forceinline__ Row row_of(const SsmArgs &a, int64_t r) {
    Row o;
    o.r = r;
    o.i = r % a.P;
    o.h = (r / a.P) % a.H;
    o.s = r / ((int64_t)a.P * a.H);
    o.g = o.h / (a.H / a.G);
    return o;
}

// ---- step sizes ------------------------------------------------------------------------
__global__ void __launch_bounds__(256) ssm_step_kernel(const SsmArgs a) {
    const int64_t n = (int64_t)a.n_seqs * a.T * a.H;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const float z = a.dt[idx];
        a.dstep[idx] = a.softplus ? (z > 20.f ? z : log1pf(expf(z))) : z;
    }
}

// ---- forward -------------------------------------------------------------------------------
template <int NPL, bool APS>
__global__ void __launch_bounds__(256) ssm_fwd_kernel(const SsmArgs a) {
    const int sub = threadIdx.x & 15;
    const Row w = row_of(a, (int64_t)blockIdx.x * ROWS + (threadIdx.x >> 4));
    const int c0 = sub * NPL;
    const int64_t N = a.N, T = a.T, H = a.H, G = a.G;
    const int nwin = (a.T + WIN - 1) / WIN;
    float st[NPL], Aj[NPL];
    ldv<NPL>(a.s0 + w.r * N + c0, st);
    float Ah = 0.f;
    if constexpr (APS) ldv<NPL>(a.A + w.h * N + c0, Aj);
    else Ah = a.A[w.h];
    const float *xr = a.x + (w.s * T * H + w.h) * a.P + w.i;      // + t H P
    const float *dr = a.dstep + w.s * T * H + w.h;                 // + t H
    const float *br = a.B + (w.s * T * G + w.g) * N + c0;          // + t G N
    const float *cr = a.C + (w.s * T * G + w.g) * N + c0;
    float *yr = a.y ? a.y + (w.s * T * H + w.h) * a.P + w.i : nullptr;
    for (int win = 0; win < nwin; ++win) {
        stv<NPL>(a.ck + (w.r * nwin + win) * N + c0, st);         // state before the window
        const int t0 = win * WIN;
#pragma unroll
        for (int k = 0; k < WIN; ++k) {
            const int64_t t = t0 + k;
            if (t >= T) break;                                     // uniform
            const float d = dr[t * H];
            const float b = d * xr[t * H * a.P];
            float Bv[NPL], Cv[NPL];
            ldv<NPL>(br + t * G * N, Bv);
            ldv<NPL>(cr + t * G * N, Cv);
            float yp = 0.f;
            const float ah = APS ? 0.f : dexp(d * Ah);
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const float aj = APS ? dexp(d * Aj[j]) : ah;
                st[j] = fmaf(aj, st[j], b * Bv[j]);
                yp = fmaf(st[j], Cv[j], yp);
            }
            yp = row16_sum(yp);
            if (yr && sub == 0) yr[t * H * a.P] = yp;
        }
    }
    if (a.s_out) stv<NPL>(a.s_out + w.r * N + c0, st);
}

// ---- backward ------------------------------------------------------------------------------
template <int NPL, bool APS>
__global__ void __launch_bounds__(256) ssm_bwd_kernel(const SsmArgs a) {
    __shared__ float red[WIN][4][2][128];          // [token][wave][dC | dB][column]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = threadIdx.x & 15, rho = lane >> 4;
    const Row w = row_of(a, (int64_t)blockIdx.x * ROWS + (threadIdx.x >> 4));
    const int c0 = sub * NPL;
    const int64_t N = a.N, T = a.T, H = a.H, G = a.G, P = a.P;
    const int nwin = (a.T + WIN - 1) / WIN;
    float gs[NPL], Aj[NPL];
    if (a.gs) ldv<NPL>(a.gs + w.r * N + c0, gs);
    else {
#pragma unroll
        for (int j = 0; j < NPL; ++j) gs[j] = 0.f;
    }
    float Ah = 0.f;
    if constexpr (APS) ldv<NPL>(a.A + w.h * N + c0, Aj);
    else Ah = a.A[w.h];
    const float *xr = a.x + (w.s * T * H + w.h) * P + w.i;
    const float *gyr = a.gy + (w.s * T * H + w.h) * P + w.i;
    const float *dr = a.dstep + w.s * T * H + w.h;
    const float *br = a.B + (w.s * T * G + w.g) * N + c0;
    const float *cr = a.C + (w.s * T * G + w.g) * N + c0;
    float *dxr = a.dx + (w.s * T * H + w.h) * P + w.i;
    float *ddr = a.ddrow + (w.s * T * H + w.h) * P + w.i;
    float *part = a.part + (int64_t)blockIdx.x * T * 2 * N;
    for (int win = nwin - 1; win >= 0; --win) {
        const int t0 = win * WIN;
        const int cnt = min(WIN, a.T - t0);
        float sp[NPL], S[WIN][NPL];
        ldv<NPL>(a.ck + (w.r * nwin + win) * N + c0, sp);
        // replay the window: S[k] is the state after token t0 + k
#pragma unroll
        for (int k = 0; k < WIN; ++k) {
            if (k < cnt) {
                const int64_t t = t0 + k;
                const float d = dr[t * H];
                const float b = d * xr[t * H * P];
                float Bv[NPL];
                ldv<NPL>(br + t * G * N, Bv);
                const float ah = APS ? 0.f : dexp(d * Ah);
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const float aj = APS ? dexp(d * Aj[j]) : ah;
                    S[k][j] = fmaf(aj, k ? S[k - 1][j] : sp[j], b * Bv[j]);
                }
            }
        }
        // walk the window backwards
#pragma unroll
        for (int k = WIN - 1; k >= 0; --k) {
            if (k < cnt) {
                const int64_t t = t0 + k;
                const float d = dr[t * H];
                const float xv = xr[t * H * P];
                const float gyv = gyr[t * H * P];
                float Bv[NPL], Cv[NPL];
                ldv<NPL>(br + t * G * N, Bv);
                ldv<NPL>(cr + t * G * N, Cv);
                const float ah = APS ? 0.f : dexp(d * Ah);
                const float dxv = d * xv;
                float v[2 * NPL];             // column partials: dC then dB
                float gB = 0.f, dec = 0.f;
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const float aj = APS ? dexp(d * Aj[j]) : ah;
                    const float prev = k ? S[k - 1][j] : sp[j];
                    gs[j] = fmaf(gyv, Cv[j], gs[j]);
                    v[j] = gyv * S[k][j];
                    v[NPL + j] = gs[j] * dxv;
                    gB = fmaf(gs[j], Bv[j], gB);
                    dec = APS ? fmaf(gs[j] * (Aj[j] * aj), prev, dec) : fmaf(gs[j], prev, dec);
                    gs[j] = aj * gs[j];
                }
                gB = row16_sum(gB);
                dec = row16_sum(dec);
                if (sub == 0) {
                    dxr[t * H * P] = d * gB;
                    ddr[t * H * P] = (APS ? dec : Ah * ah * dec) + xv * gB;
                }
                // reduce-scatter the column partials over the wave's four row groups
                float u[NPL];
#pragma unroll
                for (int m = 0; m < NPL; ++m) {
                    auto p = __builtin_amdgcn_permlane32_swap(as_i(v[m]), as_i(v[NPL + m]), false, false);
                    u[m] = as_f(p[0]) + as_f(p[1]);   // rows 0-1: dC, rows 2-3: dB (columns m)
                }
                if constexpr (NPL == 1) {
                    auto p = __builtin_amdgcn_permlane16_swap(as_i(u[0]), as_i(u[0]), false, false);
                    const float q = as_f(p[0]) + as_f(p[1]);
                    if ((rho & 1) == 0) red[k][wave][rho >> 1][c0] = q;
                } else {
#pragma unroll
                    for (int m = 0; m < NPL / 2; ++m) {
                        auto p = __builtin_amdgcn_permlane16_swap(as_i(u[m]), as_i(u[NPL / 2 + m]), false, false);
                        // rows 0, 2: columns m; rows 1, 3: columns NPL / 2 + m
                        red[k][wave][rho >> 1][c0 + (rho & 1) * (NPL / 2) + m] = as_f(p[0]) + as_f(p[1]);
                    }
                }
            }
        }
        __syncthreads();
        {   // the window's column sums over the four waves: NPL consecutive outputs per thread
            const int o = threadIdx.x * NPL;                  // of WIN x 2 x N
            const int tok = o / (2 * a.N), qty = (o / a.N) & 1, col = o % a.N;
            if (tok < cnt) {
                float acc[NPL];
#pragma unroll
                for (int m = 0; m < NPL; ++m)
                    acc[m] = ((red[tok][0][qty][col + m] + red[tok][1][qty][col + m]) + red[tok][2][qty][col + m]) +
                             red[tok][3][qty][col + m];
                stv<NPL>(part + (int64_t)(t0 + tok) * 2 * N + qty * N + col, acc);
            }
        }
        __syncthreads();
    }
    stv<NPL>(a.ds0 + w.r * N + c0, gs);
}

// ---- combine: dB, dC over the segments of each group; ddt over the rows of each head ------
__global__ void __launch_bounds__(256) ssm_combine_kernel(const SsmArgs a) {
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, P = a.P;
    const int64_t nbc = (int64_t)a.n_seqs * T * G * N;   // dB / dC elements
    const int64_t ndt = (int64_t)a.n_seqs * T * H;
    const int64_t segs_per_group = P * (H / G) / ROWS;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nbc + ndt;
         idx += (int64_t)gridDim.x * blockDim.x) {
        if (idx < nbc) {
            const int64_t n = idx % N, g = (idx / N) % G, t = (idx / (N * G)) % T, s = idx / (N * G * T);
            const int64_t seg0 = (s * H * P + g * P * (H / G)) / ROWS;
            float db = 0.f, dc = 0.f;
            for (int64_t k = 0; k < segs_per_group; ++k) {
                const float *pp = a.part + ((seg0 + k) * T + t) * 2 * N;
                dc += pp[n];
                db += pp[N + n];
            }
            a.dB[idx] = db;
            a.dC[idx] = dc;
        } else {
            const int64_t j = idx - nbc;                      // (s, t, h)
            const float *rr = a.ddrow + j * P;
            float acc = 0.f;
            for (int64_t i = 0; i < P; ++i) acc += rr[i];
            if (a.softplus) acc *= 1.f / (1.f + expf(-a.dt[j]));
            a.ddt[j] = acc;
        }
    }
}

template <int NPL>
hipError_t launch_scan(const SsmArgs &a, bool bwd, hipStream_t st) {
    const int64_t rows = (int64_t)a.n_seqs * a.H * a.P;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    const void *fn;
    if (bwd) fn = a.aps ? (const void *)ssm_bwd_kernel<NPL, true> : (const void *)ssm_bwd_kernel<NPL, false>;
    else fn = a.aps ? (const void *)ssm_fwd_kernel<NPL, true> : (const void *)ssm_fwd_kernel<NPL, false>;
    return hipLaunchKernel(fn, dim3((unsigned)(rows / ROWS)), dim3(256), params, 0, st);
}

unsigned grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    return (unsigned)(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

}  // namespace

hipError_t launch_ssm_step(const SsmArgs &a, hipStream_t st) {
    const int64_t n = (int64_t)a.n_seqs * a.T * a.H;
    if (n <= 0) return hipSuccess;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    return hipLaunchKernel((const void *)ssm_step_kernel, dim3(grid_for(n)), dim3(256), params, 0, st);
}

hipError_t launch_ssm(const SsmArgs &a, bool bwd, hipStream_t st) {
    if ((int64_t)a.n_seqs * a.H * a.P <= 0) return hipSuccess;
    switch (a.N) {
        case 16: return launch_scan<1>(a, bwd, st);
        case 32: return launch_scan<2>(a, bwd, st);
        case 64: return launch_scan<4>(a, bwd, st);
        case 128: return launch_scan<8>(a, bwd, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ssm_combine(const SsmArgs &a, hipStream_t st) {
    const int64_t n = (int64_t)a.n_seqs * a.T * ((int64_t)a.G * a.N + a.H);
    if (n <= 0) return hipSuccess;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    return hipLaunchKernel((const void *)ssm_combine_kernel, dim3(grid_for(n)), dim3(256), params, 0, st);
}

}  // namespace gdn
