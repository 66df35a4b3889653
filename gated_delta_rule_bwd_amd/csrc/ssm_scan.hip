// ssm_scan.hip -- gfx950 kernels of the selective state-space scan (Mamba-1: one decay per
// state; Mamba-2: one per head) and of its backward, the reverse recurrence (page "S1-24:
// chunked attention", the SSM_SCAN_BACK commit notes and the n_group fold).  Per sequence s,
// head h (group g = h / (H / G)), head element i and state n, with step d = softplus(dt) (or dt):
//   a = exp(d A[h, n]),  s[i, n] = a s[i, n] + d x[i] B[g, n],  y[i] = sum_n s[i, n] C[g, n].
//
// Layout of the work: a row is one (s, h, i); 16 lanes own a row, each lane NPL = N / 16 state
// columns (see col_of); a workgroup is 16 rows (4 per wave), which must lie in one group.
// The forward keeps the row's state in registers, writes y through a 16-lane DPP sum and saves
// the state before every 8-token window.  The backward walks the windows in reverse: it
// replays a window from its saved state into registers, then walks its tokens backwards with
// the state gradient gs in registers.  Row sums (dx, the decay term of ddt) are 16-lane DPP
// sums; the column sums of a token (dC = sum_i gy s, dB = sum_i gs d x over the 16 rows) are
// reduce-scattered over the four row groups of a wave with permlane swaps, summed over the four
// waves in LDS at the window's end and written as the segment's partial; a combine kernel adds
// the segments of each group (and the rows of each head for ddt) in a fixed order.  With 16
// states and whole 128-row blocks per group the backward instead runs in two passes (the state
// gradient entering every window, then the windows in parallel with two lanes per row: see
// ssm_gsw_kernel and ssm_win16_kernel); one decay per head with head size 64 and 128 states
// runs in chunks on the matrix cores (ssm_chunk.hip).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"
#include "ssm_common.h"

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
// The row-wise kernels for 16 states keep A scaled by log2(e) and take their decays as
// 2^(step A log2 e): one multiply and the hardware base-2 exponential per decay.
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// row_of for a wave-uniform row, with 32-bit divisions when the row and the rows of a sequence
// fit in 32 bits
__device__ __forceinline__ Row row_of_uniform(const SsmArgs &a, int64_t r) {
    const int64_t rows_seq = (int64_t)a.P * a.H;
    if (r > 0xffffffffll || rows_seq > 0xffffffffll) return row_of(a, r);
    const uint32_t ru = (uint32_t)r, P = (uint32_t)a.P, H = (uint32_t)a.H;
    const uint32_t q = ru / P, s = q / H, h = q - s * H;
    Row o;
    o.r = r;
    o.i = ru - q * P;
    o.h = h;
    o.s = s;
    o.g = h / (H / (uint32_t)a.G);
    return o;
}

// ---- window staging --------------------------------------------------------------------
// The 16 rows of a workgroup share one (sequence, group), so a window's B and C rows are
// common to all of them; x, the step (and gy) are per row.  Each window is staged in LDS once
// and the next one is loaded into registers while the current one is computed.
// (sized for NC = N states: the LDS a workgroup takes bounds how many fit on a CU)
template <int NC>
struct Stage {
    float B[WIN][NC], C[WIN][NC];
    float x[WIN][ROWS], d[WIN][ROWS], gy[WIN][ROWS];
};

template <int NPL, bool GY>
struct Loader {
    static constexpr int NQ = NPL >= 4 ? NPL / 4 : 1;   // float4s of B|C per thread
    float4 q[NQ];
    float s0v, s1v;                                     // x or step; gy
    int tid;
    int64_t seq, g;
    int64_t lh, li;                                     // head and element of the loader's row

    __device__ void init(const SsmArgs &a, int64_t r0, int t) {
        tid = t;
        const Row lw = row_of(a, r0 + (t & 15));
        seq = lw.s; g = lw.g; lh = lw.h; li = lw.i;
    }
    __device__ void load(const SsmArgs &a, int t0, int cnt) {
        const int64_t N = a.N, T = a.T, H = a.H, P = a.P, G = a.G;
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int qq = tid + 256 * m;               // of 2 arrays x WIN tokens x N / 4
            if (qq < 4 * a.N) {
                const int arr = qq >= 2 * a.N;
                const int q2 = qq - arr * 2 * a.N;
                const int tok = q2 / (a.N / 4), c4 = q2 % (a.N / 4);
                const int64_t t = t0 + min(tok, cnt - 1);
                q[m] = *reinterpret_cast<const float4 *>((arr ? a.C : a.B) + ((seq * T + t) * G + g) * N + 4 * c4);
            }
        }
        const int tok = (tid & 127) >> 4;
        const int64_t t = t0 + min(tok, cnt - 1);
        if (tid < 128) s0v = a.x[((seq * T + t) * H + lh) * P + li];
        else s0v = a.dt[(seq * T + t) * H + lh];   // raw: the step is taken in put()
        if constexpr (GY) {
            if (tid < 128) s1v = a.gy[((seq * T + t) * H + lh) * P + li];
        }
    }
    __device__ void put(const SsmArgs &a, Stage<16 * NPL> &st) const {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int qq = tid + 256 * m;
            if (qq < 4 * a.N) {
                const int arr = qq >= 2 * a.N;
                const int q2 = qq - arr * 2 * a.N;
                const int tok = q2 / (a.N / 4), c4 = q2 % (a.N / 4);
                *reinterpret_cast<float4 *>(&(arr ? st.C : st.B)[tok][4 * c4]) = q[m];
            }
        }
        const int tok = (tid & 127) >> 4, rr = tid & 15;
        if (tid < 128) st.x[tok][rr] = s0v;
        else st.d[tok][rr] = ssm_step(s0v, a.softplus);
        if constexpr (GY) {
            if (tid < 128) st.gy[tok][rr] = s1v;
        }
    }
};

// The state columns a lane owns.  With NPL >= 4 they are float4 chunks 64 columns apart
// (columns 4 sub .. 4 sub + 3, then 64 + 4 sub .., ...), so the 16 lanes of a row read 256
// contiguous bytes per 16-byte access and LDS rows are read without bank conflicts; with
// NPL < 4 the NPL columns from sub NPL on.
template <int NPL>
__device__ __forceinline__ int col_of(int sub, int j) {
    if constexpr (NPL >= 4) return (j >> 2) * 64 + 4 * sub + (j & 3);
    else return sub * NPL + j;
}
template <int NPL>
__device__ __forceinline__ void ld_cols(const float *row, int sub, float (&v)[NPL]) {
    if constexpr (NPL >= 4) {
#pragma unroll
        for (int q = 0; q < NPL / 4; ++q) {
            const float4 t = *reinterpret_cast<const float4 *>(row + q * 64 + 4 * sub);
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    } else {
        ldv<NPL>(row + sub * NPL, v);
    }
}
template <int NPL>
__device__ __forceinline__ void st_cols(float *row, int sub, const float (&v)[NPL]) {
    if constexpr (NPL >= 4) {
#pragma unroll
        for (int q = 0; q < NPL / 4; ++q)
            *reinterpret_cast<float4 *>(row + q * 64 + 4 * sub) =
                make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
        stv<NPL>(row + sub * NPL, v);
    }
}

// ---- forward -------------------------------------------------------------------------------
template <int NPL, bool APS>
__global__ void __launch_bounds__(256) ssm_fwd_kernel(const SsmArgs a) {
    __shared__ Stage<16 * NPL> stg[2];
    __shared__ float ys[2][WIN][ROWS];
    const int tid = threadIdx.x, sub = tid & 15, rho = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const Row w = row_of(a, r0 + rho);
    const int64_t N = a.N, T = a.T, H = a.H, P = a.P;
    const int nwin = (a.T + WIN - 1) / WIN;
    float st[NPL], Aj[NPL];
    ld_cols<NPL>(a.s0 + w.r * N, sub, st);
    float Ah = 0.f;
    if constexpr (APS) ld_cols<NPL>(a.A + w.h * N, sub, Aj);
    else Ah = a.A[w.h];
    // window j is loaded into register set j % PD at the start of window j - PD + 1, staged
    // into LDS at the end of window j - 1: PD - 1 windows of compute cover its load latency
    constexpr int PD = 3;
    Loader<NPL, false> ld[PD];
#pragma unroll
    for (int q = 0; q < PD; ++q) ld[q].init(a, r0, tid);
    const int wr = tid & 15, wtok = (tid & 127) >> 4;   // y writer: row, token
    const Row ow = row_of(a, r0 + wr);
    auto wcnt = [&](int j) { return min(WIN, a.T - j * WIN); };
#pragma unroll
    for (int q = 0; q < PD - 1; ++q)
        if (q < nwin) ld[q].load(a, q * WIN, wcnt(q));
    if (nwin > 0) ld[0].put(a, stg[0]);
    __syncthreads();
    auto window = [&](int win, auto u) __attribute__((always_inline)) {
        constexpr int U = decltype(u)::value;            // win % PD
        const int cur = win & 1;
        const int t0 = win * WIN, cnt = wcnt(win);
        if (win + PD - 1 < nwin) ld[(U + PD - 1) % PD].load(a, (win + PD - 1) * WIN, wcnt(win + PD - 1));
        if (win % a.ckw == 0)                                       // state before the window
            st_cols<NPL>(a.ck + (w.r * a.nck + win / a.ckw) * N, sub, st);
        const Stage<16 * NPL> &sg = stg[cur];
#pragma unroll
        for (int k = 0; k < WIN; ++k) {
            if (k < cnt) {                                           // uniform
                const float d = sg.d[k][rho];
                const float b = d * sg.x[k][rho];
                float Bv[NPL], Cv[NPL];
                ld_cols<NPL>(&sg.B[k][0], sub, Bv);
                ld_cols<NPL>(&sg.C[k][0], sub, Cv);
                float yp = 0.f;
                const float ah = APS ? 0.f : dexp(d * Ah);
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const float aj = APS ? dexp(d * Aj[j]) : ah;
                    st[j] = fmaf(aj, st[j], b * Bv[j]);
                    yp = fmaf(st[j], Cv[j], yp);
                }
                yp = row16_sum(yp);
                if (sub == 0) ys[cur][k][rho] = yp;
            }
        }
        if (win + 1 < nwin) ld[(U + 1) % PD].put(a, stg[cur ^ 1]);
        __syncthreads();
        if (a.y && tid < 128 && wtok < cnt)
            a.y[((ow.s * T + t0 + wtok) * H + ow.h) * P + ow.i] = ys[cur][wtok][wr];
    };
    for (int win = 0; win < nwin; win += PD) {
        window(win, std::integral_constant<int, 0>{});
        if (win + 1 < nwin) window(win + 1, std::integral_constant<int, 1>{});
        if (win + 2 < nwin) window(win + 2, std::integral_constant<int, 2>{});
    }
    if (a.s_out) st_cols<NPL>(a.s_out + w.r * N, sub, st);
}

// ---- backward ------------------------------------------------------------------------------
template <int NPL, bool APS>
__global__ void __launch_bounds__(256) ssm_bwd_kernel(const SsmArgs a) {
    __shared__ Stage<16 * NPL> stg[2];
    __shared__ float red[WIN][4][2][16 * NPL];     // [token][wave][dC | dB][column]
    __shared__ float os[2][WIN][ROWS];             // dx, ddt term per (token, row)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = tid & 15, rho = tid >> 4, rg = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const Row w = row_of(a, r0 + rho);
    const int64_t N = a.N, T = a.T, H = a.H, P = a.P;
    const int nwin = (a.T + WIN - 1) / WIN;
    float gs[NPL], Aj[NPL];
    if (a.gs) ld_cols<NPL>(a.gs + w.r * N, sub, gs);
    else {
#pragma unroll
        for (int j = 0; j < NPL; ++j) gs[j] = 0.f;
    }
    float Ah = 0.f;
    if constexpr (APS) ld_cols<NPL>(a.A + w.h * N, sub, Aj);
    else Ah = a.A[w.h];
    Loader<NPL, true> ld;
    ld.init(a, r0, tid);
    const int wr = tid & 15, wtok = (tid & 127) >> 4, wq = tid >> 7;   // dx / dd writer
    const Row ow = row_of(a, r0 + wr);
    float *part = a.part + (int64_t)blockIdx.x * T * 2 * N;
    if (nwin > 0) {
        const int t0 = (nwin - 1) * WIN;
        ld.load(a, t0, a.T - t0);
        ld.put(a, stg[0]);
    }
    __syncthreads();
    for (int it = 0; it < nwin; ++it) {
        const int win = nwin - 1 - it, cur = it & 1;
        const int t0 = win * WIN, cnt = min(WIN, a.T - t0);
        if (win > 0) ld.load(a, t0 - WIN, WIN);
        const Stage<16 * NPL> &sg = stg[cur];
        float sp[NPL], S[WIN][NPL];
        ld_cols<NPL>(a.ck + (w.r * a.nck + win) * N, sub, sp);   // every window saved
        // replay the window: S[k] is the state after token t0 + k
#pragma unroll
        for (int k = 0; k < WIN; ++k) {
            if (k < cnt) {
                const float d = sg.d[k][rho];
                const float b = d * sg.x[k][rho];
                float Bv[NPL];
                ld_cols<NPL>(&sg.B[k][0], sub, Bv);
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
                const float d = sg.d[k][rho];
                const float xv = sg.x[k][rho];
                const float gyv = sg.gy[k][rho];
                float Bv[NPL], Cv[NPL];
                ld_cols<NPL>(&sg.B[k][0], sub, Bv);
                ld_cols<NPL>(&sg.C[k][0], sub, Cv);
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
                    os[0][k][rho] = d * gB;
                    os[1][k][rho] = (APS ? dec : Ah * ah * dec) + xv * gB;
                }
                // reduce-scatter the column partials over the wave's four row groups
                float u[NPL];
#pragma unroll
                for (int m = 0; m < NPL; ++m) {
                    auto pr = __builtin_amdgcn_permlane32_swap(as_i(v[m]), as_i(v[NPL + m]), false, false);
                    u[m] = as_f(pr[0]) + as_f(pr[1]);   // row groups 0-1: dC, 2-3: dB (columns m)
                }
                if constexpr (NPL == 1) {
                    auto pr = __builtin_amdgcn_permlane16_swap(as_i(u[0]), as_i(u[0]), false, false);
                    const float q = as_f(pr[0]) + as_f(pr[1]);
                    if ((rg & 1) == 0) red[k][wave][rg >> 1][sub] = q;
                } else {
                    // row groups 0, 2: the lane's columns m; 1, 3: its columns NPL / 2 + m, which
                    // are consecutive, so one vector store per lane (32 lanes: 512 contiguous B)
                    float q[NPL / 2];
#pragma unroll
                    for (int m = 0; m < NPL / 2; ++m) {
                        auto pr = __builtin_amdgcn_permlane16_swap(as_i(u[m]), as_i(u[NPL / 2 + m]), false, false);
                        q[m] = as_f(pr[0]) + as_f(pr[1]);
                    }
                    float *dst = &red[k][wave][rg >> 1][col_of<NPL>(sub, (rg & 1) * (NPL / 2))];
                    if constexpr (NPL == 8) *reinterpret_cast<float4 *>(dst) = make_float4(q[0], q[1], q[2], q[3]);
                    else if constexpr (NPL == 4) *reinterpret_cast<float2 *>(dst) = make_float2(q[0], q[1]);
                    else dst[0] = q[0];
                }
            }
        }
        if (win > 0) ld.put(a, stg[cur ^ 1]);
        __syncthreads();
        {   // the window's column sums over the four waves (WIN x 2 x N outputs): groups of
            // V consecutive outputs, consecutive threads on consecutive groups
            constexpr int V = NPL >= 4 ? 4 : NPL;
#pragma unroll
            for (int u = 0; u < NPL / V; ++u) {
                const int o = V * tid + 256 * V * u;
                const int tok = o / (2 * a.N), qty = (o / a.N) & 1, col = o % a.N;
                if (tok < cnt) {
                    float acc[V];
#pragma unroll
                    for (int m = 0; m < V; ++m)
                        acc[m] = ((red[tok][0][qty][col + m] + red[tok][1][qty][col + m]) + red[tok][2][qty][col + m]) +
                                 red[tok][3][qty][col + m];
                    stv<V>(part + (int64_t)(t0 + tok) * 2 * N + qty * N + col, acc);
                }
            }
            if (wtok < cnt) {
                const int64_t at = ((ow.s * T + t0 + wtok) * H + ow.h) * P + ow.i;
                (wq ? a.ddrow : a.dx)[at] = os[wq][wtok][wr];
            }
        }
        __syncthreads();
    }
    st_cols<NPL>(a.ds0 + w.r * N, sub, gs);
}

// ---- row-wise backward for 16 states ---------------------------------------------------
// With 16 states a lane of the per-token walk above owns one state element, so most of its
// instructions are the per-token sums across lanes.  Here the walk is split in two passes:
// pass 1 runs the state gradient's own recurrence (gs += gy C, gs *= a from the last token) in
// the forward's layout and stores the gradient entering every window from the right (and
// d_s0); pass 2 then takes every window independently, two lanes per row with eight states
// each in registers, so a row's sums (dx, the ddt term) are one pair sum, and only the column
// sums of a token (dC, dB over rows) cross more lanes: a reduce-scatter over the wave after which
// each lane holds one (quantity, state) sum over the wave's 32 rows, then a sum over the four
// waves in LDS.  (One lane per row, all 16 states in registers, needed 238 registers, two waves
// per SIMD, and was 8 % slower.)  The gradient chain runs the walk's own operations in the
// walk's order, so pass 2 starts each window from the gradient the single-pass walk would have
// there.
constexpr int GB = 32;   // tokens per staging block of pass 1

template <bool APS>
__global__ void __launch_bounds__(256) ssm_gsw_kernel(const SsmArgs a) {
    // per block of GB tokens: the rows' gy and step, the group's C (16 states)
    __shared__ float sgy[2][GB][ROWS], sd[2][GB][ROWS], sC[2][GB][16];
    const int tid = threadIdx.x, sub = tid & 15, rho = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const Row w = row_of(a, r0 + rho);
    const int64_t N = a.N, T = a.T, H = a.H, P = a.P, G = a.G;
    const int nwin = (a.T + WIN - 1) / WIN;
    const int nblk = (a.T + GB - 1) / GB;
    float gs = a.gs ? a.gs[w.r * N + sub] : 0.f;
    const float Aj = (APS ? a.A[w.h * N + sub] : a.A[w.h]) * kLog2e;
    // thread tid stages token pairs (tokens 2 (tid >> 4) + {0, 1}) of row tid & 15: gy, dt; and
    // C of those tokens, state tid & 15
    const Row lw = row_of(a, r0 + sub);
    const int tk = 2 * rho;
    // the block's 16 rows share a sequence: its first token's entries are the loads' base, the
    // row's own entries a lane offset (tokens past the end read the last one)
    const int64_t s0 = row_of_uniform(a, r0).s, HP = H * P, GN = G * N;
    const float *const gyq = a.gy + s0 * T * HP, *const dtq = a.dt + s0 * T * H, *const cq = a.C + s0 * T * GN;
    const uint32_t og = (uint32_t)(lw.h * P + lw.i) * 4, od = (uint32_t)lw.h * 4, oc = (uint32_t)(lw.g * N + sub) * 4;
    float pg[2], pd[2], pc[2];
    auto load = [&](int blk) {
        const int tb = blk * GB, last = a.T - 1 - tb;
        const Rsrc rg = rsrc(gyq + tb * HP), rd = rsrc(dtq + (int64_t)tb * H), rc = rsrc(cq + tb * GN);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t tl = (uint32_t)min(tk + u, last);
            pg[u] = bld(rg, tl * (uint32_t)HP * 4 + og, 0);
            pd[u] = bld(rd, tl * (uint32_t)H * 4 + od, 0);
            pc[u] = bld(rc, tl * (uint32_t)GN * 4 + oc, 0);
        }
    };
    // a token past the end gets gy = 0 and step 0 (decay 1): it leaves gs as it is, so the
    // token loop below needs no branch and its LDS reads can run ahead
    auto put = [&](int blk, int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool ok = blk * GB + tk + u < a.T;
            sgy[buf][tk + u][sub] = ok ? pg[u] : 0.f;
            sd[buf][tk + u][sub] = ok ? ssm_step(pd[u], a.softplus) : 0.f;
            sC[buf][tk + u][sub] = pc[u];
        }
    };
    if (nblk > 0) {
        load(nblk - 1);
        put(nblk - 1, 0);
    }
    __syncthreads();
    for (int it = 0; it < nblk; ++it) {
        const int blk = nblk - 1 - it, cur = it & 1;
        const int t0 = blk * GB;
        if (blk > 0) load(blk - 1);
#pragma unroll
        for (int k = GB - 1; k >= 0; --k) {
            if ((k & (WIN - 1)) == WIN - 1)   // the gradient entering the window (a window past
                // the end stores the unchanged value into the last window's slot, which that
                // window then writes again with the same bits)
                a.gsw[(w.r * nwin + min((t0 + k) / WIN, nwin - 1)) * N + sub] = gs;
            gs = fmaf(sgy[cur][k][rho], sC[cur][k][sub], gs);
            gs = dexp2(sd[cur][k][rho] * Aj) * gs;
        }
        if (blk > 0) put(blk - 1, cur ^ 1);
        __syncthreads();
    }
    a.ds0[w.r * N + sub] = gs;
}

constexpr int RB = 128;   // rows per block of pass 2 (and per column-sum segment): two lanes per
                          // row, eight states each

// Row j of the RB-row block starting at row r0 (a multiple of RB): the block lies in one
// (sequence, group), since a group's rows are a multiple of RB, so only the head and position
// differ from the block's first row (found once, with scalar arithmetic).
__device__ __forceinline__ Row block_row(const SsmArgs &a, const Row &w0, int j) {
    Row w = w0;
    const int q = (int)w0.i + j;
    const int dh = a.P == 1 ? q : q / a.P;
    w.r = w0.r + j;
    w.i = q - dh * a.P;
    w.h = w0.h + dh;
    return w;
}

__device__ __forceinline__ void ld8(const float *p, float (&v)[8]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float4 t = reinterpret_cast<const float4 *>(p)[q];
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
}

// One workgroup per (128 rows, 8-token window); lane l owns states 8 (l & 1) .. + 7 of row l / 2.
// Replay the window from its saved state, walk it back from the window's gradient; the token's
// dC and dB are reduce-scattered over the wave's 32 rows in three steps (permlane32: dC or dB,
// permlane16: 4 states, row_ror:8: 2), so lane l ends with states 8 (l & 1) + 4 bit4 + 2 bit3
// + {0, 1} of dC (l < 32) or dB over 8 of the rows; the window's end sums the four lanes (bits
// 1, 2) of each of the four waves from LDS in a fixed order.
template <bool APS>
__global__ void __launch_bounds__(256) ssm_win16_kernel(const SsmArgs a) {
    constexpr int N = 16, NH = 8;
    __shared__ float bc[2][WIN][N];          // B, C rows of the window's tokens
    __shared__ __align__(16) float red[WIN][4][4][2 * N];  // [token][wave][lane bits 1, 2][dC | dB state]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hb = lane & 1;
    const int nwin = (a.T + WIN - 1) / WIN;
    const int win = (int)(blockIdx.x % nwin);
    const int64_t rb = blockIdx.x / nwin;
    const Row w0 = row_of_uniform(a, rb * RB), w = block_row(a, w0, tid >> 1);
    const int64_t T = a.T, H = a.H, P = a.P, G = a.G;
    const int t0 = win * WIN, cnt = min(WIN, a.T - t0);
    {
        const int k = tid >> 5, q = (tid >> 4) & 1, n = tid & 15;
        const int64_t t = min(t0 + k, a.T - 1);
        bc[q][k][n] = (q ? a.C : a.B)[((w0.s * T + t) * G + w0.g) * N + n];
    }
    // this row's x, gy (one token apart: tstr) and step (H apart) from the window's first token
    const int64_t at0 = ((w.s * T + t0) * H + w.h) * P + w.i, tstr = H * P;
    const float *const xw = a.x + at0, *const gw = a.gy + at0, *const dtw = a.dt + (w.s * T + t0) * H + w.h;
    float sp[NH], gs[NH], Av[NH];
    ld8(a.ck + (w.r * a.nck + win) * N + NH * hb, sp);
    ld8(a.gsw + (w.r * nwin + win) * N + NH * hb, gs);
    float Ah = 0.f, Ah2 = 0.f;   // A (one per head), and scaled by log2(e)
    if constexpr (APS) {
        ld8(a.A + w.h * N + NH * hb, Av);
#pragma unroll
        for (int m = 0; m < NH; ++m) Av[m] *= kLog2e;
    } else {
        Ah = a.A[w.h];
        Ah2 = Ah * kLog2e;
    }
    float xv[WIN], gv[WIN], dv[WIN], sg[WIN];
    {
        // the pair's lanes each take the step (and softplus') of four tokens and swap them
        float m4[4], s4[4];
#pragma unroll
        for (int k = 0; k < WIN; ++k) {
            const int kk = min(k, cnt - 1);   // tokens past the end are skipped below
            const bool ok = k < cnt;
            const float xr = xw[kk * tstr], gr = gw[kk * tstr];
            xv[k] = ok ? xr : 0.f;
            gv[k] = ok ? gr : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = 4 * hb + j;
            const float z = dtw[min(k, cnt - 1) * H];
            m4[j] = k < cnt ? ssm_step(z, a.softplus) : 0.f;
            s4[j] = (P == 1 && a.softplus) ? __builtin_amdgcn_rcpf(1.f + expf(-z)) : 1.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float mo = dpp<0xB1>(m4[j]), so = dpp<0xB1>(s4[j]);   // the other lane's tokens
            dv[j] = hb ? mo : m4[j];
            dv[4 + j] = hb ? m4[j] : mo;
            sg[j] = hb ? so : s4[j];
            sg[4 + j] = hb ? s4[j] : so;
        }
    }
    __syncthreads();
    float S[WIN][NH];
#pragma unroll
    for (int k = 0; k < WIN; ++k) {
        const float b = dv[k] * xv[k];
        const float ah = APS ? 0.f : dexp2(dv[k] * Ah2);
#pragma unroll
        for (int m = 0; m < NH; ++m) {
            const float aj = APS ? dexp2(dv[k] * Av[m]) : ah;
            S[k][m] = fmaf(aj, k ? S[k - 1][m] : sp[m], b * bc[0][k][NH * hb + m]);
        }
    }
    const bool b3 = lane & 8;
    // this lane's pair of sums in red[k][wave]: row (lane bits 1, 2), column of its first state
    const int rcol = ((lane >> 1) & 3) * 2 * N + (lane >> 5) * N + NH * hb + 4 * ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1);
    // the window's dx and ddt (or ddrow) entries of this row, one token apart
    float *const dxw = a.dx + at0, *const ddw = (P == 1 ? a.ddt : a.ddrow) + at0;
#pragma unroll
    for (int k = 0; k < WIN; ++k) asm volatile("" : "+v"(dv[k]));
    // a full window walks without a test per token (the last, partial one with it)
    auto walk = [&](auto full) {
#pragma unroll
    for (int k = WIN - 1; k >= 0; --k) {
        if (decltype(full)::value || k < cnt) {
            const float d = dv[k], xk = xv[k], gyk = gv[k], dxv = d * xk;
            const float ah = APS ? 0.f : dexp2(d * Ah2);
            float v[2 * NH];
            float gB = 0.f, dec = 0.f;   // dec: sum of gs a A s_prev (A log2(e) with APS)
#pragma unroll
            for (int m = 0; m < NH; ++m) {
                const float aj = APS ? dexp2(d * Av[m]) : ah;
                const float prev = k ? S[k - 1][m] : sp[m];
                gs[m] = fmaf(gyk, bc[1][k][NH * hb + m], gs[m]);
                v[m] = gyk * S[k][m];
                v[NH + m] = gs[m] * dxv;
                gB = fmaf(gs[m], bc[0][k][NH * hb + m], gB);
                if constexpr (APS) {
                    gs[m] = aj * gs[m];
                    dec = fmaf(gs[m] * prev, Av[m], dec);
                } else {
                    dec = fmaf(gs[m], prev, dec);
                    gs[m] = aj * gs[m];
                }
            }
            gB += dpp<0xB1>(gB);    // the pair's halves
            dec += dpp<0xB1>(dec);
            if (hb == 0) {
                dxw[k * tstr] = d * gB;
                ddw[k * tstr] = ((APS ? dec * kLn2 : Ah * ah * dec) + xk * gB) * sg[k];
            }
            float u[8], w4[4], x2[2];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                auto pr = __builtin_amdgcn_permlane32_swap(as_i(v[m]), as_i(v[8 + m]), false, false);
                u[m] = as_f(pr[0]) + as_f(pr[1]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                auto pr = __builtin_amdgcn_permlane16_swap(as_i(u[m]), as_i(u[4 + m]), false, false);
                w4[m] = as_f(pr[0]) + as_f(pr[1]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float keep = b3 ? w4[2 + m] : w4[m], send = b3 ? w4[m] : w4[2 + m];
                x2[m] = keep + dpp<0x128>(send);
            }
            *reinterpret_cast<float2 *>(&red[k][wave][0][0] + rcol) = make_float2(x2[0], x2[1]);
        }
    }
    };
    if (cnt == WIN) walk(std::true_type{});
    else walk(std::false_type{});
    __syncthreads();
    {
        const int k = tid >> 5, idx = tid & 31;
        if (k < cnt) {
            float sum = 0.f;
#pragma unroll
            for (int wv = 0; wv < 4; ++wv)
#pragma unroll
                for (int q = 0; q < 4; ++q) sum += red[k][wv][q][idx];
            a.part[(rb * T + t0 + k) * 2 * N + idx] = sum;
        }
    }
}

// ---- row-wise forward for 16 states -----------------------------------------------------
// The same shapes' forward in two passes: the state's own recurrence (s = a s + d x B from the
// first token) in the per-token layout, saving the state before every window (a window past the
// end saves into one spare slot per row, so the token loop needs no branch) and s_out; then every
// window on its own, two lanes per row, replaying from the saved state for y (a pair sum per
// token instead of the per-token kernel's 16-lane sum).  Both replay with the walk's formula, so
// the backward's replay gives the same states.
template <bool APS>
__global__ void __launch_bounds__(256) ssm_sst_kernel(const SsmArgs a) {
    // per block of GB tokens: the rows' d x and step, the group's B (16 states)
    __shared__ float sb[2][GB][ROWS], sd[2][GB][ROWS], sB[2][GB][16];
    const int tid = threadIdx.x, sub = tid & 15, rho = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const Row w = row_of(a, r0 + rho);
    const int64_t N = a.N, T = a.T, H = a.H, P = a.P, G = a.G;
    const int nwin = (a.T + WIN - 1) / WIN;
    const int nblk = (a.T + GB - 1) / GB;
    float st = a.s0[w.r * N + sub];
    const float Aj = (APS ? a.A[w.h * N + sub] : a.A[w.h]) * kLog2e;
    const Row lw = row_of(a, r0 + sub);
    const int tk = 2 * rho;
    // loads as in the gradient pass: the sequence's first token as base, the row as lane offset
    const int64_t s0 = row_of_uniform(a, r0).s, HP = H * P, GN = G * N;
    const float *const xq = a.x + s0 * T * HP, *const dtq = a.dt + s0 * T * H, *const bq = a.B + s0 * T * GN;
    const uint32_t ox = (uint32_t)(lw.h * P + lw.i) * 4, od = (uint32_t)lw.h * 4, ob = (uint32_t)(lw.g * N + sub) * 4;
    float px[2], pd[2], pb[2];
    auto load = [&](int blk) {
        const int tb = blk * GB, last = a.T - 1 - tb;
        const Rsrc rx = rsrc(xq + tb * HP), rd = rsrc(dtq + (int64_t)tb * H), rb = rsrc(bq + tb * GN);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t tl = (uint32_t)min(tk + u, last);
            px[u] = bld(rx, tl * (uint32_t)HP * 4 + ox, 0);
            pd[u] = bld(rd, tl * (uint32_t)H * 4 + od, 0);
            pb[u] = bld(rb, tl * (uint32_t)GN * 4 + ob, 0);
        }
    };
    // a token past the end gets step 0 (decay 1) and d x = 0: it leaves the state as it is
    auto put = [&](int blk, int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool ok = blk * GB + tk + u < a.T;
            const float d = ok ? ssm_step(pd[u], a.softplus) : 0.f;
            sd[buf][tk + u][sub] = d;
            sb[buf][tk + u][sub] = d * (ok ? px[u] : 0.f);
            sB[buf][tk + u][sub] = pb[u];
        }
    };
    if (nblk > 0) {
        load(0);
        put(0, 0);
    }
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        const int cur = blk & 1, t0 = blk * GB;
        if (blk + 1 < nblk) load(blk + 1);
#pragma unroll
        for (int k = 0; k < GB; ++k) {
            if ((k & (WIN - 1)) == 0)   // the state before the window (slot nwin: past the end)
                a.ck[(w.r * a.nck + min((t0 + k) / WIN, nwin)) * N + sub] = st;
            st = fmaf(dexp2(sd[cur][k][rho] * Aj), st, sb[cur][k][rho] * sB[cur][k][sub]);
        }
        if (blk + 1 < nblk) put(blk + 1, cur ^ 1);
        __syncthreads();
    }
    if (a.s_out) a.s_out[w.r * N + sub] = st;
}

template <bool APS>
__global__ void __launch_bounds__(256) ssm_y16_kernel(const SsmArgs a) {
    constexpr int N = 16, NH = 8;
    __shared__ float bc[2][WIN][N];          // B, C rows of the window's tokens
    const int tid = threadIdx.x, lane = tid & 63, hb = lane & 1;
    const int nwin = (a.T + WIN - 1) / WIN;
    const int win = (int)(blockIdx.x % nwin);
    const int64_t rb = blockIdx.x / nwin;
    const Row w0 = row_of_uniform(a, rb * RB), w = block_row(a, w0, tid >> 1);
    const int64_t T = a.T, H = a.H, P = a.P, G = a.G;
    const int t0 = win * WIN, cnt = min(WIN, a.T - t0);
    {
        const int k = tid >> 5, q = (tid >> 4) & 1, n = tid & 15;
        const int64_t t = min(t0 + k, a.T - 1);
        bc[q][k][n] = (q ? a.C : a.B)[((w0.s * T + t) * G + w0.g) * N + n];
    }
    const int64_t at0 = ((w.s * T + t0) * H + w.h) * P + w.i, tstr = H * P;
    const float *const dtw = a.dt + (w.s * T + t0) * H + w.h;
    float sv[NH], Av[NH];
    ld8(a.ck + (w.r * a.nck + win) * N + NH * hb, sv);
    float Ah = 0.f;
    if constexpr (APS) {
        ld8(a.A + w.h * N + NH * hb, Av);
#pragma unroll
        for (int m = 0; m < NH; ++m) Av[m] *= kLog2e;
    } else {
        Ah = a.A[w.h] * kLog2e;
    }
    float xv[WIN], dv[WIN];
    {
        float m4[4];
#pragma unroll
        for (int k = 0; k < WIN; ++k) {
            const float xr = a.x[at0 + min(k, cnt - 1) * tstr];
            xv[k] = k < cnt ? xr : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = 4 * hb + j;
            const float z = dtw[min(k, cnt - 1) * H];
            m4[j] = k < cnt ? ssm_step(z, a.softplus) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float mo = dpp<0xB1>(m4[j]);
            dv[j] = hb ? mo : m4[j];
            dv[4 + j] = hb ? m4[j] : mo;
        }
    }
    __syncthreads();
    float yk[WIN];
#pragma unroll
    for (int k = 0; k < WIN; ++k) {
        const float b = dv[k] * xv[k];
        const float ah = APS ? 0.f : dexp2(dv[k] * Ah);
        float y = 0.f;
#pragma unroll
        for (int m = 0; m < NH; ++m) {
            const float aj = APS ? dexp2(dv[k] * Av[m]) : ah;
            sv[m] = fmaf(aj, sv[m], b * bc[0][k][NH * hb + m]);
            y = fmaf(sv[m], bc[1][k][NH * hb + m], y);
        }
        yk[k] = y + dpp<0xB1>(y);
    }
    if (hb == 0) {
#pragma unroll
        for (int k = 0; k < WIN; ++k)
            if (k < cnt) a.y[at0 + k * tstr] = yk[k];
    }
}

// ---- combine: dB, dC over the segments of each group; ddt over the rows of each head ------
// One thread per (sequence, token, group, 4 columns) of dB / dC, summing the group's segments
// in increasing order with eight loads in flight; one per (sequence, token, head) of ddt.
__global__ void __launch_bounds__(256) ssm_combine_kernel(const SsmArgs a) {
    const int64_t T = a.T, H = a.H, G = a.G, N = a.N, P = a.P;
    const int64_t N4 = N / 4;
    const int64_t nbc = (int64_t)a.n_seqs * T * G * N4;    // float4 groups of dB / dC
    // the row-wise backward writes ddt itself when a head is one row
    const int64_t ndt = (a.seg_rows != ROWS && P == 1) ? 0 : (int64_t)a.n_seqs * T * H;
    const int64_t SR = a.seg_rows;                           // rows per segment
    const int64_t K = P * (H / G) / SR;                      // segments per group
    const int64_t kstride = T * 2 * N;                       // floats between segments
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nbc + ndt;
         idx += (int64_t)gridDim.x * blockDim.x) {
        if (idx < nbc) {
            const int64_t n4 = idx % N4, g = (idx / N4) % G, t = (idx / (N4 * G)) % T, s = idx / (N4 * G * T);
            const int64_t seg0 = (s * H * P + g * P * (H / G)) / SR;
            const float *pp = a.part + (seg0 * T + t) * 2 * N + 4 * n4;
            float4 dc = make_float4(0.f, 0.f, 0.f, 0.f), db = dc;
            int64_t k = 0;
            for (; k + 8 <= K; k += 8) {
                float4 c[8], b[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    c[u] = *reinterpret_cast<const float4 *>(pp + (k + u) * kstride);
                    b[u] = *reinterpret_cast<const float4 *>(pp + (k + u) * kstride + N);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    dc.x += c[u].x; dc.y += c[u].y; dc.z += c[u].z; dc.w += c[u].w;
                    db.x += b[u].x; db.y += b[u].y; db.z += b[u].z; db.w += b[u].w;
                }
            }
            for (; k < K; ++k) {
                const float4 c = *reinterpret_cast<const float4 *>(pp + k * kstride);
                const float4 b = *reinterpret_cast<const float4 *>(pp + k * kstride + N);
                dc.x += c.x; dc.y += c.y; dc.z += c.z; dc.w += c.w;
                db.x += b.x; db.y += b.y; db.z += b.z; db.w += b.w;
            }
            const int64_t o = idx * 4;   // dB / dC are [n][T][G][N]: the same flat index
            a.dB[o] = db.x; a.dB[o + 1] = db.y; a.dB[o + 2] = db.z; a.dB[o + 3] = db.w;
            a.dC[o] = dc.x; a.dC[o + 1] = dc.y; a.dC[o + 2] = dc.z; a.dC[o + 3] = dc.w;
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

// (the chain passes address 32 tokens of a row's entries with 32-bit byte offsets from a block's
// first token, so H P and G N stay at most 2^24 floats)
bool ssm_rowwise(int P, int H, int G, int N) {
    return N == 16 && G >= 1 && H % G == 0 && (int64_t)P * (H / G) % RB == 0 &&
           (int64_t)H * P <= (int64_t(1) << 24) && (int64_t)G * N <= (int64_t(1) << 24);
}

hipError_t launch_ssm_rowwise_fwd(const SsmArgs &a, hipStream_t st) {
    const int64_t rows = (int64_t)a.n_seqs * a.H * a.P;
    if (rows <= 0) return hipSuccess;
    const int64_t nwin = (a.T + WIN - 1) / WIN;
    if (!ssm_rowwise(a.P, a.H, a.G, a.N) || a.ckw != 1 || a.nck != nwin + 1) return hipErrorInvalidValue;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    hipError_t e = hipLaunchKernel(a.aps ? (const void *)ssm_sst_kernel<true> : (const void *)ssm_sst_kernel<false>,
                                   dim3((unsigned)(rows / ROWS)), dim3(256), params, 0, st);
    if (e == hipSuccess && a.y && nwin > 0)
        e = hipLaunchKernel(a.aps ? (const void *)ssm_y16_kernel<true> : (const void *)ssm_y16_kernel<false>,
                            dim3((unsigned)(rows / RB * nwin)), dim3(256), params, 0, st);
    return e;
}

hipError_t launch_ssm_rowwise_bwd(const SsmArgs &a, hipStream_t st) {
    const int64_t rows = (int64_t)a.n_seqs * a.H * a.P;
    if (rows <= 0) return hipSuccess;
    if (!ssm_rowwise(a.P, a.H, a.G, a.N) || a.ckw != 1 || a.seg_rows != RB) return hipErrorInvalidValue;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    hipError_t e = hipLaunchKernel(a.aps ? (const void *)ssm_gsw_kernel<true> : (const void *)ssm_gsw_kernel<false>,
                                   dim3((unsigned)(rows / ROWS)), dim3(256), params, 0, st);
    const int64_t nwin = (a.T + WIN - 1) / WIN;
    if (e == hipSuccess && nwin > 0)
        e = hipLaunchKernel(a.aps ? (const void *)ssm_win16_kernel<true> : (const void *)ssm_win16_kernel<false>,
                            dim3((unsigned)(rows / RB * nwin)), dim3(256), params, 0, st);
    if (e == hipSuccess) e = launch_ssm_combine(a, st);
    return e;
}

hipError_t launch_ssm_combine(const SsmArgs &a, hipStream_t st) {
    const bool ddt = !(a.seg_rows != ROWS && a.P == 1);
    const int64_t n = (int64_t)a.n_seqs * a.T * ((int64_t)a.G * a.N / 4 + (ddt ? a.H : 0));
    if (n <= 0) return hipSuccess;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    return hipLaunchKernel((const void *)ssm_combine_kernel, dim3(grid_for(n)), dim3(256), params, 0, st);
}

}  // namespace gdn
