// gdn_kernels.hip -- HIP kernels (gfx950) of the gated delta rule forward scan and its
// checkpointed backward.
//
// Work decomposition.  One workgroup owns one (sequence, value head) unit and its S x S
// fp32 state M = S^T (row j = value index, column i = key index).  Rows of M evolve
// independently in both directions of the recurrence ("metal: GATED_DELTA_NET_BACK",
// approval review: one worker per row of the state), so the state is spread over the
// workgroup by rows:
// a row lives on LPR = 16 lanes (one DPP row), each lane holding NC = S/16 of its columns
// (interleaved, column c = lane%16 + 16 n, so that a token vector load is coalesced), and
// each lane holds R = 4 rows.  A wave therefore holds 4 row groups x 4 rows = 16 rows and
// a unit needs S/16 waves.
//   - Row reductions (u = Mp k, y = M q, dd = dM k) stay inside one DPP row: four DPP adds.
//   - Column reductions (dq, dk, per-channel dg), which sum over rows, go in-lane over the
//     4 rows, across the 4 row groups with permlane16/permlane32 swaps, and across waves
//     through LDS, in a fixed order: no atomics, bitwise reproducible.
// The state and its gradient stay in VGPRs for the whole walk.
//
// Backward schedule (checkpointed recompute, C ~ sqrt(T), PR description of the same page):
// the forward leaves a snapshot of M before tokens 0, C, 2C, ... in the workspace; for each
// segment, last first, the backward replays the segment from its snapshot, keeping the
// decayed previous state Mp = M_{t-1} .* a of every token and the prediction error
// e = v - u of every row, and then walks the segment in reverse (the state after the token
// is rebuilt as Mp + delta k^T, the same fma the forward executed).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

// SK columns (key width), SV rows (value width)
template <int SK, int SV, int R>
struct Layout {
    static constexpr int LPR = 16;         // lanes per row
    static constexpr int NC = SK / LPR;    // columns per lane
    static constexpr int RG = 64 / LPR;    // row groups per wave
    static constexpr int RPW = RG * R;     // rows per wave
    static constexpr int NW = SV / RPW;    // waves per unit
    static constexpr int THREADS = NW * 64;
    static_assert(SV % RPW == 0 && NC >= 1 && SK % LPR == 0, "unsupported head size");
};

__device__ __forceinline__ float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int as_i(float x) { return __builtin_bit_cast(int, x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror: pairs the two quads of each half row
    v += dpp<0x140>(v);  // row_mirror: pairs the two halves of the row
    return v;
}

// Sum over lanes l, l^16, l^32, l^48 (the 4 row groups of a wave); every lane receives it.
__device__ __forceinline__ float groups4_sum(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(as_i(v), as_i(v), false, false);
    v = as_f(p[0]) + as_f(p[1]);
    auto q = __builtin_amdgcn_permlane32_swap(as_i(v), as_i(v), false, false);
    return as_f(q[0]) + as_f(q[1]);
}

// ------------------------------------------------------------------ forward scan

template <int SK, int SV, int R, bool KDA>
__global__ void __launch_bounds__((Layout<SK, SV, R>::THREADS))
fwd_kernel(const FwdArgs a) {
    using Lo = Layout<SK, SV, R>;
    constexpr int NC = Lo::NC, LPR = Lo::LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lc = lane % LPR, rg = lane / LPR;
    const int sl = blockIdx.x / a.H_v, h = blockIdx.x % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int row0 = wave * Lo::RPW + rg * R;
    const int64_t unit = s * a.H_v + h;

    const float *qp = a.q + s * a.sq.seq + hk * a.sq.head + lc;
    const float *kp = a.k + s * a.sk.seq + hk * a.sk.head + lc;
    const float *vp = a.v + s * a.sv.seq + h * a.sv.head + row0;
    const float *gp = a.g + s * a.sg.seq + h * a.sg.head + (KDA ? lc : 0);
    const float *bp = a.beta + s * a.sb.seq + h * a.sb.head;

    float M[R][NC];
    const float *st0 = a.state0 + unit * SV * SK + (int64_t)row0 * SK + lc;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int n = 0; n < NC; ++n) M[r][n] = st0[r * SK + n * LPR];

    float *snap = a.snap + unit * a.n_ck_max * SV * SK + (int64_t)row0 * SK + lc;
    int until_snap = 0;
    // A token's inputs.  Windows of W tokens are loaded one window ahead (two windows per
    // loop trip, so neither buffer is copied): the loads of a window are in flight while the
    // previous one is computed.  Loads past the sequence end are clamped to its last token.
    constexpr int W = NC == 1 ? 8 : (NC == 2 ? 4 : 2);
    struct Tok {
        float q[NC], k[NC], g[KDA ? NC : 1], v[R], beta;
    };
    auto load = [&](Tok (&b)[W], int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int64_t t = min(t0 + w, L - 1);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                b[w].q[n] = qp[t * a.sq.tok + n * LPR];
                b[w].k[n] = kp[t * a.sk.tok + n * LPR];
            }
            if constexpr (KDA) {
#pragma unroll
                for (int n = 0; n < NC; ++n) b[w].g[n] = gp[t * a.sg.tok + n * LPR];
            } else {
                b[w].g[0] = gp[t * a.sg.tok];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) b[w].v[r] = vp[t * a.sv.tok + r];
            b[w].beta = bp[t * a.sb.tok];
        }
    };
    auto step = [&](const Tok &x, int t) __attribute__((always_inline)) {
        if (until_snap == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int n = 0; n < NC; ++n) snap[r * SK + n * LPR] = M[r][n];
            snap += (int64_t)SV * SK;
            until_snap = a.C;
        }
        --until_snap;
        float av[NC];
        if constexpr (KDA) {
#pragma unroll
            for (int n = 0; n < NC; ++n) av[n] = expf(x.g[n]);
        } else {
            const float a0 = expf(x.g[0]);
#pragma unroll
            for (int n = 0; n < NC; ++n) av[n] = a0;
        }
        float ak[NC];
#pragma unroll
        for (int n = 0; n < NC; ++n) ak[n] = av[n] * x.k[n];
        float yr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float u = 0.f;
#pragma unroll
            for (int n = 0; n < NC; ++n) u = fmaf(M[r][n], ak[n], u);
            u = row16_sum(u);
            const float delta = x.beta * (x.v[r] - u);
            float y = 0.f;
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                M[r][n] = fmaf(delta, x.k[n], M[r][n] * av[n]);
                y = fmaf(M[r][n], x.q[n], y);
            }
            yr[r] = y;
        }
        if (a.y) {
#pragma unroll
            for (int r = 0; r < R; ++r) yr[r] = row16_sum(yr[r]);
            if (lc == 0) {
                float *yp = a.y + s * a.sy.seq + (int64_t)t * a.sy.tok + h * a.sy.head + row0;
#pragma unroll
                for (int r = 0; r < R; ++r) yp[r] = a.scale * yr[r];
            }
        }
    };
    Tok bufA[W], bufB[W];
    if (L > 0) load(bufA, 0);
    for (int t0 = 0; t0 < L; t0 += 2 * W) {
        if (t0 + W < L) load(bufB, t0 + W);
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (t0 + w < L) step(bufA[w], t0 + w);
        if (t0 + 2 * W < L) load(bufA, t0 + 2 * W);
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (t0 + W + w < L) step(bufB[w], t0 + W + w);
    }
    if (a.y) {
        for (int64_t t = L; t < a.T; ++t) {
            if (lc == 0) {
                float *yp = a.y + s * a.sy.seq + t * a.sy.tok + h * a.sy.head + row0;
#pragma unroll
                for (int r = 0; r < R; ++r) yp[r] = 0.f;
            }
        }
    }
    if (a.state_out) {
        float *so = a.state_out + unit * SV * SK + (int64_t)row0 * SK + lc;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int n = 0; n < NC; ++n) so[r * SK + n * LPR] = M[r][n];
    }
}

// ------------------------------------------------------------------ backward walk

template <int SK, int SV, int R, bool KDA>
__global__ void __launch_bounds__((Layout<SK, SV, R>::THREADS))
bwd_kernel(const BwdArgs a) {
    using Lo = Layout<SK, SV, R>;
    constexpr int NC = Lo::NC, LPR = Lo::LPR, NW = Lo::NW, RG = Lo::RG;
    constexpr int G = KDA ? SK : 1;
    // column partial sums per wave: [parity][wave][dq | dk | dg][column]
    __shared__ float red[2][NW][3][SK];
    __shared__ float redb[2][NW * RG];   // dbeta partials per row group
    __shared__ float redg[2][NW];        // scalar-gate dg partials per wave

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lc = lane % LPR, rg = lane / LPR;
    const int sl = blockIdx.x / a.H_v, h = blockIdx.x % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int row0 = wave * Lo::RPW + rg * R;
    const int64_t unit = s * a.H_v + h;
    const int C = a.C;

    const float *qp = a.q + s * a.sq.seq + hk * a.sq.head + lc;
    const float *kp = a.k + s * a.sk.seq + hk * a.sk.head + lc;
    const float *vp = a.v + s * a.sv.seq + h * a.sv.head + row0;
    const float *gp = a.g + s * a.sg.seq + h * a.sg.head + (KDA ? lc : 0);
    const float *bp = a.beta + s * a.sb.seq + h * a.sb.head;
    const float *gyp = a.gy + s * a.sgy.seq + h * a.sgy.head + row0;

    float dM[R][NC];
    if (a.dstate_out) {
        const float *d0 = a.dstate_out + unit * SV * SK + (int64_t)row0 * SK + lc;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int n = 0; n < NC; ++n) dM[r][n] = d0[r * SK + n * LPR];
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int n = 0; n < NC; ++n) dM[r][n] = 0.f;
    }

    float *seg = a.segbuf + unit * C * SV * SK + (int64_t)row0 * SK + lc;
    float *eb = a.ebuf_seg + unit * C * SV + row0;
    const int n_ck = (L + C - 1) / C;
    int parity = 0;

    // Token inputs come in windows loaded one window ahead (two windows per loop trip, so no
    // buffer is copied); loads past a segment's end are clamped into the segment.
    constexpr int WR = NC == 1 ? 8 : (NC == 2 ? 4 : 2);    // replay window
    constexpr int WW = NC == 1 ? 4 : (NC == 2 ? 2 : 1);    // walk window
    struct RTok {
        float k[NC], g[KDA ? NC : 1], v[R], beta;
    };
    struct WTok {
        float q[NC], k[NC], g[KDA ? NC : 1], beta, gy[R], e[R], Mp[R][NC];
    };
    auto load_gate = [&](float (&g)[KDA ? NC : 1], int64_t t) __attribute__((always_inline)) {
        if constexpr (KDA) {
#pragma unroll
            for (int n = 0; n < NC; ++n) g[n] = gp[t * a.sg.tok + n * LPR];
        } else {
            g[0] = gp[t * a.sg.tok];
        }
    };
    auto decay = [&](const float (&g)[KDA ? NC : 1], float (&av)[NC]) __attribute__((always_inline)) {
        if constexpr (KDA) {
#pragma unroll
            for (int n = 0; n < NC; ++n) av[n] = expf(g[n]);
        } else {
            const float a0 = expf(g[0]);
#pragma unroll
            for (int n = 0; n < NC; ++n) av[n] = a0;
        }
    };

    for (int sg = n_ck - 1; sg >= 0; --sg) {
        const int t0 = sg * C, t1 = min(t0 + C, L);
        // ---- replay the segment from its snapshot
        {
            float M[R][NC];
            const float *sp = a.snap + (unit * a.n_ck_max + sg) * SV * SK + (int64_t)row0 * SK + lc;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int n = 0; n < NC; ++n) M[r][n] = sp[r * SK + n * LPR];
            auto rload = [&](RTok (&b)[WR], int tb) __attribute__((always_inline)) {
#pragma unroll
                for (int w = 0; w < WR; ++w) {
                    const int64_t t = min(tb + w, t1 - 1);
#pragma unroll
                    for (int n = 0; n < NC; ++n) b[w].k[n] = kp[t * a.sk.tok + n * LPR];
                    load_gate(b[w].g, t);
#pragma unroll
                    for (int r = 0; r < R; ++r) b[w].v[r] = vp[t * a.sv.tok + r];
                    b[w].beta = bp[t * a.sb.tok];
                }
            };
            auto rstep = [&](const RTok &x, int t) __attribute__((always_inline)) {
                float av[NC];
                decay(x.g, av);
                float ak[NC];
#pragma unroll
                for (int n = 0; n < NC; ++n) ak[n] = av[n] * x.k[n];
                float *dst = seg + (int64_t)(t - t0) * SV * SK;
                float *edst = eb + (t - t0) * SV;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float u = 0.f;
#pragma unroll
                    for (int n = 0; n < NC; ++n) u = fmaf(M[r][n], ak[n], u);
                    u = row16_sum(u);
                    const float e = x.v[r] - u;
                    const float delta = x.beta * e;
#pragma unroll
                    for (int n = 0; n < NC; ++n) {
                        const float mp = M[r][n] * av[n];
                        M[r][n] = fmaf(delta, x.k[n], mp);
                        dst[r * SK + n * LPR] = mp;  // keep the decayed previous state
                    }
                    if (lc == 0) edst[r] = e;
                }
            };
            RTok ra[WR], rb[WR];
            rload(ra, t0);
            for (int tb = t0; tb < t1; tb += 2 * WR) {
                if (tb + WR < t1) rload(rb, tb + WR);
#pragma unroll
                for (int w = 0; w < WR; ++w)
                    if (tb + w < t1) rstep(ra[w], tb + w);
                if (tb + 2 * WR < t1) rload(ra, tb + 2 * WR);
#pragma unroll
                for (int w = 0; w < WR; ++w)
                    if (tb + WR + w < t1) rstep(rb[w], tb + WR + w);
            }
        }
        __threadfence_block();
        __syncthreads();

        // ---- reverse walk over the segment
        auto wload = [&](WTok (&b)[WW], int tb) __attribute__((always_inline)) {
#pragma unroll
            for (int w = 0; w < WW; ++w) {
                const int64_t t = max(tb - w, t0);
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    b[w].q[n] = qp[t * a.sq.tok + n * LPR];
                    b[w].k[n] = kp[t * a.sk.tok + n * LPR];
                }
                load_gate(b[w].g, t);
                b[w].beta = bp[t * a.sb.tok];
                const float *src = seg + (int64_t)(t - t0) * SV * SK;
                const float *esrc = eb + (t - t0) * SV;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    b[w].gy[r] = gyp[t * a.sgy.tok + r];
                    b[w].e[r] = esrc[r];
#pragma unroll
                    for (int n = 0; n < NC; ++n) b[w].Mp[r][n] = src[r * SK + n * LPR];
                }
            }
        };
        auto wstep = [&](const WTok &x, int t) __attribute__((always_inline)) {
            float av[NC];
            decay(x.g, av);
            const float beta = x.beta;
            float gyv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) gyv[r] = a.scale * x.gy[r];

            float pq[NC], pk[NC], pg[NC], dd[R];
            float redg_one = 0.f;   // scalar-gate dg of a one-wave unit
            (void)redg_one;
#pragma unroll
            for (int n = 0; n < NC; ++n) pq[n] = pk[n] = pg[n] = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float delta = beta * x.e[r];
                float d = 0.f;
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    const float mt = fmaf(delta, x.k[n], x.Mp[r][n]);  // M_t = Mp + delta k^T
                    dM[r][n] = fmaf(gyv[r], x.q[n], dM[r][n]);       // dM += scale gy q^T
                    pq[n] = fmaf(mt, gyv[r], pq[n]);                 // dq += M_t^T (scale gy)
                    d = fmaf(dM[r][n], x.k[n], d);                   // dd = dM k
                }
                dd[r] = row16_sum(d);
            }
            float pb = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float delta = beta * x.e[r];
                const float du = -beta * dd[r];
                pb = fmaf(dd[r], x.e[r], pb);                        // dbeta = dd . (v - u)
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    pk[n] = fmaf(dM[r][n], delta, pk[n]);            // dk += dM^T delta
                    pk[n] = fmaf(x.Mp[r][n], du, pk[n]);             //     + Mp^T du
                    dM[r][n] = fmaf(du, x.k[n], dM[r][n]);           // dM += du k^T
                    pg[n] = fmaf(dM[r][n], x.Mp[r][n], pg[n]);       // dg = sum dM .* Mp
                    dM[r][n] *= av[n];                               // dM = dM .* a
                }
            }
            if (lc == 0) {
                float *dvp = a.dv + ((s * a.T + t) * a.H_v + h) * SV + row0;
#pragma unroll
                for (int r = 0; r < R; ++r) dvp[r] = beta * dd[r];
                if constexpr (NW > 1) redb[parity][wave * RG + rg] = pb;
            }
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                pq[n] = groups4_sum(pq[n]);
                pk[n] = groups4_sum(pk[n]);
            }
            if constexpr (KDA) {
#pragma unroll
                for (int n = 0; n < NC; ++n) pg[n] = groups4_sum(pg[n]);
            } else {
                float gs = 0.f;
#pragma unroll
                for (int n = 0; n < NC; ++n) gs += pg[n];
                gs = groups4_sum(row16_sum(gs));
                if constexpr (NW == 1) redg_one = 0.f + gs;
                else if (lane == 0) redg[parity][wave] = gs;
            }
            const int64_t row_tok = s * a.T + t;
            if constexpr (NW == 1) {
                // one wave holds every row: the column sums above are complete, stored from
                // registers; dbeta adds the row groups' values in the same order as below
                if (rg == 0) {
#pragma unroll
                    for (int n = 0; n < NC; ++n) {
                        a.dq[(row_tok * a.dqk_head + h) * SK + lc + n * LPR] = pq[n];
                        a.dk[(row_tok * a.dqk_head + h) * SK + lc + n * LPR] = pk[n];
                        if constexpr (KDA) a.dg[(row_tok * a.H_v + h) * G + lc + n * LPR] = pg[n];
                    }
                }
                float pbs = as_f(__builtin_amdgcn_readlane(as_i(pb), 0));
#pragma unroll
                for (int q = 1; q < RG; ++q) pbs += as_f(__builtin_amdgcn_readlane(as_i(pb), q * LPR));
                if (lane == 0) {
                    a.dbeta[row_tok * a.H_v + h] = pbs;
                    if constexpr (!KDA) a.dg[row_tok * a.H_v + h] = redg_one;
                }
                return;
            }
            if (rg == 0) {
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    red[parity][wave][0][lc + n * LPR] = pq[n];
                    red[parity][wave][1][lc + n * LPR] = pk[n];
                    if constexpr (KDA) red[parity][wave][2][lc + n * LPR] = pg[n];
                }
            }
            __syncthreads();
            for (int idx = tid; idx < (KDA ? 3 : 2) * SK; idx += Lo::THREADS) {
                const int which = idx / SK, i = idx % SK;
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) acc += red[parity][w][which][i];
                if (which == 0)
                    a.dq[(row_tok * a.dqk_head + h) * SK + i] = acc;
                else if (which == 1)
                    a.dk[(row_tok * a.dqk_head + h) * SK + i] = acc;
                else
                    a.dg[(row_tok * a.H_v + h) * G + i] = acc;
            }
            if (tid == Lo::THREADS - 1) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < NW * RG; ++w) acc += redb[parity][w];
                a.dbeta[row_tok * a.H_v + h] = acc;
                if constexpr (!KDA) {
                    float g = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) g += redg[parity][w];
                    a.dg[row_tok * a.H_v + h] = g;
                }
            }
            parity ^= 1;
        };
        WTok wa[WW], wb[WW];
        wload(wa, t1 - 1);
        for (int tb = t1 - 1; tb >= t0; tb -= 2 * WW) {
            if (tb - WW >= t0) wload(wb, tb - WW);
#pragma unroll
            for (int w = 0; w < WW; ++w)
                if (tb - w >= t0) wstep(wa[w], tb - w);
            if (tb - 2 * WW >= t0) wload(wa, tb - 2 * WW);
#pragma unroll
            for (int w = 0; w < WW; ++w)
                if (tb - WW - w >= t0) wstep(wb[w], tb - WW - w);
        }
    }

    {
        float *ds = a.dstate + unit * SV * SK + (int64_t)row0 * SK + lc;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int n = 0; n < NC; ++n) ds[r * SK + n * LPR] = dM[r][n];
    }
    // padded tokens: every per-token output row of this unit is written zero
    for (int64_t t = L; t < a.T; ++t) {
        const int64_t row_tok = s * a.T + t;
        for (int i = tid; i < SK; i += Lo::THREADS) {
            a.dq[(row_tok * a.dqk_head + h) * SK + i] = 0.f;
            a.dk[(row_tok * a.dqk_head + h) * SK + i] = 0.f;
        }
        for (int i = tid; i < SV; i += Lo::THREADS) a.dv[(row_tok * a.H_v + h) * SV + i] = 0.f;
        for (int i = tid; i < G; i += Lo::THREADS) a.dg[(row_tok * a.H_v + h) * G + i] = 0.f;
        if (tid == 0) a.dbeta[row_tok * a.H_v + h] = 0.f;
    }
}

// ------------------------------------------------------------------ grouped-head sum

__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs a) {
    const int64_t total = (int64_t)a.n_seqs * a.T * a.H_k * a.S;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int i = (int)(idx % a.S);
        const int64_t rest = idx / a.S;
        const int hk = (int)(rest % a.H_k);
        const int64_t st = rest / a.H_k;
        float q = 0.f, k = 0.f;
        for (int h = hk; h < a.H_v; h += a.H_k) {  // increasing value head
            const int64_t src = (st * a.H_v + h) * a.S + i;
            q += a.dq_part[src];
            k += a.dk_part[src];
        }
        a.dq[idx] = q;
        a.dk[idx] = k;
    }
}

// ------------------------------------------------------------------ half-precision inputs

// dst[s][t][h][i] = src(s, t, h, i) widened to fp32 (exact for both half formats).  A thread
// handles 8 consecutive elements of one row: one 16-byte load and two 16-byte stores when
// VEC (the host checked that every row start is 16-byte aligned and W is a multiple of 8).
__device__ __forceinline__ float widen1(uint16_t b, bool bf16) {
    return bf16 ? __builtin_bit_cast(float, (uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
}

template <bool VEC>
__global__ void __launch_bounds__(256) widen_kernel(const WidenArgs a) {
    const int64_t chunks = (a.W + 7) / 8;
    const int64_t total = a.n * a.T * a.H * chunks;
    const bool bf16 = a.bf16 != 0;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = idx % chunks, row = idx / chunks;
        const int64_t h = row % a.H, st = row / a.H;
        const int64_t t = st % a.T, s = st / a.T;
        const uint16_t *src = a.src + s * a.st.seq + t * a.st.tok + h * a.st.head + c * 8;
        float *dst = a.dst + row * a.W + c * 8;
        if constexpr (VEC) {
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[2 * j] = widen1((uint16_t)(w4[j] & 0xFFFFu), bf16);
                f[2 * j + 1] = widen1((uint16_t)(w4[j] >> 16), bf16);
            }
            reinterpret_cast<float4 *>(dst)[0] = make_float4(f[0], f[1], f[2], f[3]);
            reinterpret_cast<float4 *>(dst)[1] = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            const int m = (int)min<int64_t>(8, a.W - c * 8);
            for (int j = 0; j < m; ++j) dst[j] = widen1(src[j], bf16);
        }
    }
}

template <typename Args>
hipError_t launch(const void *fn, const Args &args, int blocks, int threads, hipStream_t st) {
    if (blocks <= 0) return hipSuccess;
    void *params[] = {const_cast<Args *>(&args)};
    return hipLaunchKernel(fn, dim3(blocks), dim3(threads), params, 0, st);
}

template <int SK, int SV, int R>
constexpr int kThreads = Layout<SK, SV, R>::THREADS;

// Rows per lane.  The forward's rows are independent, so it spreads a unit over more waves
// (one row per lane group up to 64 rows): the scan is one serial chain per wave, and with a
// few hundred units on 1024 SIMDs more, shorter waves finish sooner.  The backward keeps four
// rows per lane (its column sums cross waves through LDS once per token).
template <bool FWD, int SV>
constexpr int kRows = FWD ? (SV <= 64 ? 1 : 2) : 4;

// Launch a kernel template over the supported (key width, value width) pairs: every pair of
// {16, 32, 64, 128} except 128 x 128 (the row-quarter kernels of gdn_s128.hip).
template <bool FWD, int SK, int SV, typename Args, typename Pick>
hipError_t launch_pair(const Args &a, bool kda, int blocks, hipStream_t st, Pick pick) {
    if constexpr (SK == 128 && SV == 128) {
        return hipErrorInvalidValue;
    } else {
        constexpr int R = kRows<FWD, SV>;
        return launch(pick(std::integral_constant<int, SK>{}, std::integral_constant<int, SV>{},
                           std::integral_constant<int, R>{}, kda),
                      a, blocks, kThreads<SK, SV, R>, st);
    }
}

template <bool FWD, int SK, typename Args, typename Pick>
hipError_t launch_sv(const Args &a, int SV, bool kda, int blocks, hipStream_t st, Pick pick) {
    switch (SV) {
        case 16: return launch_pair<FWD, SK, 16>(a, kda, blocks, st, pick);
        case 32: return launch_pair<FWD, SK, 32>(a, kda, blocks, st, pick);
        case 64: return launch_pair<FWD, SK, 64>(a, kda, blocks, st, pick);
        case 128: return launch_pair<FWD, SK, 128>(a, kda, blocks, st, pick);
    }
    return hipErrorInvalidValue;
}

template <bool FWD, typename Args, typename Pick>
hipError_t launch_sizes(const Args &a, int SK, int SV, bool kda, int blocks, hipStream_t st, Pick pick) {
    switch (SK) {
        case 16: return launch_sv<FWD, 16>(a, SV, kda, blocks, st, pick);
        case 32: return launch_sv<FWD, 32>(a, SV, kda, blocks, st, pick);
        case 64: return launch_sv<FWD, 64>(a, SV, kda, blocks, st, pick);
        case 128: return launch_sv<FWD, 128>(a, SV, kda, blocks, st, pick);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int SK, int SV, bool kda, int n_seqs_launch, hipStream_t st) {
    return launch_sizes<true>(a, SK, SV, kda, n_seqs_launch * a.H_v, st, [](auto sk, auto sv, auto r, bool k) {
        constexpr int K = decltype(sk)::value, V = decltype(sv)::value, RR = decltype(r)::value;
        return k ? (const void *)fwd_kernel<K, V, RR, true> : (const void *)fwd_kernel<K, V, RR, false>;
    });
}

hipError_t launch_bwd(const BwdArgs &a, int SK, int SV, bool kda, int n_seqs_launch, hipStream_t st) {
    return launch_sizes<false>(a, SK, SV, kda, n_seqs_launch * a.H_v, st, [](auto sk, auto sv, auto r, bool k) {
        constexpr int K = decltype(sk)::value, V = decltype(sv)::value, RR = decltype(r)::value;
        return k ? (const void *)bwd_kernel<K, V, RR, true> : (const void *)bwd_kernel<K, V, RR, false>;
    });
}

hipError_t launch_widen(const WidenArgs &a, hipStream_t st) {
    const int64_t total = a.n * a.T * a.H * ((a.W + 7) / 8);
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    // 16-byte vectors when every row start is 16-byte aligned (the fp32 rows then are too)
    const bool vec = a.W % 8 == 0 && ((uintptr_t)a.src & 15) == 0 && a.st.seq % 8 == 0 &&
                     a.st.tok % 8 == 0 && a.st.head % 8 == 0 && ((uintptr_t)a.dst & 15) == 0;
    return vec ? launch((const void *)widen_kernel<true>, a, (int)blocks, 256, st)
               : launch((const void *)widen_kernel<false>, a, (int)blocks, 256, st);
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.n_seqs * a.T * a.H_k * a.S;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    return launch((const void *)combine_kernel, a, (int)blocks, 256, st);
}

}  // namespace gdn
