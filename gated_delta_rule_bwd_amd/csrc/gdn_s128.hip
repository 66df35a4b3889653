// gdn_s128.hip -- gfx950 kernels of the gated delta rule for head size S = 128.
//
// Work decomposition.  A (sequence, value head) unit owns a 128 x 128 fp32 state M = S^T
// (row j = value index, column i = key index).  Rows evolve independently in both
// directions of the recurrence ("metal: GATED_DELTA_NET_BACK", approval review: thread j
// owns row j of M), so each unit is split into four row quarters of 32 rows and every
// quarter is one workgroup of four waves (eight rows per wave).  At the layer shape
// (192 units) that is 768 workgroups: three per compute unit, so all 256 CUs carry equal
// work.  The only coupling between quarters is the set of column sums of the backward
// (dq, dk and the per-channel dg sum over rows, dbeta over rows); each quarter writes its
// partial sums and a fixed-order kernel adds the four quarters (and, for dq/dk, the value
// heads of each key head in increasing order), so results are bitwise reproducible.
//
// Forward (fwd128_kernel): lanes are laid out as 16 lanes per row (one DPP row) with eight
// contiguous columns per lane and two rows per lane, so the two row reductions per token
// (u = Mp k and y = M q) are four DPP adds each.  Token vectors are staged through LDS in
// chunks of 8 tokens.  Besides y, the final state and the snapshots every C tokens, the
// forward saves two per-token vectors to the workspace: the gates a = exp(g) and the
// prediction errors e = v - u of every row.  With e saved, replaying a token is just
// Mp = M .* a, M = Mp + (beta e) k^T, bit-identical to the forward's own arithmetic.
//
// Backward (bwd128_kernel): lanes are laid out as 64 lanes per row with two columns per
// lane (columns lane and lane + 64) and eight rows per lane, so every column sum is in-lane
// and the only row reduction per token (dd = dM k) is a permlane/DPP reduce-scatter followed
// by v_readlane broadcasts.  The checkpointed schedule has three storage levels:
//   - snapshots every C tokens in HBM (from the forward),
//   - states every 8 tokens inside a 64-token stretch, in registers (a 64-token stretch
//     longer segments are cut into starts from a state saved to the workspace),
//   - the decayed previous states Mp of the 8 tokens being walked, in LDS (128 KiB).
// A replay pass over each 64-token stretch records the 8-token states, then each 8-token
// sub-segment, last first, is replayed into LDS and walked in reverse.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int S = 128;
constexpr int QR = 32;         // rows per workgroup (one row quarter)
constexpr int NQ = S / QR;     // quarters per unit
constexpr int THREADS = 256;   // four waves
constexpr int TC = 8;          // tokens per staged chunk in the forward
constexpr int C2 = 8;          // tokens per sub-segment walked from LDS
constexpr int VS = 64;         // tokens per stretch with register-resident sub-snapshots
constexpr int NSUB = VS / C2;  // sub-snapshots per stretch

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
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}

// Sum over all 64 lanes; every lane receives the sum.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    auto p = __builtin_amdgcn_permlane16_swap(as_i(v), as_i(v), false, false);
    v = as_f(p[0]) + as_f(p[1]);
    auto q = __builtin_amdgcn_permlane32_swap(as_i(v), as_i(v), false, false);
    return as_f(q[0]) + as_f(q[1]);
}

// Eight per-lane partial sums d[0..7] (one per row) reduced over the 64 lanes; returns the
// eight row totals as wave-uniform values.  permlane32_swap(A, B) yields ([A_lo|B_lo],
// [A_hi|B_hi]) and permlane16_swap(A, B) yields ([A0,B0,A2,B2], [A1,B1,A3,B3]) over the
// four 16-lane rows, so after the two swap stages the 16-lane rows of g0 hold the partials
// of rows 0, 2, 1, 3 and those of g1 rows 4, 6, 5, 7.
__device__ __forceinline__ void rows8_sum(const float (&d)[8], float (&out)[8]) {
    float h[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        auto sw = __builtin_amdgcn_permlane32_swap(as_i(d[2 * p]), as_i(d[2 * p + 1]), false, false);
        h[p] = as_f(sw[0]) + as_f(sw[1]);
    }
    float g[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        auto sw = __builtin_amdgcn_permlane16_swap(as_i(h[2 * p]), as_i(h[2 * p + 1]), false, false);
        g[p] = row16_sum(as_f(sw[0]) + as_f(sw[1]));
    }
    out[0] = as_f(__builtin_amdgcn_readlane(as_i(g[0]), 0));
    out[2] = as_f(__builtin_amdgcn_readlane(as_i(g[0]), 16));
    out[1] = as_f(__builtin_amdgcn_readlane(as_i(g[0]), 32));
    out[3] = as_f(__builtin_amdgcn_readlane(as_i(g[0]), 48));
    out[4] = as_f(__builtin_amdgcn_readlane(as_i(g[1]), 0));
    out[6] = as_f(__builtin_amdgcn_readlane(as_i(g[1]), 16));
    out[5] = as_f(__builtin_amdgcn_readlane(as_i(g[1]), 32));
    out[7] = as_f(__builtin_amdgcn_readlane(as_i(g[1]), 48));
}

// Block index -> (unit within the launch, row quarter).  The four quarters of a unit read
// the same token vectors, so they are placed on the same XCD (blocks are dispatched to the
// eight XCDs round robin) when the grid allows it.
__device__ __forceinline__ void map_block(int b, int nb, int &unit, int &qb) {
    int lin = b;
    if (nb % (8 * NQ) == 0) lin = (b % 8) * (nb / 8) + b / 8;
    unit = lin / NQ;
    qb = lin % NQ;
}

// ------------------------------------------------------------------ forward scan

template <bool KDA>
__global__ void __launch_bounds__(THREADS)
fwd128_kernel(const FwdArgs a) {
    constexpr int GW = KDA ? S : 1;
    __shared__ float qs[2][TC][S], ks[2][TC][S], gs[2][TC][GW];
    __shared__ float vs[2][TC][QR], bs[2][TC];
    __shared__ float ys[TC][QR], es[TC][QR];

    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lc = lane & 15, rg = lane >> 4;
    const int lr0 = w * 8 + rg * 2;           // first local row of this lane (two rows)
    const int row0 = qb * QR + lr0;           // first global row
    const bool write_y = a.y != nullptr;

    const float *qp = a.q + s * a.sq.seq + hk * a.sq.head;
    const float *kp = a.k + s * a.sk.seq + hk * a.sk.head;
    const float *gp = a.g + s * a.sg.seq + h * a.sg.head;
    const float *vp = a.v + s * a.sv.seq + h * a.sv.head + qb * QR;
    const float *bp = a.beta + s * a.sb.seq + h * a.sb.head;
    const int64_t tok_ae = (int64_t)a.H_v;   // token stride of abuf / ebuf rows, in rows
    float *abase = a.abuf + (s * a.T * a.H_v + h) * GW;
    float *ebase = a.ebuf + (s * a.T * a.H_v + h) * S + qb * QR;

    float M[2][8];
    {
        const float *st0 = a.state0 + unit * S * S + (int64_t)row0 * S + lc * 8;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int n = 0; n < 8; ++n) M[r][n] = st0[r * S + n];
    }

    // staging: thread -> (token tt of the chunk, four consecutive columns cc)
    const int stt = tid >> 5, scc = (tid & 31) * 4, srow = tid & 31;
    float rq[4], rk[4], rg4[4], rv = 0.f, rb = 0.f;
    auto load_chunk = [&](int c) {
        const int t = c * TC + stt;
        const bool ok = t < L;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rq[i] = ok ? qp[t * a.sq.tok + scc + i] : 0.f;
            rk[i] = ok ? kp[t * a.sk.tok + scc + i] : 0.f;
            if constexpr (KDA) rg4[i] = ok ? gp[t * a.sg.tok + scc + i] : 0.f;
        }
        rv = ok ? vp[t * a.sv.tok + srow] : 0.f;
        if (tid < TC) {
            const int tb = c * TC + tid;
            rb = tb < L ? bp[tb * a.sb.tok] : 0.f;
        } else if (!KDA && tid < 2 * TC) {
            const int tb = c * TC + tid - TC;
            rb = tb < L ? gp[tb * a.sg.tok] : 0.f;
        }
    };
    auto store_chunk = [&](int c, int buf) {
        const int t = c * TC + stt;
        const bool ok = t < L;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qs[buf][stt][scc + i] = rq[i];
            ks[buf][stt][scc + i] = rk[i];
        }
        if constexpr (KDA) {
            float av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = expf(rg4[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) gs[buf][stt][scc + i] = av[i];
            if (qb == 0 && ok) {
#pragma unroll
                for (int i = 0; i < 4; ++i) abase[t * tok_ae * GW + scc + i] = av[i];
            }
        }
        vs[buf][stt][srow] = rv;
        if (tid < TC) {
            bs[buf][tid] = rb;
        } else if (!KDA && tid < 2 * TC) {
            const float av = expf(rb);
            gs[buf][tid - TC][0] = av;
            const int tb = c * TC + tid - TC;
            if (qb == 0 && tb < L) abase[tb * tok_ae] = av;
        }
    };

    const int nchunks = (L + TC - 1) / TC;
    float *snap = a.snap + unit * a.n_ck_max * S * S + (int64_t)row0 * S + lc * 8;
    int next_snap = 0;
    if (nchunks > 0) {
        load_chunk(0);
        store_chunk(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < nchunks) load_chunk(c + 1);
        const int cnt = min(TC, L - c * TC);
        for (int tt = 0; tt < cnt; ++tt) {
            const int t = c * TC + tt;
            if (t == next_snap) {
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int n = 0; n < 8; ++n) snap[r * S + n] = M[r][n];
                snap += (int64_t)S * S;
                next_snap += a.C;
            }
            float qv[8], kv[8], av[8];
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                qv[n] = qs[buf][tt][lc * 8 + n];
                kv[n] = ks[buf][tt][lc * 8 + n];
                av[n] = gs[buf][tt][KDA ? lc * 8 + n : 0];
            }
            const float beta = bs[buf][tt];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float vr = vs[buf][tt][lr0 + r];
                float mp[8], u = 0.f;
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    mp[n] = M[r][n] * av[n];
                    u = fmaf(mp[n], kv[n], u);
                }
                u = row16_sum(u);
                const float e = vr - u;
                const float de = beta * e;
                float y = 0.f;
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    M[r][n] = fmaf(de, kv[n], mp[n]);
                    y = fmaf(M[r][n], qv[n], y);
                }
                y = row16_sum(y);
                if (lc == 0) {
                    ys[tt][lr0 + r] = a.scale * y;
                    es[tt][lr0 + r] = e;
                }
            }
        }
        __syncthreads();
        if (stt < cnt) {
            const int64_t t = c * TC + stt;
            if (write_y)
                a.y[s * a.sy.seq + t * a.sy.tok + h * a.sy.head + qb * QR + srow] = ys[stt][srow];
            ebase[t * tok_ae * S + srow] = es[stt][srow];
        }
        if (c + 1 < nchunks) store_chunk(c + 1, buf ^ 1);
        __syncthreads();
    }
    if (write_y) {
        for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += THREADS) {
            const int64_t t = L + idx / QR;
            a.y[s * a.sy.seq + t * a.sy.tok + h * a.sy.head + qb * QR + idx % QR] = 0.f;
        }
    }
    if (a.state_out) {
        float *so = a.state_out + unit * S * S + (int64_t)row0 * S + lc * 8;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int n = 0; n < 8; ++n) so[r * S + n] = M[r][n];
    }
}

// ------------------------------------------------------------------ backward walk

// Token data of one chunk of C2 tokens, staged in LDS for the four waves of a workgroup.
template <int GW>
struct TokStage {
    float q[C2][S];
    float k[C2][S];
    float a[C2][GW];
    float e[C2][QR];     // prediction errors of this quarter's rows
    float gy[C2][QR];    // output cotangent of this quarter's rows
    float beta[C2];
};

template <bool KDA>
__global__ void __launch_bounds__(THREADS, 1)
bwd128_kernel(const BwdArgs a) {
    constexpr int GW = KDA ? S : 1;
    constexpr int NP = KDA ? 3 : 2;   // partial slots per quarter: dq | dk (| dg)
    // decayed previous states of one sub-segment; after its walk the same memory holds the
    // per-wave column sums of the sub-segment's tokens until they are reduced
    __shared__ float4 mp_lds[C2][4][THREADS];
    __shared__ float redb[C2][4], redg[C2][4];  // per-wave dbeta and scalar-gate dg
    __shared__ TokStage<GW> ts;

    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row0 = qb * QR + w * 8;   // eight rows of this wave
    const int C = a.C;

    const float *snapu = a.snap + unit * a.n_ck_max * S * S + (int64_t)row0 * S + lane;
    float4 *vsb = reinterpret_cast<float4 *>(a.vsbuf) +
                  ((unit * NQ + qb) * (int64_t)a.nvs_max) * (4 * THREADS) + tid;

    // ---- staging of token data: thread -> (token stt of the chunk, 4 columns scc, row srow)
    const int stt = tid >> 5, scc = (tid & 31) * 4, srow = tid & 31;
    const float *qp = a.q + s * a.sq.seq + hk * a.sq.head + scc;
    const float *kp = a.k + s * a.sk.seq + hk * a.sk.head + scc;
    const float *ap = a.abuf + (s * a.T * a.H_v + h) * GW + (KDA ? scc : 0);
    const float *ep = a.ebuf + (s * a.T * a.H_v + h) * S + qb * QR + srow;
    const float *gyp = a.gy + s * a.sgy.seq + h * a.sgy.head + qb * QR + srow;
    const float *bp = a.beta + s * a.sb.seq + h * a.sb.head;
    const int64_t tok_ae = a.H_v;
    float pq4[4], pk4[4], pa4[4], pe = 0.f, pgy = 0.f, pb1 = 0.f;
    int pcnt = 0;
    auto load_chunk = [&](int tstart, int cnt, bool walk) {
        pcnt = cnt;
        const int t = tstart + stt;
        if (stt < cnt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pk4[i] = kp[t * a.sk.tok + i];
                if (walk) pq4[i] = qp[t * a.sq.tok + i];
                if constexpr (KDA) pa4[i] = ap[t * tok_ae * GW + i];
            }
            pe = ep[t * tok_ae * S];
            if (walk) pgy = gyp[t * a.sgy.tok];
        }
        if (tid < cnt) {
            pb1 = bp[(tstart + tid) * a.sb.tok];
        } else if (!KDA && tid >= C2 && tid < C2 + cnt) {
            pb1 = ap[(tstart + tid - C2) * tok_ae];
        }
    };
    auto store_chunk = [&](bool walk) {
        if (stt < pcnt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ts.k[stt][scc + i] = pk4[i];
                if (walk) ts.q[stt][scc + i] = pq4[i];
                if constexpr (KDA) ts.a[stt][scc + i] = pa4[i];
            }
            ts.e[stt][srow] = pe;
            if (walk) ts.gy[stt][srow] = pgy;
        }
        if (tid < pcnt) {
            ts.beta[tid] = pb1;
        } else if (!KDA && tid >= C2 && tid < C2 + pcnt) {
            ts.a[tid - C2][0] = pb1;
        }
    };

    float X[8][2];
    if (a.dstate_out) {
        const float *d0 = a.dstate_out + unit * S * S + (int64_t)row0 * S + lane;
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) X[r][n] = d0[r * S + n * 64];
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) X[r][0] = X[r][1] = 0.f;
    }

    // one replayed token from the staged chunk: Mp = M .* a; M = Mp + (beta e) k^T
    auto replay = [&](int tt, float (&M)[8][2], float4 *slot) {
        float kv[2], av[2], ev[8];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            kv[n] = ts.k[tt][lane + 64 * n];
            av[n] = ts.a[tt][KDA ? lane + 64 * n : 0];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) ev[r] = ts.e[tt][w * 8 + r];
        const float beta = ts.beta[tt];
        float mp[8][2];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float de = beta * ev[r];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                mp[r][n] = M[r][n] * av[n];
                M[r][n] = fmaf(de, kv[n], mp[r][n]);
            }
        }
        if (slot) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                slot[c * THREADS] = make_float4(mp[2 * c][0], mp[2 * c][1],
                                                mp[2 * c + 1][0], mp[2 * c + 1][1]);
        }
    };

    // one token of the reverse walk (token t, chunk position tt).  Once a thread has read its
    // LDS state of token tt it owns that slot again, so it leaves its column sums of the
    // token there (dq, dk, dg for its two columns in the first two float4 of the slot) for the
    // reduction at the end of the sub-segment.
    auto walk = [&](int t, int tt) {
        const float4 *slot = &mp_lds[tt][0][tid];
        float Mp[8][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 v = slot[c * THREADS];
            Mp[2 * c][0] = v.x; Mp[2 * c][1] = v.y; Mp[2 * c + 1][0] = v.z; Mp[2 * c + 1][1] = v.w;
        }
        float qs[2], kv[2], kn[2], av[2], gy[8], ev[8];
        const float beta = ts.beta[tt];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            qs[n] = a.scale * ts.q[tt][lane + 64 * n];
            kv[n] = ts.k[tt][lane + 64 * n];
            kn[n] = -beta * kv[n];
            av[n] = ts.a[tt][KDA ? lane + 64 * n : 0];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            gy[r] = ts.gy[tt][w * 8 + r];
            ev[r] = ts.e[tt][w * 8 + r];
        }
        float pq[2] = {0.f, 0.f}, pe2[2] = {0.f, 0.f}, pm[2] = {0.f, 0.f}, pg[2] = {0.f, 0.f};
        float dpart[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float de = beta * ev[r];
            dpart[r] = 0.f;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float mt = fmaf(de, kv[n], Mp[r][n]);    // state after token t
                X[r][n] = fmaf(gy[r], qs[n], X[r][n]);         // dM += scale gy q^T
                pq[n] = fmaf(mt, gy[r], pq[n]);                // dq  (x scale below)
                pe2[n] = fmaf(X[r][n], de, pe2[n]);            // dk: dM^T delta
                dpart[r] = fmaf(X[r][n], kv[n], dpart[r]);     // dd = dM k
            }
        }
        float dd[8];
        rows8_sum(dpart, dd);
        float pb = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            pb = fmaf(dd[r], ev[r], pb);                       // dbeta = dd . (v - u)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                pm[n] = fmaf(Mp[r][n], dd[r], pm[n]);          // Mp^T dd (du = -beta dd)
                X[r][n] = fmaf(dd[r], kn[n], X[r][n]);         // dM += du k^T
                pg[n] = fmaf(X[r][n], Mp[r][n], pg[n]);        // dg = sum dM .* Mp
                X[r][n] *= av[n];                              // dM = dM .* a
            }
        }
        if (lane == 0) {
            float *dvp = a.dv + ((s * a.T + t) * a.H_v + h) * S + row0;
#pragma unroll
            for (int r = 0; r < 8; ++r) dvp[r] = beta * dd[r];
        }
        float4 *own = &mp_lds[tt][0][tid];
        own[0] = make_float4(a.scale * pq[0], a.scale * pq[1], fmaf(-beta, pm[0], pe2[0]),
                             fmaf(-beta, pm[1], pe2[1]));
        if constexpr (KDA) own[THREADS] = make_float4(pg[0], pg[1], 0.f, 0.f);
        if constexpr (!KDA) {
            const float gs = wave_sum(pg[0] + pg[1]);
            if (lane == 0) redg[tt][w] = gs;
        }
        if (lane == 0) redb[tt][w] = pb;
    };
    // the column sums of the cnt walked tokens starting at token ta, summed over the four
    // waves in a fixed order and written to the quarter's partial buffers
    auto reduce_columns = [&](int ta, int cnt) {
        __syncthreads();   // every wave has left its column sums in the LDS slots
        const float *lds = reinterpret_cast<const float *>(&mp_lds[0][0][0]);
        for (int idx = tid; idx < cnt * NP * S; idx += THREADS) {
            const int tt = idx / (NP * S), rem = idx % (NP * S);
            const int which = rem / S, c = rem % S;
            // value (which, column c) of wave w sits in thread w*64 + c%64 at component
            // 2*which + c/64 of its first two float4 of slot tt
            const int comp = 2 * which + (c >> 6);
            const float *base = lds + ((tt * 4 + (comp >> 2)) * THREADS + (c & 63)) * 4 + (comp & 3);
            a.part[(((s * a.T + ta + tt) * a.H_v + h) * NQ + qb) * NP * S + which * S + c] =
                ((base[0] + base[64 * 4]) + base[128 * 4]) + base[192 * 4];
        }
        if (tid < cnt) {
            const int64_t rt = ((s * a.T + ta + tid) * a.H_v + h) * NQ + qb;
            a.pbuf[rt] = ((redb[tid][0] + redb[tid][1]) + redb[tid][2]) + redb[tid][3];
            if constexpr (!KDA)
                a.pgbuf[rt] = ((redg[tid][0] + redg[tid][1]) + redg[tid][2]) + redg[tid][3];
        }
        __syncthreads();   // LDS slots free for the next sub-segment
    };

    auto load_state = [&](const float *src, float (&M)[8][2]) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) M[r][n] = src[r * S + n * 64];
    };

    const int n_ck = (L + C - 1) / C;
    for (int sg = n_ck - 1; sg >= 0; --sg) {
        const int t0 = sg * C, t1 = min(t0 + C, L);
        const int nvs = (t1 - t0 + VS - 1) / VS;
        float M[8][2];
        load_state(snapu + (int64_t)sg * S * S, M);
        // stretch starts beyond the first: replay once and keep them in the workspace
        if (nvs > 1) {
            const int tend = t0 + VS * (nvs - 1);
            load_chunk(t0, C2, false);
            __syncthreads();
            store_chunk(false);
            __syncthreads();
            for (int tc = t0; tc < tend; tc += C2) {
                if (tc > t0 && (tc - t0) % VS == 0) {
                    float4 *dst = vsb + (int64_t)((tc - t0) / VS) * (4 * THREADS);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        dst[c * THREADS] = make_float4(M[2 * c][0], M[2 * c][1], M[2 * c + 1][0],
                                                       M[2 * c + 1][1]);
                }
                if (tc + C2 < tend) load_chunk(tc + C2, C2, false);
                for (int tt = 0; tt < C2; ++tt) replay(tt, M, nullptr);
                __syncthreads();
                if (tc + C2 < tend) store_chunk(false);
                __syncthreads();
            }
        }
        for (int v = nvs - 1; v >= 0; --v) {
            const int va = t0 + v * VS, vb = min(va + VS, t1);
            const int nsub = (vb - va + C2 - 1) / C2;
            if (v < nvs - 1) {
                if (v == 0) {
                    load_state(snapu + (int64_t)sg * S * S, M);
                } else {
                    const float4 *src = vsb + (int64_t)v * (4 * THREADS);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float4 x = src[c * THREADS];
                        M[2 * c][0] = x.x; M[2 * c][1] = x.y; M[2 * c + 1][0] = x.z; M[2 * c + 1][1] = x.w;
                    }
                }
            }
            // first chunk of the stretch: L1 chunk 0, or the walk of the only sub-segment
            auto cnt_of = [&](int j) { return min(C2, vb - (va + j * C2)); };
            load_chunk(va, nsub > 1 ? C2 : cnt_of(0), nsub == 1);
            __syncthreads();
            store_chunk(nsub == 1);
            __syncthreads();
            // replay the stretch, keeping the state every C2 tokens in registers
            float SS[NSUB][8][2];
#pragma unroll
            for (int r = 0; r < 8; ++r) SS[0][r][0] = M[r][0], SS[0][r][1] = M[r][1];
#pragma unroll
            for (int j = 0; j < NSUB - 1; ++j) {
                if (j < nsub - 1) {
                    const bool next_walk = j + 1 == nsub - 1;
                    load_chunk(va + (j + 1) * C2, next_walk ? cnt_of(j + 1) : C2, next_walk);
                    for (int tt = 0; tt < C2; ++tt) replay(tt, M, nullptr);
#pragma unroll
                    for (int r = 0; r < 8; ++r) SS[j + 1][r][0] = M[r][0], SS[j + 1][r][1] = M[r][1];
                    __syncthreads();
                    store_chunk(next_walk);
                    __syncthreads();
                }
            }
            // sub-segments last first: replay into LDS, then walk in reverse
#pragma unroll
            for (int j = NSUB - 1; j >= 0; --j) {
                if (j < nsub) {
                    if (j > 0) load_chunk(va + (j - 1) * C2, C2, true);
#pragma unroll
                    for (int r = 0; r < 8; ++r) M[r][0] = SS[j][r][0], M[r][1] = SS[j][r][1];
                    const int ta = va + j * C2, cnt = cnt_of(j);
                    for (int tt = 0; tt < cnt; ++tt) replay(tt, M, &mp_lds[tt][0][tid]);
                    for (int tt = cnt - 1; tt >= 0; --tt) walk(ta + tt, tt);
                    reduce_columns(ta, cnt);
                    if (j > 0) store_chunk(true);
                    __syncthreads();
                }
            }
        }
    }

    {
        float *ds = a.dstate + unit * S * S + (int64_t)row0 * S + lane;
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) ds[r * S + n * 64] = X[r][n];
    }
    for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += THREADS) {
        const int64_t t = L + idx / QR;
        a.dv[((s * a.T + t) * a.H_v + h) * S + qb * QR + idx % QR] = 0.f;
    }
}

// ------------------------------------------------------------------ quarter / head sums

__global__ void __launch_bounds__(256) combine128_kernel(const Combine128Args a) {
    const int64_t T = a.T, n = a.n_seqs_launch, Hk = a.H_k, Hv = a.H_v;
    const int64_t G = a.kda ? S : 1;
    const int64_t n_qk = n * T * Hk * S;   // dq and dk elements (each)
    const int64_t n_g = n * T * Hv * G;    // dg elements
    const int64_t n_b = n * T * Hv;        // dbeta elements
    const int64_t NP = a.kda ? 3 : 2;
    const int64_t total = n_qk + n_g + n_b;
    const int64_t seq0 = (int64_t)a.s_base;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        if (idx < n_qk) {
            const int i = (int)(idx % S);
            int64_t rest = idx / S;
            const int kh = (int)(rest % Hk);
            rest /= Hk;
            const int t = (int)(rest % T);
            const int sl = (int)(rest / T);
            float q = 0.f, k = 0.f;
            if (t < a.lens[sl]) {
                for (int h = kh; h < Hv; h += (int)Hk) {   // value heads in increasing order
                    const float *pp = a.part + ((((seq0 + sl) * T + t) * Hv + h) * NQ) * NP * S + i;
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        q += pp[(qb * NP + 0) * S];
                        k += pp[(qb * NP + 1) * S];
                    }
                }
            }
            const int64_t o = (((seq0 + sl) * T + t) * Hk + kh) * S + i;
            a.dq[o] = q;
            a.dk[o] = k;
        } else if (idx < n_qk + n_g) {
            const int64_t j = idx - n_qk;
            const int i = (int)(j % G);
            int64_t rest = j / G;
            const int h = (int)(rest % Hv);
            rest /= Hv;
            const int t = (int)(rest % T);
            const int sl = (int)(rest / T);
            float g = 0.f;
            if (t < a.lens[sl]) {
                const int64_t rt = (((seq0 + sl) * T + t) * Hv + h) * NQ;
#pragma unroll
                for (int qb = 0; qb < NQ; ++qb)
                    g += a.kda ? a.part[((rt + qb) * NP + 2) * S + i] : a.pgbuf[rt + qb];
            }
            a.dg[(((seq0 + sl) * T + t) * Hv + h) * G + i] = g;
        } else {
            const int64_t j = idx - n_qk - n_g;
            const int h = (int)(j % Hv);
            const int64_t rest = j / Hv;
            const int t = (int)(rest % T);
            const int sl = (int)(rest / T);
            float b = 0.f;
            if (t < a.lens[sl]) {
                const int64_t rt = (((seq0 + sl) * T + t) * Hv + h) * NQ;
#pragma unroll
                for (int qb = 0; qb < NQ; ++qb) b += a.pbuf[rt + qb];
            }
            a.dbeta[((seq0 + sl) * T + t) * Hv + h] = b;
        }
    }
}

template <typename Args>
hipError_t launch(const void *fn, const Args &args, int blocks, int threads, hipStream_t st) {
    if (blocks <= 0) return hipSuccess;
    void *params[] = {const_cast<Args *>(&args)};
    return hipLaunchKernel(fn, dim3(blocks), dim3(threads), params, 0, st);
}

}  // namespace

hipError_t launch_fwd128(const FwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st) {
    const int blocks = n_seqs_launch * a.H_v * NQ;
    return kda ? launch((const void *)fwd128_kernel<true>, a, blocks, THREADS, st)
               : launch((const void *)fwd128_kernel<false>, a, blocks, THREADS, st);
}

hipError_t launch_bwd128(const BwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st) {
    const int blocks = n_seqs_launch * a.H_v * NQ;
    return kda ? launch((const void *)bwd128_kernel<true>, a, blocks, THREADS, st)
               : launch((const void *)bwd128_kernel<false>, a, blocks, THREADS, st);
}

hipError_t launch_combine128(const Combine128Args &a, hipStream_t st) {
    const int64_t G = a.kda ? S : 1;
    const int64_t total = (int64_t)a.n_seqs_launch * a.T * (a.H_k * S + a.H_v * G + a.H_v);
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    return launch((const void *)combine128_kernel, a, (int)blocks, 256, st);
}

}  // namespace gdn
