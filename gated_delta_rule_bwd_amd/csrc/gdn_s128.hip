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
// Forward (fwd128_kernel): lanes are laid out as 8 lanes per row with 16 contiguous columns
// per lane and one row per lane, so the two row reductions per token (u = Mp k and
// y = M q) are three DPP adds each.  Token vectors are staged through LDS in
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

// Token vectors in the forward's LDS: the 16-column block of lane lc starts at word 20 lc,
// so the eight lanes of a row read disjoint bank groups.
constexpr int SP = S + S / 4;
__device__ __forceinline__ int padc(int c) { return c + (c >> 4) * 4; }

template <bool KDA>
__global__ void __launch_bounds__(THREADS)
fwd128_kernel(const FwdArgs a) {
    constexpr int GW = KDA ? SP : 1;
    __shared__ float qs[2][TC][SP], ks[2][TC][SP], gs[2][TC][GW];
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
    const int lc = lane & 7, rg = lane >> 3;  // 8 lanes per row, 16 columns per lane
    const int lr0 = w * 8 + rg;               // local row of this lane
    const int row0 = qb * QR + lr0;           // global row
    const bool write_y = a.y != nullptr;

    const float *qp = a.q + s * a.sq.seq + hk * a.sq.head;
    const float *kp = a.k + s * a.sk.seq + hk * a.sk.head;
    const float *gp = a.g + s * a.sg.seq + h * a.sg.head;
    const float *vp = a.v + s * a.sv.seq + h * a.sv.head + qb * QR;
    const float *bp = a.beta + s * a.sb.seq + h * a.sb.head;
    const int64_t tok_ae = (int64_t)a.H_v;   // token stride of abuf / ebuf rows, in rows
    float *abase = a.abuf + (s * a.T * a.H_v + h) * (KDA ? S : 1);
    float *ebase = a.ebuf + (s * a.T * a.H_v + h) * S + qb * QR;

    float M[16];
    {
        const float *st0 = a.state0 + unit * S * S + (int64_t)row0 * S + lc * 16;
#pragma unroll
        for (int n = 0; n < 16; ++n) M[n] = st0[n];
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
            qs[buf][stt][padc(scc + i)] = rq[i];
            ks[buf][stt][padc(scc + i)] = rk[i];
        }
        if constexpr (KDA) {
            float av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = expf(rg4[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) gs[buf][stt][padc(scc + i)] = av[i];
            if (qb == 0 && ok) {
#pragma unroll
                for (int i = 0; i < 4; ++i) abase[t * tok_ae * S + scc + i] = av[i];
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
    float *snap = a.snap + unit * a.n_ck_max * S * S + (int64_t)row0 * S + lc * 16;
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
                for (int n = 0; n < 16; ++n) snap[n] = M[n];
                snap += (int64_t)S * S;
                next_snap += a.C;
            }
            float qv[16], kv[16], av[16];
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                qv[n] = qs[buf][tt][lc * 20 + n];
                kv[n] = ks[buf][tt][lc * 20 + n];
                av[n] = gs[buf][tt][KDA ? lc * 20 + n : 0];
            }
            const float beta = bs[buf][tt];
            const float vr = vs[buf][tt][lr0];
            float mp[16], u4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                mp[n] = M[n] * av[n];
                u4[n & 3] = fmaf(mp[n], kv[n], u4[n & 3]);
            }
            float u = (u4[0] + u4[1]) + (u4[2] + u4[3]);
            u += dpp<0xB1>(u);   // quad_perm [1,0,3,2]
            u += dpp<0x4E>(u);   // quad_perm [2,3,0,1]
            u += dpp<0x141>(u);  // row_half_mirror: the two quads of each 8-lane row
            const float e = vr - u;
            const float de = beta * e;
            float y4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                M[n] = fmaf(de, kv[n], mp[n]);
                y4[n & 3] = fmaf(M[n], qv[n], y4[n & 3]);
            }
            float y = (y4[0] + y4[1]) + (y4[2] + y4[3]);
            y += dpp<0xB1>(y);
            y += dpp<0x4E>(y);
            y += dpp<0x141>(y);
            if (lc == 0) {
                ys[tt][lr0] = a.scale * y;
                es[tt][lr0] = e;
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
        float *so = a.state_out + unit * S * S + (int64_t)row0 * S + lc * 16;
#pragma unroll
        for (int n = 0; n < 16; ++n) so[n] = M[n];
    }
}

// ------------------------------------------------------------------ backward walk

// Token data of one chunk of C2 tokens, staged in LDS for the waves of a workgroup.
template <int GW>
struct TokStage {
    float q[C2][S];
    float k[C2][S];
    float a[C2][GW];
    float e[C2][QR];     // prediction errors of this quarter's rows
    float de[C2][QR];    // beta * e (the forward's rounding)
    float gy[C2][QR];    // output cotangent of this quarter's rows
    float beta[C2];
};

// LDS of the backward: the small arrays come first so that their addresses fit the 16-bit
// immediate offsets of ds instructions; the per-thread states follow.
template <int GW, int RW>
struct BwdLds {
    static constexpr int NT = 64 * (QR / RW);
    static constexpr int NV = 2 * RW;   // floats per thread per token state
    TokStage<GW> ts;
    float redb[C2][QR / RW], redg[C2][QR / RW];
    // decayed previous states of a sub-segment, thread-private and component-major:
    // value k of thread tid for chunk position tt sits at st[tt][k][tid], so a wave's
    // accesses are consecutive words (no bank conflicts).  After a token is walked its
    // slot holds the thread's column sums of that token (k = 0..5: dq, dk, dg for its
    // two columns) until the sub-segment's reduction.
    float st[C2][NV][NT];
};

// RW rows per wave, 32 / RW waves per workgroup; each lane holds columns lane and lane + 64
// of its wave's rows, so column sums are in-lane and the row sum dd = dM k is rows_sum.
template <bool KDA, int RW>
__global__ void __launch_bounds__(64 * (QR / RW), 1)
bwd128_kernel(const BwdArgs a) {
    constexpr int GW = KDA ? S : 1;
    constexpr int NP = KDA ? 3 : 2;     // partial slots per quarter: dq | dk (| dg)
    constexpr int NW = QR / RW;         // waves
    constexpr int NT = 64 * NW;         // threads
    constexpr int NV = 2 * RW;          // floats per thread per token state
    static_assert(NV >= 6, "the column-sum stash needs six words per thread");
    __shared__ BwdLds<GW, RW> sm;
    auto &ts = sm.ts;

    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr0 = w * RW;             // first row of this wave within the quarter
    const int row0 = qb * QR + wr0;     // first global row of this wave
    const int C = a.C;
    // after rows_sum, lane 16 i of a 4-row group holds row 4p + {0, 2, 1, 3}[i]
    const int dv_row = ((lane >> 4) & 1) * 2 + (lane >> 5);

    const float *snapu = a.snap + unit * a.n_ck_max * S * S + (int64_t)row0 * S + lane;
    float4 *vsb = reinterpret_cast<float4 *>(a.vsbuf) +
                  ((unit * NQ + qb) * (int64_t)a.nvs_max) * (RW / 2 * NT) + tid;

    // ---- staging of token data (register prefetch of the next chunk, then LDS).  Thread tid
    // stages column sc = tid % S of tokens stt + m * (NT / S) of the q, k, a vectors, and
    // row rrow = tid % QR of token rtt = tid / QR of the e and gy vectors.
    constexpr int TG = NT / S;          // tokens covered by one pass over the threads
    constexpr int PV = C2 / TG;         // vector elements per thread per chunk
    static_assert(C2 % TG == 0 && C2 * QR <= NT, "staging layout");
    const int64_t tok_ae = a.H_v;
    const int sc = tid % S, stt = tid / S;
    const int rtt = tid / QR, rrow = tid % QR;
    const float *kp0 = a.k + s * a.sk.seq + hk * a.sk.head + sc + stt * a.sk.tok;
    const float *qp0 = a.q + s * a.sq.seq + hk * a.sq.head + sc + stt * a.sq.tok;
    const float *ap0 = a.abuf + (s * a.T * a.H_v + h) * GW + (KDA ? sc + stt * tok_ae * GW : 0);
    const float *ep0 = a.ebuf + (s * a.T * a.H_v + h) * S + qb * QR + rrow + rtt * tok_ae * S;
    const float *gyp0 = a.gy + s * a.sgy.seq + h * a.sgy.head + qb * QR + rrow + rtt * a.sgy.tok;
    const float *bp = a.beta + s * a.sb.seq + h * a.sb.head;
    const float *as0 = a.abuf + (s * a.T * a.H_v + h) * GW;   // scalar gate values
    float pq[PV], pk[PV], pa[PV], pe = 0.f, pgy = 0.f, pb1 = 0.f, pbe = 0.f;
    int pcnt = 0;
    auto load_chunk = [&](int tstart, int cnt, bool walk) {
        pcnt = cnt;
#pragma unroll
        for (int m = 0; m < PV; ++m) {
            if (stt + m * TG < cnt) {
                const int64_t t = tstart + m * TG;
                pk[m] = kp0[t * a.sk.tok];
                if (walk) pq[m] = qp0[t * a.sq.tok];
                if constexpr (KDA) pa[m] = ap0[t * tok_ae * GW];
            }
        }
        if (tid < C2 * QR && rtt < cnt) {
            pe = ep0[(int64_t)tstart * tok_ae * S];
            pbe = bp[(tstart + rtt) * a.sb.tok];
            if (walk) pgy = gyp0[(int64_t)tstart * a.sgy.tok];
        }
        if (tid < cnt) {
            pb1 = bp[(tstart + tid) * a.sb.tok];
        } else if (!KDA && tid >= C2 && tid < C2 + cnt) {
            pb1 = as0[(tstart + tid - C2) * tok_ae];
        }
    };
    auto store_chunk = [&](bool walk) {
#pragma unroll
        for (int m = 0; m < PV; ++m) {
            const int tt = stt + m * TG;
            if (tt < pcnt) {
                ts.k[tt][sc] = pk[m];
                if (walk) ts.q[tt][sc] = pq[m];
                if constexpr (KDA) ts.a[tt][sc] = pa[m];
            }
        }
        if (tid < C2 * QR && rtt < pcnt) {
            ts.e[rtt][rrow] = pe;
            ts.de[rtt][rrow] = pbe * pe;
            if (walk) ts.gy[rtt][rrow] = pgy;
        }
        if (tid < pcnt) {
            ts.beta[tid] = pb1;
        } else if (!KDA && tid >= C2 && tid < C2 + pcnt) {
            ts.a[tid - C2][0] = pb1;
        }
    };

    float X[RW][2];
    if (a.dstate_out) {
        const float *d0 = a.dstate_out + unit * S * S + (int64_t)row0 * S + lane;
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) X[r][n] = d0[r * S + n * 64];
    } else {
#pragma unroll
        for (int r = 0; r < RW; ++r) X[r][0] = X[r][1] = 0.f;
    }

    auto put4 = [&](float4 *dst, const float (&M)[RW][2]) {
#pragma unroll
        for (int c = 0; c < RW / 2; ++c)
            dst[c * NT] = make_float4(M[2 * c][0], M[2 * c][1], M[2 * c + 1][0], M[2 * c + 1][1]);
    };
    auto get4 = [&](const float4 *src, float (&M)[RW][2]) {
#pragma unroll
        for (int c = 0; c < RW / 2; ++c) {
            const float4 x = src[c * NT];
            M[2 * c][0] = x.x; M[2 * c][1] = x.y; M[2 * c + 1][0] = x.z; M[2 * c + 1][1] = x.w;
        }
    };

    // one replayed token from the staged chunk: Mp = M .* a; M = Mp + (beta e) k^T
    auto replay = [&](int tt, float (&M)[RW][2], bool keep) {
        float kv[2], av[2], de[RW];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            kv[n] = ts.k[tt][lane + 64 * n];
            av[n] = ts.a[tt][KDA ? lane + 64 * n : 0];
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) de[r] = ts.de[tt][wr0 + r];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float mp = M[r][n] * av[n];
                if (keep) sm.st[tt][2 * r + n][tid] = mp;
                M[r][n] = fmaf(de[r], kv[n], mp);
            }
    };

    // one token of the reverse walk (token t, chunk position tt).  Once a thread has read its
    // LDS state of token tt it owns that slot again and leaves its column sums there.
    auto walk = [&](int t, int tt) {
        float Mp[RW][2];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) Mp[r][n] = sm.st[tt][2 * r + n][tid];
        float qs[2], kv[2], kn[2], av[2], gy[RW], ev[RW], de[RW];
        const float beta = ts.beta[tt];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            qs[n] = a.scale * ts.q[tt][lane + 64 * n];
            kv[n] = ts.k[tt][lane + 64 * n];
            kn[n] = -beta * kv[n];
            av[n] = ts.a[tt][KDA ? lane + 64 * n : 0];
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            gy[r] = ts.gy[tt][wr0 + r];
            ev[r] = ts.e[tt][wr0 + r];
            de[r] = ts.de[tt][wr0 + r];
        }
        float pq[2] = {0.f, 0.f}, pe2[2] = {0.f, 0.f}, pm[2] = {0.f, 0.f}, pg[2] = {0.f, 0.f};
        float dpart[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            dpart[r] = 0.f;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float mt = fmaf(de[r], kv[n], Mp[r][n]);  // state after token t
                X[r][n] = fmaf(gy[r], qs[n], X[r][n]);         // dM += scale gy q^T
                pq[n] = fmaf(mt, gy[r], pq[n]);                // dq  (x scale below)
                pe2[n] = fmaf(X[r][n], de[r], pe2[n]);         // dk: dM^T delta
                dpart[r] = fmaf(X[r][n], kv[n], dpart[r]);     // dd = dM k
            }
        }
        // dd = dM k over the 64 lanes; lane 16 i of each 16-lane row holds one row's total
        float hh[RW / 2];
#pragma unroll
        for (int p = 0; p < RW / 2; ++p) {
            auto sw = __builtin_amdgcn_permlane32_swap(as_i(dpart[2 * p]), as_i(dpart[2 * p + 1]),
                                                       false, false);
            hh[p] = as_f(sw[0]) + as_f(sw[1]);
        }
        float dd[RW];
#pragma unroll
        for (int p = 0; p < RW / 4; ++p) {
            auto sw = __builtin_amdgcn_permlane16_swap(as_i(hh[2 * p]), as_i(hh[2 * p + 1]), false,
                                                       false);
            const float g = row16_sum(as_f(sw[0]) + as_f(sw[1]));
            dd[4 * p + 0] = as_f(__builtin_amdgcn_readlane(as_i(g), 0));
            dd[4 * p + 2] = as_f(__builtin_amdgcn_readlane(as_i(g), 16));
            dd[4 * p + 1] = as_f(__builtin_amdgcn_readlane(as_i(g), 32));
            dd[4 * p + 3] = as_f(__builtin_amdgcn_readlane(as_i(g), 48));
            if ((lane & 15) == 0)                              // dv = beta dd
                a.dv[((s * a.T + t) * a.H_v + h) * S + row0 + 4 * p + dv_row] = beta * g;
        }
        float pb = 0.f;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            pb = fmaf(dd[r], ev[r], pb);                       // dbeta = dd . (v - u)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                pm[n] = fmaf(Mp[r][n], dd[r], pm[n]);          // Mp^T dd (du = -beta dd)
                X[r][n] = fmaf(dd[r], kn[n], X[r][n]);         // dM += du k^T
                pg[n] = fmaf(X[r][n], Mp[r][n], pg[n]);        // dg = sum dM .* Mp
                X[r][n] *= av[n];                              // dM = dM .* a
            }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            sm.st[tt][n][tid] = a.scale * pq[n];
            sm.st[tt][2 + n][tid] = fmaf(-beta, pm[n], pe2[n]);
            if constexpr (KDA) sm.st[tt][4 + n][tid] = pg[n];
        }
        if constexpr (!KDA) {
            const float gs = wave_sum(pg[0] + pg[1]);
            if (lane == 0) sm.redg[tt][w] = gs;
        }
        if (lane == 0) sm.redb[tt][w] = pb;
    };

    // the column sums of the cnt walked tokens starting at token ta, summed over the waves
    // in a fixed order and written to the quarter's partial buffers.  Thread tid reduces
    // column sc of tokens stt + m * TG.
    const int64_t part_tok = (int64_t)a.H_v * NQ * NP * S;   // floats per token
    auto reduce_columns = [&](int ta, int cnt) {
        __syncthreads();   // every wave has left its column sums in the LDS slots
        float *pp = a.part + (((s * a.T + ta) * a.H_v + h) * NQ + qb) * NP * S + sc;
#pragma unroll
        for (int m = 0; m < PV; ++m) {
            const int tt = stt + m * TG;
            if (tt < cnt) {
#pragma unroll
                for (int which = 0; which < NP; ++which) {
                    // value (which, column sc) of wave w: thread w*64 + sc%64, word 2*which + sc/64
                    const float *base = &sm.st[tt][2 * which + (sc >> 6)][sc & 63];
                    float acc = base[0];
#pragma unroll
                    for (int ww = 1; ww < NW; ++ww) acc += base[ww * 64];
                    pp[tt * part_tok + which * S] = acc;
                }
            }
        }
        if (tid < cnt) {
            const int64_t rt = ((s * a.T + ta + tid) * a.H_v + h) * NQ + qb;
            float b = sm.redb[tid][0];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) b += sm.redb[tid][ww];
            a.pbuf[rt] = b;
            if constexpr (!KDA) {
                float g = sm.redg[tid][0];
#pragma unroll
                for (int ww = 1; ww < NW; ++ww) g += sm.redg[tid][ww];
                a.pgbuf[rt] = g;
            }
        }
        __syncthreads();   // LDS slots free for the next sub-segment
    };

    auto load_state = [&](const float *src, float (&M)[RW][2]) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) M[r][n] = src[r * S + n * 64];
    };

    const int n_ck = (L + C - 1) / C;
    for (int sg = n_ck - 1; sg >= 0; --sg) {
        const int t0 = sg * C, t1 = min(t0 + C, L);
        const int nvs = (t1 - t0 + VS - 1) / VS;
        float M[RW][2];
        load_state(snapu + (int64_t)sg * S * S, M);
        // stretch starts beyond the first: replay once and keep them in the workspace
        if (nvs > 1) {
            const int tend = t0 + VS * (nvs - 1);
            load_chunk(t0, C2, false);
            __syncthreads();
            store_chunk(false);
            __syncthreads();
            for (int tc = t0; tc < tend; tc += C2) {
                if (tc > t0 && (tc - t0) % VS == 0)
                    put4(vsb + (int64_t)((tc - t0) / VS) * (RW / 2 * NT), M);
                if (tc + C2 < tend) load_chunk(tc + C2, C2, false);
                for (int tt = 0; tt < C2; ++tt) replay(tt, M, false);
                __syncthreads();
                if (tc + C2 < tend) store_chunk(false);
                __syncthreads();
            }
        }
        for (int v = nvs - 1; v >= 0; --v) {
            const int va = t0 + v * VS, vb = min(va + VS, t1);
            const int nsub = (vb - va + C2 - 1) / C2;
            if (v < nvs - 1) {
                if (v == 0)
                    load_state(snapu + (int64_t)sg * S * S, M);
                else
                    get4(vsb + (int64_t)v * (RW / 2 * NT), M);
            }
            auto cnt_of = [&](int j) { return min(C2, vb - (va + j * C2)); };
            // first chunk of the stretch: replay chunk 0, or the walk of the only sub-segment
            load_chunk(va, nsub > 1 ? C2 : cnt_of(0), nsub == 1);
            __syncthreads();
            store_chunk(nsub == 1);
            __syncthreads();
            // replay the stretch, keeping the state every C2 tokens in registers
            float SS[NSUB][RW][2];
#pragma unroll
            for (int r = 0; r < RW; ++r) SS[0][r][0] = M[r][0], SS[0][r][1] = M[r][1];
#pragma unroll
            for (int j = 0; j < NSUB - 1; ++j) {
                if (j < nsub - 1) {
                    const bool next_walk = j + 1 == nsub - 1;
                    load_chunk(va + (j + 1) * C2, next_walk ? cnt_of(j + 1) : C2, next_walk);
                    for (int tt = 0; tt < C2; ++tt) replay(tt, M, false);
#pragma unroll
                    for (int r = 0; r < RW; ++r) SS[j + 1][r][0] = M[r][0], SS[j + 1][r][1] = M[r][1];
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
                    for (int r = 0; r < RW; ++r) M[r][0] = SS[j][r][0], M[r][1] = SS[j][r][1];
                    const int ta = va + j * C2, cnt = cnt_of(j);
                    for (int tt = 0; tt < cnt; ++tt) replay(tt, M, true);
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
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) ds[r * S + n * 64] = X[r][n];
    }
    for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += NT) {
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

constexpr int kBwdRW = 4;   // rows per wave of the backward (8 waves per quarter)

hipError_t launch_bwd128(const BwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st) {
    const int blocks = n_seqs_launch * a.H_v * NQ;
    constexpr int nt = 64 * (QR / kBwdRW);
    return kda ? launch((const void *)bwd128_kernel<true, kBwdRW>, a, blocks, nt, st)
               : launch((const void *)bwd128_kernel<false, kBwdRW>, a, blocks, nt, st);
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
