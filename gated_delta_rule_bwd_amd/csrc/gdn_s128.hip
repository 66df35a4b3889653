// gdn_s128.hip -- gfx950 kernels of the gated delta rule for head size S = 128.
//
// Work decomposition.  A (sequence, value head) unit owns a 128 x 128 fp32 state M = S^T
// (row j = value index, column i = key index).  Rows evolve independently in both
// directions of the recurrence ("metal: GATED_DELTA_NET_BACK", approval review: thread j
// owns row j of M), so each unit is split into four row quarters of 32 rows, one workgroup
// each.  At the layer shape (192 units) that is 768 workgroups, three per compute unit, so
// all 256 CUs carry equal work.  The quarters are coupled only through column sums of the
// backward (dq, dk, the per-channel dg) and the row sum dbeta; each quarter writes its
// partial sums and a fixed-order kernel adds the four quarters (and, for dq/dk, the value
// heads of each key head in increasing order), so results are bitwise reproducible.
//
// Column-scaled state.  The gate only scales columns: M_t = M_{t-1} diag(a_t) + delta_t k_t^T.
// Inside a window of tokens starting at t0 the state is carried as M_t = Mh_t diag(c_t) with
// c_t = a_t0 * ... * a_t (running product per column), which turns the update into a single
// fma per element, Mh_t = Mh_{t-1} + delta_t (k_t / c_t)^T, while the readouts use the vectors
// c_t .* k_t and c_t .* q_t.  At the end of a window the product is folded back into the
// state (one multiply per element).  The backward carries dM the same way, with the suffix
// product d_t = a_{t+1} * ... * a_end of the window, so its two rank-one updates and the
// decay become two fmas per element.  Windows are the 8-token blocks of the sequence
// (checkpoints fall on them), so both directions use the same windows and the backward's
// replay reproduces the forward's states bit for bit.  A window whose running product would
// leave [2^-60, 1] (a gate above one, or a decay below 2^-60 over the window) is processed
// unscaled instead, with the decay applied per token; both directions take that decision
// from the same values.
//
// Kernels: gate128_kernel writes each window's gate factors once (both directions read
// them); fwd128_kernel
// (four waves, 8 lanes per row with 16 columns each, so the row sums u = Mp k and y = M q
// are three DPP adds) writes y, the final state, the snapshots every C tokens and the
// prediction errors e = v - u; bwd128_kernel (eight waves, 64 lanes per row with columns
// lane and lane + 64 and four rows per lane, so column sums are in-lane and the row sum
// dd = dM k is a permlane/DPP reduce-scatter) replays and walks; combine128_kernel adds
// the partial sums.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int S = 128;
constexpr int QR = 32;         // rows per workgroup (one row quarter)
constexpr int NQ = S / QR;     // quarters per unit
constexpr int WIN = 8;         // tokens per window
constexpr int VS = 64;         // tokens per stretch in the backward
constexpr int NWS = VS / WIN;  // windows per stretch
constexpr float kScaleMin = 0x1p-60f;

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

// Sum over each 32-lane half of the wave; every lane receives its half's sum.
__device__ __forceinline__ float half_sum(float v) {
    v = row16_sum(v);
    auto p = __builtin_amdgcn_permlane16_swap(as_i(v), as_i(v), false, false);
    return as_f(p[0]) + as_f(p[1]);
}

// Sum over all 64 lanes; every lane receives the sum.
__device__ __forceinline__ float wave_sum(float v) {
    v = half_sum(v);
    auto q = __builtin_amdgcn_permlane32_swap(as_i(v), as_i(v), false, false);
    return as_f(q[0]) + as_f(q[1]);
}

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Global accesses as a wave-uniform base plus a 32-bit element offset, so the address is a
// scalar base and one vector offset register instead of a per-lane 64-bit pointer.
template <typename T>
__device__ __forceinline__ T ldg(const T *base, uint32_t i) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + i * (uint32_t)sizeof(T));
}
template <typename T>
__device__ __forceinline__ void stg(T *base, uint32_t i, T v) {
    *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + i * (uint32_t)sizeof(T)) = v;
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Element type DT (GDN_DTYPE_*) of the caller's q, k, v, g, beta and gy: fp32, IEEE binary16
// or bfloat16, read as such and widened to fp32 exactly at the load.
template <int DT>
struct InT {
    using type = float;
};
template <>
struct InT<GDN_DTYPE_F16> {
    using type = _Float16;
};
template <>
struct InT<GDN_DTYPE_BF16> {
    using type = uint16_t;
};
template <int DT>
using In = typename InT<DT>::type;
template <int DT>
__device__ __forceinline__ float fin(In<DT> x) {
    if constexpr (DT == GDN_DTYPE_BF16) return __builtin_bit_cast(float, (uint32_t)x << 16);
    else return (float)x;
}
template <int DT>
__device__ __forceinline__ const In<DT> *inp(const float *p) {
    return reinterpret_cast<const In<DT> *>(p);
}
// Compiler-only memory barrier: bounds how far the compiler hoists LDS loads (and so how many
// registers they hold); it emits no instruction.
__device__ __forceinline__ void hoist_fence() { asm volatile("" ::: "memory"); }

// Block index -> (unit within the launch, row quarter).  The four quarters of a unit read
// the same token vectors, so they are placed on the same XCD (blocks are dispatched to the
// eight XCDs round robin) when the grid allows it.
__device__ __forceinline__ void map_block(int b, int nb, int &unit, int &qb) {
    int lin = b;
    if (nb % (8 * NQ) == 0) lin = (b % 8) * (nb / 8) + b / 8;
    unit = lin / NQ;
    qb = lin % NQ;
}

// A window is processed column-scaled when every gate in it is at most one and the product
// over the window stays at or above 2^-60; then every prefix and suffix product of the
// window lies in [2^-60, 1].  (NaN gates fail both tests.)
__device__ __forceinline__ bool gate_ok(float a) { return a <= 1.f; }
__device__ __forceinline__ bool prod_ok(float c) { return c >= kScaleMin; }

// ------------------------------------------------------------------ gates

// For every 8-token window of every (sequence, value head): the gates a = exp(g) of its
// tokens, the running product c_t = a_t0 * ... * a_t from the window's first token t0 (taken
// in token order, so every kernel that scales by it uses the same bits), the product d_t of
// the window's gates after t, and the flag of a window that must be processed unscaled.  A
// column-scaled window stores (c, d) per token, an unscaled one (a, 1), so the kernels load
// the same array in both cases and need the flag only when they use the values.  One wave
// per window for the per-channel gate (lane: columns lane, lane + 64), one thread per window
// for the scalar gate.
template <int DT>
__global__ void __launch_bounds__(256) gate128_kernel(const GateArgs a) {
    const int nwin = (a.T + WIN - 1) / WIN;
    const int64_t items = (int64_t)a.n_seqs_launch * nwin * a.H_v;
    const bool kda = a.G != 1;
    const int lane = threadIdx.x & 63;
    const int64_t first = kda ? (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)
                              : (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t step = kda ? (int64_t)gridDim.x * (blockDim.x >> 6) : (int64_t)gridDim.x * blockDim.x;
    for (int64_t it = first; it < items; it += step) {
        const int h = (int)(it % a.H_v);
        const int64_t rest = it / a.H_v;
        const int m = (int)(rest % nwin), sl = (int)(rest / nwin);
        const int t0 = m * WIN;
        const int cnt = min(WIN, a.lens[sl] - t0);
        if (cnt <= 0) continue;
        const int64_t s = a.s_base + sl;
        const int NC = kda ? 2 : 1;
        float av[WIN][2], cv[WIN][2];
        bool ok = true;
#pragma unroll
        for (int tt = 0; tt < WIN; ++tt)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                av[tt][n] = 1.f;
                if (tt < cnt && n < NC) {
                    const In<DT> *gp = inp<DT>(a.g) + s * a.sg.seq + (int64_t)(t0 + tt) * a.sg.tok + h * a.sg.head;
                    av[tt][n] = expf(fin<DT>(gp[kda ? lane + 64 * n : 0]));
                }
            }
        float c[2] = {1.f, 1.f};
#pragma unroll
        for (int tt = 0; tt < WIN; ++tt)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                ok = ok && gate_ok(av[tt][n]);
                c[n] *= av[tt][n];
                cv[tt][n] = c[n];
            }
        ok = ok && prod_ok(c[0]) && prod_ok(c[1]);   // the padding gates are 1
        const bool direct = kda ? __ballot(!ok) != 0 : !ok;
        float d[2] = {1.f, 1.f};
#pragma unroll
        for (int tt = WIN - 1; tt >= 0; --tt)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                if (tt < cnt && n < NC) {
                    const int64_t o = ((s * a.T + t0 + tt) * a.H_v + h) * a.G + (kda ? lane + 64 * n : 0);
                    a.cbuf[o] = direct ? av[tt][n] : cv[tt][n];
                    a.dbuf[o] = direct ? 1.f : d[n];
                }
                d[n] *= av[tt][n];
            }
        if (!kda || lane == 0) a.wflag[(s * nwin + m) * a.H_v + h] = direct ? 1 : 0;
    }
}

// ------------------------------------------------------------------ forward scan

// Forward rows per lane FR: 2 (four waves of eight rows) when the launch has enough
// workgroups to fill the chip, 1 (eight waves of four rows) when it has few, so that each
// SIMD runs more, shorter scan chains.  The window staging is done by the first 256 threads.
constexpr int FC = 8;              // columns per lane in the forward (16 lanes per row)
constexpr int SP = S + 8;          // padded vector: column c at word c + 4 (c / 64)
__device__ __forceinline__ int padc(int c) { return c + 4 * (c >> 6); }

template <bool KDA>
struct alignas(16) FwdLds {
    static constexpr int GW = KDA ? SP : 1;
    float kc[WIN][SP], kr[WIN][SP], qc[WIN][SP];         // c.*k, k./c, c.*q (scaled window)
    float kraw[WIN][SP], qraw[WIN][SP], araw[WIN][GW];   // unscaled window
    float cend[GW];                                      // product over the window
    float vq[WIN][QR];                                   // v of this quarter's rows
    float bt[WIN];                                       // beta
    float ys[2][WIN][QR], es[2][WIN][QR];                // outputs of the last two windows
};

template <bool KDA, int FR, int DT>
__global__ void __launch_bounds__(512 / FR)
fwd128_kernel(const FwdArgs a) {
    constexpr int GW = KDA ? S : 1;
    constexpr int FT = 512 / FR;                  // threads
    __shared__ FwdLds<KDA> sm;
    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int C = a.C;
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lc = lane & 15;                     // 8-column block of this lane
    const int lrow = w * (4 * FR) + (lane >> 4) * FR;   // first of the lane's rows (quarter)
    const int row = qb * QR + lrow;               // first of the lane's rows (state)
    // With two rows per lane, lanes 8-15 of each 16-lane row group hold them in swapped order
    // (register r holds row lrow + (r ^ hsw)): lanes i and i ^ 8 then hold the same row in
    // registers 0 and 1, so both rows' sums are one reduce-scatter without selects.
    const int hsw = (FR == 2 && (lc & 8)) ? 1 : 0;
    const int cb = padc(lc * FC);                 // padded offset of the lane's columns
    const bool write_y = a.y != nullptr;

    // staging roles: threads 0..127 hold the k and gate values of column ci for the window's
    // tokens, threads 128..255 the q and gate values; thread tid also holds v of row srow of
    // token stt, threads 0..7 beta
    // Global addresses are a uniform base (scalar arithmetic) plus a 32-bit per-thread offset.
    const int ci = tid & (S - 1), pci = padc(ci);
    const bool kside = uni(tid) < S;   // uniform: waves 0 and 1
    const bool stager = uni(tid) < 2 * S;   // uniform: waves 0 to 3 stage the windows
    const int stt = tid >> 5, srow = tid & 31;
    const In<DT> *xp = kside ? inp<DT>(a.k) + s * a.sk.seq + hk * a.sk.head
                             : inp<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const int64_t xtok = kside ? a.sk.tok : a.sq.tok;
    const In<DT> *vp = inp<DT>(a.v) + s * a.sv.seq + h * a.sv.head + qb * QR;
    const In<DT> *bp = inp<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
    const int64_t tok_ae = a.H_v;   // token stride of cbuf / ebuf rows, in rows
    const float *cp = a.cbuf + (s * a.T * a.H_v + h) * GW;
    const int nwin_T = (a.T + WIN - 1) / WIN;
    const int32_t *wfl = a.wflag + s * nwin_T * a.H_v + h;   // window stride H_v
    float *ebase = a.ebuf + (s * a.T * a.H_v + h) * S + qb * QR;

    float M[FR][FC];
    auto rw_state = [&](float *base, bool store) {   // the lane's 2 x 8 block of a state
#pragma unroll
        for (int r = 0; r < FR; ++r)
#pragma unroll
            for (int j = 0; j < FC; j += 4) {
                float4 *p4 = reinterpret_cast<float4 *>(base + (int64_t)(row + (r ^ hsw)) * S + lc * FC + j);
                if (store) *p4 = make_float4(M[r][j], M[r][j + 1], M[r][j + 2], M[r][j + 3]);
                else { const float4 v = *p4; M[r][j] = v.x; M[r][j + 1] = v.y; M[r][j + 2] = v.z; M[r][j + 3] = v.w; }
            }
    };
    const bool st_vec = ((uintptr_t)a.state0 & 15) == 0;
    if (st_vec) {
        rw_state(const_cast<float *>(a.state0) + unit * S * S, false);
    } else {
#pragma unroll
        for (int r = 0; r < FR; ++r)
#pragma unroll
            for (int n = 0; n < FC; ++n) M[r][n] = a.state0[unit * S * S + (int64_t)(row + (r ^ hsw)) * S + lc * FC + n];
    }
    // the state has arrived before the scan starts, so no wait inside the scan is charged to it
    __builtin_amdgcn_s_waitcnt(0);

    // Per token of a window: the gate factor (the running product c in a column-scaled window,
    // the gate a in an unscaled one), the k or q value, v and beta, and the window's flag.  Two
    // register sets take turns, so each window's loads are issued two windows before its
    // staging uses them.
    struct WinRegs {   // k / q, v and beta kept in the input type until staged
        float av[WIN];
        In<DT> xv[WIN], rv, rb;
        int wdir;
    };
    auto load_window = [&](WinRegs &W, int t0, int cnt) __attribute__((always_inline)) {
        W.wdir = wfl[(int64_t)(t0 / WIN) * a.H_v];
        if (FR == 2 || stager) {
#pragma unroll
        for (int tt = 0; tt < WIN; ++tt) {   // clamped loads: no branch per token
            const int64_t t = t0 + min(tt, cnt - 1);
            const float g = ldg(cp + t * tok_ae * GW, (uint32_t)(KDA ? ci : 0));
            const In<DT> x = ldg(xp + t * xtok, (uint32_t)ci);
            W.av[tt] = tt < cnt ? g : 1.f;
            W.xv[tt] = tt < cnt ? x : In<DT>(0);
        }
        const int tv = min(stt, cnt - 1), tb = min(tid & (WIN - 1), cnt - 1);
        W.rv = ldg(vp + (int64_t)t0 * a.sv.tok, (uint32_t)(tv * a.sv.tok + srow));
        W.rb = ldg(bp + (int64_t)t0 * a.sb.tok, (uint32_t)(tb * a.sb.tok));
        }
    };
    // outputs of the window at t (cnt tokens) from output buffer ob
    auto flush = [&](int t, int cnt, int ob) {
        if (stt < cnt) {
            if (write_y)
                stg(a.y + s * a.sy.seq + (int64_t)t * a.sy.tok + h * a.sy.head + qb * QR,
                    (uint32_t)(stt * a.sy.tok + srow), sm.ys[ob][stt][srow]);
            stg(ebase + (int64_t)t * tok_ae * S, (uint32_t)(stt * tok_ae * S + srow), sm.es[ob][stt][srow]);
        }
    };

    float *snap = a.snap + unit * a.n_ck_max * S * S;
    int ta = 0, prev_ta = 0, prev_cnt = 0;
    int cnt = min(WIN, L);
    WinRegs R0, R1;
    if (cnt > 0) load_window(R0, 0, cnt);
    if (min(WIN, L - cnt) > 0) load_window(R1, cnt, min(WIN, L - cnt));
    // reads of the lane's 8 columns of a padded vector
    auto ld8 = [&](const float *base, float (&x)[FC]) {
        const float4 v0 = *reinterpret_cast<const float4 *>(base);
        const float4 v1 = *reinterpret_cast<const float4 *>(base + 4);
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    };
    // Two rows per lane: the row of register 0 summed over the eight lanes of each half of the
    // 16-lane group (lanes i and i ^ 8 first pair register 0 with the partner's register 1,
    // which holds the same row); every lane of a half receives its half's sum.
    auto pair_reduce = [&](float r0, float r1) __attribute__((always_inline)) {
        float t = r0 + dpp<0x128>(r1);   // row_ror:8, lane i <- lane i ^ 8
        t += dpp<0xB1>(t);               // quad_perm [1,0,3,2]
        t += dpp<0x4E>(t);               // quad_perm [2,3,0,1]
        t += dpp<0x141>(t);              // row_half_mirror
        return t;
    };
    // the row sums of u on every lane of the row group
    auto row_sums = [&](float (&u)[FR]) __attribute__((always_inline)) {
        if constexpr (FR == 2) {
            const float t = pair_reduce(u[0], u[1]);
            u[1] = dpp<0x128>(t);        // the other half's sum: this lane's register-1 row
            u[0] = t;
        } else {
            u[0] = row16_sum(u[0]);
        }
    };
    auto finish = [&](int tt, int ob, float (&y)[FR], const float (&e)[FR]) {
        if constexpr (FR == 2) {
            // The two output sums only need to reach one lane each: lanes 0-7 sum register 0's
            // row, lanes 8-15 register 0's (the other) row.
            const float keep = pair_reduce(y[0], y[1]);
            if ((lc & 7) == 0) sm.ys[ob][tt][lrow + hsw] = a.scale * keep;
            if (lc == 0) *reinterpret_cast<float2 *>(&sm.es[ob][tt][lrow]) = make_float2(e[0], e[1]);
            return;
        }
#pragma unroll
        for (int r = 0; r < FR; ++r) y[r] = row16_sum(y[r]);
        if (lc == 0) {
            if constexpr (FR == 2) {
            } else {
                sm.ys[ob][tt][lrow] = a.scale * y[0];
                sm.es[ob][tt][lrow] = e[0];
            }
        }
    };
    auto vrows = [&](int tt, float (&vr)[FR]) __attribute__((always_inline)) {
        if constexpr (FR == 2) {
            vr[0] = sm.vq[tt][lrow + hsw];
            vr[1] = sm.vq[tt][lrow + (hsw ^ 1)];
        } else {
            vr[0] = sm.vq[tt][lrow];
        }
    };
    // One window from register set W: stage its vectors; store the previous window's outputs
    // and the checkpoint; prefetch the window after the next into W; scan.  The stores go out
    // before the prefetch loads, so a staging's wait for loads never waits for them too.
    auto window = [&](WinRegs &W, auto par) __attribute__((always_inline)) {
        constexpr int ob = decltype(par)::value;   // output buffer: the window's parity
        __syncthreads();   // the previous window's vectors are no longer read
        const bool direct = W.wdir != 0;
        // (one store target per wave, chosen up front: k rows for waves 0 and 1, q rows else)
        if (FR == 1 && !stager) {
        } else if (!direct) {
            float ce = W.av[0];   // product over the window: c at its last token
            float *xc = kside ? &sm.kc[0][0] : &sm.qc[0][0];
#pragma unroll
            for (int tt = 0; tt < WIN; ++tt) {
                if (tt < cnt) ce = W.av[tt];
                const float xv = fin<DT>(W.xv[tt]);
                xc[tt * SP + pci] = xv * W.av[tt];
                if (kside) sm.kr[tt][pci] = xv * rcp(W.av[tt]);
            }
            if (kside && (KDA || ci == 0)) sm.cend[KDA ? pci : 0] = ce;
        } else {
            float *xr = kside ? &sm.kraw[0][0] : &sm.qraw[0][0];
#pragma unroll
            for (int tt = 0; tt < WIN; ++tt) {
                xr[tt * SP + pci] = fin<DT>(W.xv[tt]);
                if (kside && (KDA || ci == 0)) sm.araw[tt][KDA ? pci : 0] = W.av[tt];
            }
        }
        if (stt < cnt) sm.vq[stt][srow] = fin<DT>(W.rv);
        if (tid < cnt) sm.bt[tid] = fin<DT>(W.rb);
        __syncthreads();
        flush(prev_ta, prev_cnt, ob ^ 1);
        if (ta % C == 0) rw_state(snap + (int64_t)(ta / C) * S * S, true);   // checkpoint
        const int next = ta + cnt;
        const int ncnt = min(WIN, L - next);
        if (ncnt > 0 && min(WIN, L - next - ncnt) > 0) load_window(W, next + ncnt, min(WIN, L - next - ncnt));
        if (!direct) {
            for (int tt = 0; tt < cnt; ++tt) {
                float kc[FC], kr[FC], qc[FC];
                ld8(&sm.kc[tt][cb], kc);
                ld8(&sm.kr[tt][cb], kr);
                ld8(&sm.qc[tt][cb], qc);
                float vr[FR];
                vrows(tt, vr);
                const float beta = sm.bt[tt];
                float u[FR], e[FR], y[FR];
#pragma unroll
                for (int r = 0; r < FR; ++r) {
                    u[r] = M[r][0] * kc[0];
#pragma unroll
                    for (int n = 1; n < FC; ++n) u[r] = fmaf(M[r][n], kc[n], u[r]);
                }
                row_sums(u);
#pragma unroll
                for (int r = 0; r < FR; ++r) e[r] = vr[r] - u[r];
#pragma unroll
                for (int r = 0; r < FR; ++r) {
                    const float de = beta * e[r];
#pragma unroll
                    for (int n = 0; n < FC; ++n) M[r][n] = fmaf(de, kr[n], M[r][n]);
                    y[r] = M[r][0] * qc[0];
#pragma unroll
                    for (int n = 1; n < FC; ++n) y[r] = fmaf(M[r][n], qc[n], y[r]);
                }
                finish(tt, ob, y, e);
            }
            float ce[FC];
            if constexpr (KDA) {
                ld8(&sm.cend[cb], ce);
            } else {
#pragma unroll
                for (int n = 0; n < FC; ++n) ce[n] = sm.cend[0];
            }
#pragma unroll
            for (int r = 0; r < FR; ++r)
#pragma unroll
                for (int n = 0; n < FC; ++n) M[r][n] *= ce[n];
        } else {
            for (int tt = 0; tt < cnt; ++tt) {
                float kv[FC], qv[FC], gv[FC];
                ld8(&sm.kraw[tt][cb], kv);
                ld8(&sm.qraw[tt][cb], qv);
                if constexpr (KDA) {
                    ld8(&sm.araw[tt][cb], gv);
                } else {
#pragma unroll
                    for (int n = 0; n < FC; ++n) gv[n] = sm.araw[tt][0];
                }
                float vr[FR];
                vrows(tt, vr);
                const float beta = sm.bt[tt];
                float u[FR], e[FR], y[FR];
#pragma unroll
                for (int r = 0; r < FR; ++r) {
                    u[r] = 0.f;
#pragma unroll
                    for (int n = 0; n < FC; ++n) u[r] = fmaf(M[r][n], gv[n] * kv[n], u[r]);
                }
                row_sums(u);
#pragma unroll
                for (int r = 0; r < FR; ++r) e[r] = vr[r] - u[r];
#pragma unroll
                for (int r = 0; r < FR; ++r) {
                    const float de = beta * e[r];
#pragma unroll
                    for (int n = 0; n < FC; ++n) M[r][n] = fmaf(M[r][n], gv[n], de * kv[n]);
                    y[r] = 0.f;
#pragma unroll
                    for (int n = 0; n < FC; ++n) y[r] = fmaf(M[r][n], qv[n], y[r]);
                }
                finish(tt, ob, y, e);
            }
        }
        prev_ta = ta;
        prev_cnt = cnt;
        ta = next;
        cnt = ncnt;
    };
    while (cnt > 0) {
        window(R0, std::integral_constant<int, 0>{});
        if (cnt <= 0) break;
        window(R1, std::integral_constant<int, 1>{});
    }
    __syncthreads();
    flush(prev_ta, prev_cnt, (L + WIN - 1) / WIN % 2 ^ 1);   // the last window's buffer
    if (write_y) {
        for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += FT) {
            const int64_t t = L + idx / QR;
            a.y[s * a.sy.seq + t * a.sy.tok + h * a.sy.head + qb * QR + idx % QR] = 0.f;
        }
    }
    if (a.state_out) {
        if (((uintptr_t)a.state_out & 15) == 0) {
            rw_state(a.state_out + unit * S * S, true);
        } else {
#pragma unroll
            for (int r = 0; r < FR; ++r)
#pragma unroll
                for (int n = 0; n < FC; ++n) a.state_out[unit * S * S + (int64_t)(row + (r ^ hsw)) * S + lc * FC + n] = M[r][n];
        }
    }
}

// ------------------------------------------------------------------ backward walk

constexpr int RW = 4;              // rows per wave
constexpr int NW = QR / RW;        // waves per workgroup (two per SIMD)
constexpr int BT = 64 * NW;        // backward threads
constexpr int CT = BT / S;         // threads per column in the stretch staging
static_assert(RW == 4 && NW == WIN && WIN * QR <= BT, "backward layout");

template <bool KDA>
struct alignas(16) BwdLds {
    union {
        // the thread's column sums over its rows at columns (lane, lane + 64), per walked
        // token: cqce = (Mt^T gy lo, hi, dM^T delta lo, hi), cm = Mt^T dd; hx: the window-start
        // dg partials (dM_out .* M0)
        struct {
            float4 cqce[WIN][BT];
            float2 cm[WIN][BT];
            float2 hx[BT];
        } sl;
        // stretch data of the window-start pass: k./c for columns (lane, lane + 64), beta e
        // of the quarter's rows, window products
        struct {
            float2 kt[VS][64];
            float4 det[VS][QR / 4];
            float2 cend[NWS][64];
        } sa;
    };
    int wflag[NWS];            // unscaled windows of the stretch
    float hsc[NW];             // scalar gate: per-wave window-start dg
    // window data for columns (lane, lane + 64): (d.*k, scale q./d), -beta k./d, k./c for the
    // replay (raw k in an unscaled window), (c, d) and k for the column sums, the window
    // product; rows: beta e, gy, e; per token: beta, sum over the quarter's rows of
    // (beta e) gy, and the dbeta of each wave's rows
    float4 wv[WIN][64];
    float2 wh[WIN][64];
    float2 kt8[WIN][64];
    float4 de8[WIN][QR / 4], gy8[WIN][QR / 4], e8[WIN][QR / 4];
    float4 pcd[WIN][64];
    float bt[WIN], s1[WIN];
    float2 pP[64];
    float dd8[WIN][QR];        // dd of the quarter's rows per token
    float D1[WIN][WIN];        // [s][t]: delta_s . gy_t over the quarter's rows
    float D2w[NW][WIN][WIN];   // [wave][t][s]: delta_s . dd_t over the wave's rows
};

template <bool KDA, int DT>
__global__ void __launch_bounds__(BT, 1)
bwd128_kernel(const BwdArgs a) {
    constexpr int GW = KDA ? S : 1;
    constexpr int NP = KDA ? 3 : 2;     // partial slots per quarter: dq | dk (| dg)
    __shared__ BwdLds<KDA> sm;

    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int C = a.C;
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr0 = w * RW;             // first row of this wave within the quarter
    const int row0 = qb * QR + wr0;     // first state row of this wave
    const float scale = a.scale;
    // after the dd reduce-scatter, lane 16 m of the wave holds row {0, 2, 1, 3}[m]
    const int dd_row = ((lane >> 4) & 1) * 2 + (lane >> 5);
    const int ci = tid & (S - 1), cr = tid >> 7;   // stretch staging: column, column thread

    const int64_t tok_ae = a.H_v;
    const float *snapu = a.snap + unit * a.n_ck_max * S * S + (int64_t)row0 * S + lane;
    float4 *vsb = reinterpret_cast<float4 *>(a.vsbuf) +
                  ((unit * NQ + qb) * (int64_t)a.nvs_max) * (RW / 2 * BT) + tid;
    const In<DT> *kp = inp<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qp = inp<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    // window gate factors, token stride tok_ae * GW: running products c and suffix products d
    // (an unscaled window: the gates a, and 1)
    const float *cb = a.cbuf + (s * a.T * a.H_v + h) * GW;
    const float *db = a.dbuf + (s * a.T * a.H_v + h) * GW;
    const int nwin_T = (a.T + WIN - 1) / WIN;
    const int32_t *wfl = a.wflag + s * nwin_T * a.H_v + h;            // window stride H_v
    const float *eb = a.ebuf + (s * a.T * a.H_v + h) * S + qb * QR;  // errors, token stride tok_ae*S
    const In<DT> *gyp = inp<DT>(a.gy) + s * a.sgy.seq + h * a.sgy.head + qb * QR;
    const In<DT> *bp = inp<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;

    float X[RW][2];   // the walked gradient dM (scaled by d inside a window)
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
    auto rows4 = [](const float4 &v, float (&x)[RW]) { x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w; };

    // ---- stretch staging: k./c per token (the forward's arithmetic, so the replay is bit
    // exact), beta e, the product over each window and the unscaled-window flags
    auto stage_stretch = [&](int va, int vb) {
        constexpr int NTASK = NWS / CT;   // windows per thread
        In<DT> kv[NTASK][WIN];            // in the input type until used
        float cv[NTASK][WIN];
        int cn[NTASK];
#pragma unroll
        for (int x = 0; x < NTASK; ++x) {
            const int t0 = va + (cr + CT * x) * WIN;
            cn[x] = t0 < vb ? min(WIN, vb - t0) : 0;
#pragma unroll
            for (int tt = 0; tt < WIN; ++tt) {   // clamped loads (no branch per token)
                const int64_t t = min(t0 + tt, vb - 1);
                const In<DT> k = kp[t * a.sk.tok + ci];
                const float c = cb[t * tok_ae * GW + (KDA ? ci : 0)];
                kv[x][tt] = tt < cn[x] ? k : In<DT>(0);
                cv[x][tt] = tt < cn[x] ? c : 1.f;
            }
        }
        int fl = 0;
        if (tid < NWS && va + tid * WIN < vb) fl = wfl[(int64_t)((va + tid * WIN) / WIN) * a.H_v];
        constexpr int NDE = VS * QR / BT;
        float ev[NDE];
        In<DT> bv[NDE];
#pragma unroll
        for (int x = 0; x < NDE; ++x) {
            const int tr = (tid >> 5) + (BT / QR) * x;   // token within the stretch
            const int64_t t = va + tr;
            ev[x] = va + tr < vb ? eb[t * tok_ae * S + (tid & 31)] : 0.f;
            bv[x] = va + tr < vb ? bp[t * a.sb.tok] : In<DT>(0);
        }
        __syncthreads();   // the previous users of the slot area are done
        if (tid < NWS) sm.wflag[tid] = fl;
#pragma unroll
        for (int x = 0; x < NDE; ++x)
            reinterpret_cast<float *>(sm.sa.det[(tid >> 5) + (BT / QR) * x])[tid & 31] = fin<DT>(bv[x]) * ev[x];
        __syncthreads();
#pragma unroll
        for (int x = 0; x < NTASK; ++x) {
            const int m = cr + CT * x;
            float c = 1.f;   // window product: c at the last token
#pragma unroll
            for (int tt = 0; tt < WIN; ++tt) {
                if (tt < cn[x]) c = cv[x][tt];
                reinterpret_cast<float *>(&sm.sa.kt[m * WIN + tt][ci & 63])[ci >> 6] = fin<DT>(kv[x][tt]) * rcp(cv[x][tt]);
            }
            if (KDA || ci < 64) {
                if (KDA) reinterpret_cast<float *>(&sm.sa.cend[m][ci & 63])[ci >> 6] = c;
                else sm.sa.cend[m][ci] = make_float2(c, c);
            }
        }
        __syncthreads();
    };

    // ---- replay of window m of the stretch from M (its start state) to its end
    auto replay_window = [&](float (&M)[RW][2], int va, int vb, int m) {
        const int t0 = va + m * WIN;
        const int cnt = min(WIN, vb - t0);
        if (sm.wflag[m] == 0) {
            auto step = [&](int tt) {
                const int tr = m * WIN + tt;
                const float2 kv = sm.sa.kt[tr][lane];
                float dv[RW];
                rows4(sm.sa.det[tr][w], dv);
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    M[r][0] = fmaf(dv[r], kv.x, M[r][0]);
                    M[r][1] = fmaf(dv[r], kv.y, M[r][1]);
                }
            };
            if (cnt == WIN) {   // full window: unrolled, so all its LDS reads go out together
#pragma unroll
                for (int tt = 0; tt < WIN; ++tt) step(tt);
            } else {
                for (int tt = 0; tt < cnt; ++tt) step(tt);
            }
            const float2 ce = sm.sa.cend[m][lane];
#pragma unroll
            for (int r = 0; r < RW; ++r) M[r][0] *= ce.x, M[r][1] *= ce.y;
        } else {
            // unscaled window: keys and gates come from memory directly (rare path)
            for (int tt = 0; tt < cnt; ++tt) {
                const int tr = m * WIN + tt;
                const int64_t t = t0 + tt;
                const float kv[2] = {fin<DT>(kp[t * a.sk.tok + lane]), fin<DT>(kp[t * a.sk.tok + lane + 64])};
                const float av[2] = {cb[t * tok_ae * GW + (KDA ? lane : 0)],
                                     cb[t * tok_ae * GW + (KDA ? lane + 64 : 0)]};
                float dv[RW];
                rows4(sm.sa.det[tr][w], dv);
#pragma unroll
                for (int r = 0; r < RW; ++r)
#pragma unroll
                    for (int n = 0; n < 2; ++n) M[r][n] = fmaf(M[r][n], av[n], dv[r] * kv[n]);
            }
        }
    };

    // ---- window data, prefetched into registers one window ahead: thread (tok = w, lane)
    // holds, for columns (lane, lane + 64) of token tok, the window's running product c and
    // the product d of its later gates (an unscaled window: the gate a, and 1), k, q, and
    // beta; thread tid < WIN * QR holds gy, e and beta of row tid & 31 of token tid >> 5
    // (k, q, beta and gy kept in the input type until staged)
    float wc[2], wd[2], re = 0.f;
    In<DT> wk[2], wq[2], wbt = In<DT>(0), rgy = In<DT>(0), rb = In<DT>(0);
    int wlast = 0;   // the window's last token
    auto load_window = [&](int t0, int cnt) {
        const int64_t t = t0 + w;
        wlast = cnt - 1;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            wc[n] = w < cnt ? cb[t * tok_ae * GW + (KDA ? lane + 64 * n : 0)] : 1.f;
            wd[n] = w < cnt ? db[t * tok_ae * GW + (KDA ? lane + 64 * n : 0)] : 1.f;
            wk[n] = w < cnt ? kp[t * a.sk.tok + lane + 64 * n] : In<DT>(0);
            wq[n] = w < cnt ? qp[t * a.sq.tok + lane + 64 * n] : In<DT>(0);
        }
        wbt = w < cnt ? bp[t * a.sb.tok] : In<DT>(0);
        if (tid < WIN * QR && (tid >> 5) < cnt) {
            const int64_t tr = t0 + (tid >> 5);
            rgy = gyp[tr * a.sgy.tok + (tid & 31)];
            re = eb[tr * tok_ae * S + (tid & 31)];
            rb = bp[tr * a.sb.tok];
        }
    };
    // store the window's data and its derived vectors (cnt tokens; unscaled when direct)
    auto stage_window = [&](int cnt, bool direct) {
        const int tt = w;
        const float c[2] = {wc[0], wc[1]}, d[2] = {wd[0], wd[1]};   // unscaled: the gate, 1
        const float rd[2] = {direct ? 1.f : rcp(d[0]), direct ? 1.f : rcp(d[1])};
        const float kk[2] = {fin<DT>(wk[0]), fin<DT>(wk[1])}, qq[2] = {fin<DT>(wq[0]), fin<DT>(wq[1])};
        const float bt = fin<DT>(wbt);
        sm.wv[tt][lane] = make_float4(kk[0] * d[0], kk[1] * d[1], scale * qq[0] * rd[0], scale * qq[1] * rd[1]);
        sm.wh[tt][lane] = make_float2(-bt * kk[0] * rd[0], -bt * kk[1] * rd[1]);
        sm.kt8[tt][lane] = direct ? make_float2(kk[0], kk[1])
                                  : make_float2(kk[0] * rcp(c[0]), kk[1] * rcp(c[1]));
        sm.pcd[tt][lane] = make_float4(c[0], c[1], d[0], d[1]);
        if (tt == wlast) sm.pP[lane] = direct ? make_float2(1.f, 1.f) : make_float2(c[0], c[1]);   // window product
        if (lane == 0) sm.bt[tt] = bt;
        if (tid < WIN * QR) {   // rows: beta e, gy, e, and the sum of (beta e) gy per token
            const int rt = tid >> 5, r = tid & 31;
            const float gyv = fin<DT>(rgy);
            const float de = fin<DT>(rb) * re;
            reinterpret_cast<float *>(sm.de8[rt])[r] = de;
            reinterpret_cast<float *>(sm.gy8[rt])[r] = gyv;
            reinterpret_cast<float *>(sm.e8[rt])[r] = re;
            const float p = half_sum(rt < cnt ? de * gyv : 0.f);
            if (r == 0) sm.s1[rt] = p;
        }
    };


    // ---- dg.  Each token's dg is colsum(dMp .* Mp).  At the first token t0 of a window it
    // equals colsum(dM_out .* M0), with dM_out the walked gradient before the window and M0
    // the state at its start; inside the window dg_t = dg_{t+1} + q.*dq_t
    // - k.*(dM_t^T delta_t - Mp_t^T du_t), from the next window's dg_t0 down (after the
    // sequence's last token: the column sums of dstate_out .* M_final).  The quarter writes,
    // per token, the increment (at t0: dg_t0 itself) and, per sequence, the final column
    // sums; the partial-sum kernel runs the recursion over each window.
    // column sums over the wave's rows of dM .* M (per column; the scalar gate: per wave)
    auto colsum_xm = [&](const float (&M)[RW][2], float (&hp)[2]) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            hp[n] = X[0][n] * M[0][n];
#pragma unroll
            for (int r = 1; r < RW; ++r) hp[n] = fmaf(X[r][n], M[r][n], hp[n]);
        }
    };
    // the recursion's start: column sums over the quarter's rows of dstate_out .* M_final
    auto start_dg = [&](const float (&Mf)[RW][2]) {
        float hp[2];
        colsum_xm(Mf, hp);
        __syncthreads();   // the stretch data (sharing the slot area) is no longer read
        if constexpr (KDA) {
            sm.sl.hx[tid] = make_float2(hp[0], hp[1]);
        } else {
            const float hs = wave_sum(hp[0] + hp[1]);
            if (lane == 0) sm.hsc[w] = hs;
        }
        __syncthreads();
        float *hf = a.hfin + (unit * NQ + qb) * GW;
        if constexpr (KDA) {
            if (tid < S) {
                float g = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) g += reinterpret_cast<const float *>(&sm.sl.hx[ww * 64 + (tid & 63)])[tid >> 6];
                hf[tid] = g;
            }
        } else {
            if (tid == 0) {
                float g = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) g += sm.hsc[ww];
                hf[0] = g;
            }
        }
    };

    // outputs of a reduced window, stored after the next window is staged and its successor's
    // loads are issued, so no wait for loads ever stands behind them
    float o_dq[2] = {0.f, 0.f}, o_dk[2] = {0.f, 0.f}, o_dg[2] = {0.f, 0.f}, o_dv = 0.f, o_db = 0.f;
    int o_ta = 0, o_cnt = 0;
    auto flush_outputs = [&]() {
        const int tt = w;
        if (tt < o_cnt) {
            const int64_t rq = ((s * a.T + o_ta + tt) * a.H_v + h) * NQ + qb;
            float *pp = a.part + rq * NP * S + lane;
            pp[0] = o_dq[0]; pp[64] = o_dq[1];
            pp[S] = o_dk[0]; pp[S + 64] = o_dk[1];
            if constexpr (KDA) {
                pp[2 * S] = o_dg[0]; pp[2 * S + 64] = o_dg[1];
            } else if (lane == 0) {
                a.pgbuf[rq << 1] = o_dg[0];
                a.pgbuf[(rq << 1) + 1] = 0.f;
            }
            if (lane < QR) a.dv[((s * a.T + o_ta + tt) * a.H_v + h) * S + qb * QR + lane] = o_dv;
            if (lane == 0) a.pbuf[rq] = o_db;
        }
        o_cnt = 0;
    };

    // ---- column sums of the cnt walked tokens of the window at ta: fixed-order sum over the
    // waves, scaling, and the quarter's partial outputs; dv and dbeta from the rows' dd.
    // Wave w handles token w, lane the columns (lane, lane + 64) and row lane (< 32).
    auto reduce_columns = [&](int ta, int cnt, bool direct) {
        const int tt = w;
        if (tt < cnt) {   // uniform over the wave
            float4 A = sm.sl.cqce[tt][lane];
            float2 B = sm.sl.cm[tt][lane];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) {
                const float4 x = sm.sl.cqce[tt][ww * 64 + lane];
                const float2 y = sm.sl.cm[tt][ww * 64 + lane];
                A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
                B.x += y.x; B.y += y.y;
            }
            if (!direct && tt > 0) {   // from the window-start state to the state before token tt
                float d2 = 0.f;        // lane s: delta_s . dd_tt over the quarter
                if (lane < WIN) {
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) d2 += sm.D2w[ww][tt][lane];
                }
#pragma unroll
                for (int sx = 0; sx < WIN - 1; ++sx) {   // all reads issued together; tokens sx >= tt add zero
                    const float2 kc = sm.kt8[sx][lane];
                    const float d1v = sx < tt ? sm.D1[sx][tt] : 0.f;
                    const float d2v = sx < tt ? as_f(__builtin_amdgcn_readlane(as_i(d2), sx)) : 0.f;
                    A.x = fmaf(kc.x, d1v, A.x); A.y = fmaf(kc.y, d1v, A.y);
                    B.x = fmaf(kc.x, d2v, B.x); B.y = fmaf(kc.y, d2v, B.y);
                }
            }
            const float4 cd = sm.pcd[tt][lane];
            const float4 v4 = sm.wv[tt][lane];
            const float beta = sm.bt[tt], s1 = sm.s1[tt];
            const float cq[2] = {A.x, A.y}, ce[2] = {A.z, A.w}, cm[2] = {B.x, B.y};
            const float c[2] = {cd.x, cd.y}, d[2] = {cd.z, cd.w};
            // k = (k.*d)./d (d is 1 in an unscaled window), scale q = (scale q./d).*d
            const float kv[2] = {v4.x * rcp(d[0]), v4.y * rcp(d[1])}, sq[2] = {v4.z * d[0], v4.w * d[1]};
            float inc[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float qs = fmaf(c[n], cq[n], kv[n] * s1);   // dq / scale
                o_dq[n] = scale * qs;
                const float e1 = d[n] * ce[n], e2 = beta * c[n] * cm[n];   // dM^T delta, -Mp^T du
                o_dk[n] = e1 - e2;
                // dg increment: q.*dq - k.*(dM^T delta - Mp^T du)
                inc[n] = fmaf(sq[n], qs, -kv[n] * (e1 + e2));
            }
            if (tt == 0 && KDA) {   // the window's first token: dg itself, from the window-start partials
                inc[0] = inc[1] = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    const float2 v = sm.sl.hx[ww * 64 + lane];
                    inc[0] += v.x;
                    inc[1] += v.y;
                }
            }
            if constexpr (KDA) {
                o_dg[0] = inc[0];
                o_dg[1] = inc[1];
            } else {
                float gsum = wave_sum(inc[0] + inc[1]);
                if (tt == 0) {
                    gsum = sm.hsc[0];
#pragma unroll
                    for (int ww = 1; ww < NW; ++ww) gsum += sm.hsc[ww];
                }
                o_dg[0] = gsum;
            }
            // dv = beta dd and dbeta = sum over rows of dd (v - u), row lane of the quarter
            const float ddr = lane < QR ? sm.dd8[tt][lane] : 0.f;
            const float er = lane < QR ? reinterpret_cast<const float *>(sm.e8[tt])[lane] : 0.f;
            o_dv = beta * ddr;
            o_db = half_sum(ddr * er);
        }
        o_ta = ta;
        o_cnt = cnt;
    };

    // one token of the reverse walk (window position tt of the window at ta); leaves the
    // thread's column sums of the token in its slots.
    // In a column-scaled window the column sums are taken against the window-start state Mh;
    // the state before token t differs from it by sum_{s<t} delta_s (k_s./c_s)^T, whose
    // contribution the column-sum phase adds from the row products delta_s . gy_t and
    // delta_s . dd_t.  An unscaled window (rare) replays the state before token tt from the
    // window start, with the forward's arithmetic: M <- M .* a_s + delta_s k_s^T.
    auto walk_token = [&](int ta, int tt, const float (&Mh)[RW][2], auto direct_tag) {
        constexpr bool direct = decltype(direct_tag)::value;
        float Mt[RW][2];
#pragma unroll
        for (int r = 0; r < RW; ++r) Mt[r][0] = Mh[r][0], Mt[r][1] = Mh[r][1];
        if constexpr (direct) {
            for (int sx = 0; sx < tt; ++sx) {
                const float4 cd = sm.pcd[sx][lane];   // the gates (unscaled window)
                const float2 kv = sm.kt8[sx][lane];   // raw k (unscaled window)
                float dv[RW];
                rows4(sm.de8[sx][w], dv);
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    Mt[r][0] = fmaf(Mt[r][0], cd.x, dv[r] * kv.x);
                    Mt[r][1] = fmaf(Mt[r][1], cd.y, dv[r] * kv.y);
                }
            }
        }
        const float4 v4 = sm.wv[tt][lane];
        const float2 h2 = sm.wh[tt][lane];
        const float kd[2] = {v4.x, v4.y}, qh[2] = {v4.z, v4.w};
        const float kh[2] = {h2.x, h2.y};
        float gy[RW], de[RW];
        rows4(sm.gy8[tt][w], gy);
        rows4(sm.de8[tt][w], de);
        // dM += scale gy q^T (q./d carries the scale and the column factor)
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) X[r][n] = fmaf(gy[r], qh[n], X[r][n]);
        float dpart[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) dpart[r] = fmaf(X[r][1], kd[1], X[r][0] * kd[0]);
        // column sums that do not need dd
        float cq[2], ce[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            cq[n] = Mt[0][n] * gy[0];
            ce[n] = X[0][n] * de[0];
#pragma unroll
            for (int r = 1; r < RW; ++r) {
                cq[n] = fmaf(Mt[r][n], gy[r], cq[n]);
                ce[n] = fmaf(X[r][n], de[r], ce[n]);
            }
        }
        // dd = dM k: reduce-scatter over the 64 lanes, then broadcast
        float hsum[2];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            auto sw = __builtin_amdgcn_permlane32_swap(as_i(dpart[2 * pr]), as_i(dpart[2 * pr + 1]),
                                                       false, false);
            hsum[pr] = as_f(sw[0]) + as_f(sw[1]);
        }
        auto sw16 = __builtin_amdgcn_permlane16_swap(as_i(hsum[0]), as_i(hsum[1]), false, false);
        const float gsum = row16_sum(as_f(sw16[0]) + as_f(sw16[1]));
        float dd[RW];
        dd[0] = as_f(__builtin_amdgcn_readlane(as_i(gsum), 0));
        dd[2] = as_f(__builtin_amdgcn_readlane(as_i(gsum), 16));
        dd[1] = as_f(__builtin_amdgcn_readlane(as_i(gsum), 32));
        dd[3] = as_f(__builtin_amdgcn_readlane(as_i(gsum), 48));
        const float beta = sm.bt[tt];
        if ((lane & 15) == 0) sm.dd8[tt][wr0 + dd_row] = gsum;   // dv and dbeta come later
        if constexpr (!direct) {   // delta_s . dd_t over the wave's rows, lane s
            if (lane < WIN) {
                const float4 x = sm.de8[lane][w];
                sm.D2w[w][tt][lane] = fmaf(x.w, dd[3], fmaf(x.z, dd[2], fmaf(x.y, dd[1], x.x * dd[0])));
            }
        }
        float cm[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            cm[n] = Mt[0][n] * dd[0];
#pragma unroll
            for (int r = 1; r < RW; ++r) cm[n] = fmaf(Mt[r][n], dd[r], cm[n]);
        }
        // dM += du k^T with du = -beta dd (k./d carries -beta)
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) X[r][n] = fmaf(dd[r], kh[n], X[r][n]);
        if constexpr (direct) {   // unscaled window: dM .* a now
            const float4 cd = sm.pcd[tt][lane];
#pragma unroll
            for (int r = 0; r < RW; ++r) X[r][0] *= cd.x, X[r][1] *= cd.y;
        }
        sm.sl.cqce[tt][tid] = make_float4(cq[0], cq[1], ce[0], ce[1]);
        sm.sl.cm[tt][tid] = make_float2(cm[0], cm[1]);
    };

    const int n_ck = (L + C - 1) / C;
    bool first = true;
    for (int sg = n_ck - 1; sg >= 0; --sg) {
        const int t0 = sg * C, t1 = min(t0 + C, L);
        const int nvs = (t1 - t0 + VS - 1) / VS;
        float M[RW][2];
        auto load_snapshot = [&]() {
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int n = 0; n < 2; ++n) M[r][n] = snapu[(int64_t)sg * S * S + r * S + n * 64];
        };
        if (nvs > 1) {   // stretch starts beyond the first, kept in the workspace
            load_snapshot();
            for (int v = 0; v < nvs - 1; ++v) {
                const int va = t0 + v * VS, vb = va + VS;
                stage_stretch(va, vb);
                for (int m = 0; m < NWS; ++m) replay_window(M, va, vb, m);
#pragma unroll
                for (int c = 0; c < RW / 2; ++c)
                    vsb[(int64_t)(v + 1) * (RW / 2 * BT) + c * BT] =
                        make_float4(M[2 * c][0], M[2 * c][1], M[2 * c + 1][0], M[2 * c + 1][1]);
            }
        }
        for (int v = nvs - 1; v >= 0; --v) {
            const int va = t0 + v * VS, vb = min(va + VS, t1);
            const int nwin = (vb - va + WIN - 1) / WIN;
            if (v == 0) {
                load_snapshot();
            } else {
#pragma unroll
                for (int c = 0; c < RW / 2; ++c) {
                    const float4 x = vsb[(int64_t)v * (RW / 2 * BT) + c * BT];
                    M[2 * c][0] = x.x; M[2 * c][1] = x.y; M[2 * c + 1][0] = x.z; M[2 * c + 1][1] = x.w;
                }
            }
            stage_stretch(va, vb);
            // states at every window start of the stretch
            float SS[NWS][RW][2];
            int flags = 0;
#pragma unroll
            for (int m = 0; m < NWS; ++m) {
                if (m < nwin) {
#pragma unroll
                    for (int r = 0; r < RW; ++r) SS[m][r][0] = M[r][0], SS[m][r][1] = M[r][1];
                    if (m + 1 < nwin) replay_window(M, va, vb, m);
                    flags |= (sm.wflag[m] != 0) << m;
                }
            }
            if (first) {   // the final state, for the start of the dg recursion
                replay_window(M, va, vb, nwin - 1);
                start_dg(M);
                first = false;
            }
            load_window(va + (nwin - 1) * WIN, vb - (va + (nwin - 1) * WIN));
            for (int m = nwin - 1; m >= 0; --m) {
                const int ta = va + m * WIN;
                const int cnt = min(WIN, vb - ta);
                const bool direct = (flags >> m) & 1;
                __syncthreads();   // the previous window (or the stretch pass) is done
                stage_window(cnt, direct);
                if (m > 0) load_window(ta - WIN, WIN);   // prefetch: the registers are free now
                __syncthreads();
                {   // delta_s . gy_t over the quarter's rows for s = w (lane: t = lane & 7, rows 4 (lane >> 3)..)
                    const int t = lane & 7, c4 = lane >> 3;
                    const float4 x = sm.de8[w][c4], y = sm.gy8[t][c4];
                    float p = fmaf(x.w, y.w, fmaf(x.z, y.z, fmaf(x.y, y.y, x.x * y.x)));
                    p += dpp<0x128>(p);   // row_ror 8
                    auto p16 = __builtin_amdgcn_permlane16_swap(as_i(p), as_i(p), false, false);
                    p = as_f(p16[0]) + as_f(p16[1]);
                    auto p32 = __builtin_amdgcn_permlane32_swap(as_i(p), as_i(p), false, false);
                    p = as_f(p32[0]) + as_f(p32[1]);
                    if (lane < WIN) sm.D1[w][lane] = p;
                }
                flush_outputs();   // the previous window's results
                float M0[RW][2];   // state at the window start
                switch (m) {
#define GDN_PICK(k)                                                                    \
    case k:                                                                            \
        for (int r = 0; r < RW; ++r) M0[r][0] = SS[k][r][0], M0[r][1] = SS[k][r][1];   \
        break;
                    GDN_PICK(0) GDN_PICK(1) GDN_PICK(2) GDN_PICK(3)
                    GDN_PICK(4) GDN_PICK(5) GDN_PICK(6) GDN_PICK(7)
#undef GDN_PICK
                }
                if (cnt == WIN && !direct) {
                    // full column-scaled window: unrolled, so every LDS offset is constant
#pragma unroll
                    for (int tt = WIN - 1; tt >= 0; --tt) walk_token(ta, tt, M0, std::false_type{});
                } else if (!direct) {
                    for (int tt = cnt - 1; tt >= 0; --tt) walk_token(ta, tt, M0, std::false_type{});
                } else {
                    for (int tt = cnt - 1; tt >= 0; --tt) walk_token(ta, tt, M0, std::true_type{});
                }
                if (!direct) {   // fold the window's decay into the walked gradient
                    const float2 P = sm.pP[lane];
#pragma unroll
                    for (int r = 0; r < RW; ++r) X[r][0] *= P.x, X[r][1] *= P.y;
                }
                {   // window-start dg partials
                    float hp[2];
                    colsum_xm(M0, hp);
                    if constexpr (KDA) {
                        sm.sl.hx[tid] = make_float2(hp[0], hp[1]);
                    } else {
                        const float hs = wave_sum(hp[0] + hp[1]);
                        if (lane == 0) sm.hsc[w] = hs;
                    }
                }
                __syncthreads();
                reduce_columns(ta, cnt, direct);
            }
        }
    }

    flush_outputs();
    {
        float *ds = a.dstate + unit * S * S + (int64_t)row0 * S + lane;
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n) ds[r * S + n * 64] = X[r][n];
    }
    for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += BT) {
        const int64_t t = L + idx / QR;
        a.dv[((s * a.T + t) * a.H_v + h) * S + qb * QR + idx % QR] = 0.f;
    }
}

// ------------------------------------------------------------------ quarter / head sums

// dq and dk: sums over the four quarters and the value heads of each key head (increasing
// order); dbeta: sum over the quarters; dg: per 8-token window, the quarters' window-start
// value at its first token and, from its last token down, the next window's first-token value
// (after the sequence's last token, the final-state column sums) plus the quarters' increments.
// V columns per thread (4 when every buffer allows 16-byte accesses, else 1).
template <int V>
__device__ __forceinline__ void ldv(const float *p, float (&x)[V]) {
    if constexpr (V == 4) {
        const float4 t = *reinterpret_cast<const float4 *>(p);
        x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else {
        x[0] = *p;
    }
}
template <int V>
__device__ __forceinline__ void stv(float *p, const float (&x)[V]) {
    if constexpr (V == 4) *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    else *p = x[0];
}

template <int V>
__global__ void __launch_bounds__(256) combine128_kernel(const Combine128Args a) {
    const int64_t T = a.T, n = a.n_seqs_launch, Hk = a.H_k, Hv = a.H_v;
    const int64_t G = a.kda ? S : 1;
    const int64_t VG = a.kda ? V : 1;          // columns per dg chain item
    const int64_t nwin = (T + WIN - 1) / WIN;
    const int64_t n_qk = n * T * Hk * (S / V);     // dq and dk items (V columns each)
    const int64_t n_g = n * nwin * Hv * (G / VG);   // dg (window, column group) chains
    const int64_t n_b = n * T * Hv;                 // dbeta elements
    const int64_t NP = a.kda ? 3 : 2;
    const int64_t total = n_qk + n_g + n_b;
    const int64_t seq0 = (int64_t)a.s_base;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        if (idx < n_qk) {
            const int i = (int)(idx % (S / V)) * V;
            int64_t rest = idx / (S / V);
            const int kh = (int)(rest % Hk);
            rest /= Hk;
            const int t = (int)(rest % T);
            const int sl = (int)(rest / T);
            float q[V], k[V];
#pragma unroll
            for (int c = 0; c < V; ++c) q[c] = k[c] = 0.f;
            if (t < a.lens[sl]) {
                for (int h = kh; h < Hv; h += (int)Hk) {   // value heads in increasing order
                    const float *pp = a.part + ((((seq0 + sl) * T + t) * Hv + h) * NQ) * NP * S + i;
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        float x[V], y[V];
                        ldv<V>(pp + (qb * NP + 0) * S, x);
                        ldv<V>(pp + (qb * NP + 1) * S, y);
#pragma unroll
                        for (int c = 0; c < V; ++c) q[c] += x[c], k[c] += y[c];
                    }
                }
            }
            const int64_t o = (((seq0 + sl) * T + t) * Hk + kh) * S + i;
            stv<V>(a.dq + o, q);
            stv<V>(a.dk + o, k);
        } else if (idx < n_qk + n_g) {
            const int64_t j = idx - n_qk;
            const int i = (int)(j % (G / VG)) * (int)VG;
            int64_t rest = j / (G / VG);
            const int h = (int)(rest % Hv);
            rest /= Hv;
            const int m = (int)(rest % nwin);
            const int sl = (int)(rest / nwin);
            const int t0 = m * WIN, L = a.lens[sl];
            const int cnt = max(0, min(WIN, L - t0));
            // sum over the quarters of the dg partial of token t (columns i .. i + V - 1; the
            // scalar gate: one value)
            auto part_sum = [&](int t, float (&g)[V]) {
                const int64_t rt = (((seq0 + sl) * T + t) * Hv + h) * NQ;
#pragma unroll
                for (int c = 0; c < V; ++c) g[c] = 0.f;
                if (a.kda) {
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        float x[V];
                        ldv<V>(a.part + ((rt + qb) * NP + 2) * S + i, x);
#pragma unroll
                        for (int c = 0; c < V; ++c) g[c] += x[c];
                    }
                } else {
#pragma unroll
                    for (int x = 0; x < 2 * NQ; ++x) g[0] += a.pgbuf[rt * 2 + x];
                }
            };
            float carry[V];
#pragma unroll
            for (int c = 0; c < V; ++c) carry[c] = 0.f;
            if (cnt > 0) {
                if (t0 + WIN < L) {
                    part_sum(t0 + WIN, carry);
                } else {
                    const float *hf = a.hfin + ((seq0 + sl) * Hv + h) * NQ * G + i;
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        float x[V] = {};
                        if (a.kda) ldv<V>(hf + qb * G, x);
                        else x[0] = hf[qb * G];
#pragma unroll
                        for (int c = 0; c < V; ++c) carry[c] += x[c];
                    }
                }
            }
            for (int tt = WIN - 1; tt >= 0; --tt) {
                const int t = t0 + tt;
                if (t >= T) continue;
                float g[V];
#pragma unroll
                for (int c = 0; c < V; ++c) g[c] = 0.f;
                if (tt < cnt) {
                    float p[V];
                    part_sum(t, p);
#pragma unroll
                    for (int c = 0; c < V; ++c) {
                        if (tt == 0) {
                            g[c] = p[c];
                        } else {
                            carry[c] += p[c];
                            g[c] = carry[c];
                        }
                    }
                }
                float *dst = a.dg + (((seq0 + sl) * T + t) * Hv + h) * G + i;
                if (a.kda) stv<V>(dst, g);
                else dst[0] = g[0];
            }
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

hipError_t launch_gate128(const GateArgs &a, hipStream_t st) {
    const int64_t items = (int64_t)a.n_seqs_launch * ((a.T + WIN - 1) / WIN) * a.H_v;
    if (items <= 0) return hipSuccess;
    int64_t blocks = a.G == 1 ? (items + 255) / 256 : (items + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    const void *fn = a.dtype == GDN_DTYPE_BF16  ? (const void *)gate128_kernel<GDN_DTYPE_BF16>
                     : a.dtype == GDN_DTYPE_F16 ? (const void *)gate128_kernel<GDN_DTYPE_F16>
                                                : (const void *)gate128_kernel<GDN_DTYPE_F32>;
    return launch(fn, a, (int)blocks, 256, st);
}

hipError_t launch_fwd128(const FwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st) {
    const int blocks = n_seqs_launch * a.H_v * NQ;
    const bool few = blocks < 512;   // fewer than two workgroups per CU: one row per lane, eight waves
    const void *fn = nullptr;
#define GDN_F128(DT)                                                                                  \
    fn = few ? (kda ? (const void *)fwd128_kernel<true, 1, DT> : (const void *)fwd128_kernel<false, 1, DT>) \
             : (kda ? (const void *)fwd128_kernel<true, 2, DT> : (const void *)fwd128_kernel<false, 2, DT>);
    if (a.dtype == GDN_DTYPE_BF16) {
        GDN_F128(GDN_DTYPE_BF16)
    } else if (a.dtype == GDN_DTYPE_F16) {
        GDN_F128(GDN_DTYPE_F16)
    } else {
        GDN_F128(GDN_DTYPE_F32)
    }
#undef GDN_F128
    return launch(fn, a, blocks, few ? 512 : 256, st);
}

hipError_t launch_bwd128(const BwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st) {
    const int blocks = n_seqs_launch * a.H_v * NQ;
    const void *fn = a.dtype == GDN_DTYPE_BF16
                         ? (kda ? (const void *)bwd128_kernel<true, GDN_DTYPE_BF16> : (const void *)bwd128_kernel<false, GDN_DTYPE_BF16>)
                     : a.dtype == GDN_DTYPE_F16
                         ? (kda ? (const void *)bwd128_kernel<true, GDN_DTYPE_F16> : (const void *)bwd128_kernel<false, GDN_DTYPE_F16>)
                         : (kda ? (const void *)bwd128_kernel<true, GDN_DTYPE_F32> : (const void *)bwd128_kernel<false, GDN_DTYPE_F32>);
    return launch(fn, a, blocks, BT, st);
}

hipError_t launch_combine128(const Combine128Args &a, hipStream_t st) {
    auto a16 = [](const void *p) { return p == nullptr || ((uintptr_t)p & 15) == 0; };
    const bool vec = a16(a.part) && a16(a.hfin) && a16(a.dq) && a16(a.dk) && a16(a.dg);
    const int64_t V = vec ? 4 : 1, VG = a.kda ? V : 1;
    const int64_t G = a.kda ? S : 1;
    const int64_t total = (int64_t)a.n_seqs_launch *
                          (a.T * (a.H_k * (S / V) + a.H_v) + (int64_t)((a.T + WIN - 1) / WIN) * a.H_v * (G / VG));
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    return vec ? launch((const void *)combine128_kernel<4>, a, (int)blocks, 256, st)
               : launch((const void *)combine128_kernel<1>, a, (int)blocks, 256, st);
}

}  // namespace gdn
