// gdn_mf.hip -- gfx950 kernels of the gated delta rule for head size S = 128 on the matrix
// cores (fp32 MFMA, v_mfma_f32_16x16x4f32).
//
// Blocks of W = 16 tokens.  Per (sequence, value head) unit the state M = S^T (row j = value
// index, column i = key index) follows M_t = M_{t-1} diag(a_t) + delta_t k_t^T (meTile,
// "Training kernels and gradients", section "Recurrent delta attention").  Inside a block
// the state is carried column-scaled, M_t = Mh_t diag(c_t), with c_t the running product of
// the gates from the block's first token (taken in token order), so the 16 token steps of a
// block become three dense products against the block's start state plus 16 x 16 matrices
// that couple the tokens of the block:
//   u_t = M_start (c_t k_t) + sum_{s<t} delta_s (k_s/c_s . c_t k_t)       (Gram A)
//   y_t = scale (M_start (c_t q_t) + sum_{s<=t} delta_s (k_s/c_s . c_t q_t))   (Gram B)
// and the errors e = v - u of the block solve a unit triangular system whose inverse Te the
// prep kernel writes once per block.  The backward carries the state gradient as
// X = dM_t diag(c_t) within a block; its row sums dd = dM k solve the transposed-order
// triangular system (inverse Tb), and the column sums dq, dk are dense products against the
// block's start state (M) and end gradient (X) plus rank-16 corrections from the block's
// Gram matrices of the rows.  The per-channel gate gradient dg follows from the column sums
// by an exact telescoping identity, with its value at each block's first token taken
// directly as a column sum of the gradient times the start state.
//
// A block whose running products leave [2^-60, 2^60] in some column is processed token by
// token instead: each token is a one-token block whose state is first scaled by the token's
// gates (c = 1 after that), so the arithmetic is the per-token recurrence itself.
//
// Rows of M evolve independently in both directions ("metal: GATED_DELTA_NET_BACK",
// approval review: each row of the state is updated on its own), so a unit is split into
// four row quarters of 32 rows, one workgroup each; the quarters of the backward meet only
// in column sums, which each quarter writes as partials that the combine kernel adds in a
// fixed order (and, for dq and dk, over the value heads of a key head in increasing order).
//
// MFMA lane layout (16x16x4 f32): lane l supplies A[l%16][kappa] and B[kappa][l%16], and
// holds D[4(l/16) + r][l%16] in accumulator register r.  Every product below uses the
// contraction index kappa = 4(l/16) + s in its step s (within each block of 16), so a
// D-layout accumulator is directly the B operand of the next product.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int S = 128;
constexpr int W = 16;          // tokens per block
constexpr int QR = 32;         // rows per quarter
constexpr int NQ = S / QR;     // quarters per unit
constexpr float kLo = 0x1p-60f, kHi = 0x1p60f;
constexpr int SP = S + 4;      // [token][column] LDS rows
constexpr int KP = W + 4;      // [column][token] LDS rows
constexpr int RP = QR + 4;     // [token][row] LDS rows (backward row data)
constexpr int MATF = 3 * W * W;   // floats of block matrices: Bm, Te, Tb

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ void st4(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }
// compiler-only barrier: keeps memory accesses of one phase from being hoisted into another
__device__ __forceinline__ void fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int as_i(float x) { return __builtin_bit_cast(int, x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), CTRL, 0xF, 0xF, true));
}
// sum over the 16 lanes of a DPP row (every lane receives it)
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}
// sum over the four 16-lane rows of the wave at the same position (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows4_sum(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(as_i(v), as_i(v), false, false);
    v = as_f(p[0]) + as_f(p[1]);
    auto q = __builtin_amdgcn_permlane32_swap(as_i(v), as_i(v), false, false);
    return as_f(q[0]) + as_f(q[1]);
}

// Input element type (GDN_DTYPE_*) of q, k, v, g, beta and gy, widened exactly at the load.
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

// Global accesses go through buffer resources: a wave-uniform base (scalar registers), a 32-bit
// byte offset per lane and a scalar byte offset for the token (so a block's token loop costs
// no vector address arithmetic).  Bases are taken at the block's first token; the host keeps
// 16 token strides of every tensor below 2^31 bytes.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7fffffff, 0x00020000);
}
template <int DT>
__device__ __forceinline__ float bld(Rsrc r, uint32_t vbytes, uint32_t sbytes) {
    if constexpr (DT == GDN_DTYPE_F32) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vbytes, sbytes, 0));
    } else {
        const unsigned short x = __builtin_amdgcn_raw_buffer_load_b16(r, vbytes, sbytes, 0);
        if constexpr (DT == GDN_DTYPE_BF16) return __builtin_bit_cast(float, (uint32_t)x << 16);
        else return (float)__builtin_bit_cast(_Float16, x);
    }
}
__device__ __forceinline__ float bldf(Rsrc r, uint32_t vbytes, uint32_t sbytes) { return bld<GDN_DTYPE_F32>(r, vbytes, sbytes); }
__device__ __forceinline__ void bst(Rsrc r, float v, uint32_t vbytes, uint32_t sbytes) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, vbytes, sbytes, 0);
}
template <int DT>
__device__ __forceinline__ const In<DT> *tin(const void *p) {
    return reinterpret_cast<const In<DT> *>(p);
}

// Block index -> (unit of the launch, quarter); the four quarters of a unit go to one XCD
// (workgroups are dealt to the eight XCDs round robin) so they share its L2.
__device__ __forceinline__ void map_block(int b, int nb, int &unit, int &qb) {
    int lin = b;
    if (nb % (8 * NQ) == 0) lin = (b % 8) * (nb / 8) + b / 8;
    unit = lin / NQ;
    qb = lin % NQ;
}

// ------------------------------------------------------------------ block preparation

// Per block of every (sequence, value head): the flag of a block processed token by token,
// and the block matrices Bm (upper triangle of B with its diagonal), Te = (I + diag(beta) A)^-1
// and Tb = (I + A diag(beta))^-1, A the strict upper triangle of the Gram A; a token-by-token
// block gets Bm = diag(k_t . q_t) and Te = Tb = I.  One wave per block (lane: columns lane
// and lane + 64 over the block's tokens).
struct alignas(16) PrepLds {
    float kr[W][SP], kc[W][SP], qc[W][SP];
    float am[W][W + 1];
    float bt[W];
};

template <int DT>
__global__ void __launch_bounds__(64) prep128_kernel(const Mf128Args a) {
    __shared__ PrepLds sm;
    constexpr uint32_t ES = sizeof(In<DT>);
    const int lane = threadIdx.x, lm = lane & 15, g4 = lane >> 4;
    const int nblk = (a.T + W - 1) / W;
    const int64_t items = (int64_t)a.n_seqs_launch * nblk * a.H_v;
    const uint32_t gt = (uint32_t)a.sg.tok * ES, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int h = (int)(it % a.H_v);
        const int64_t rest = it / a.H_v;
        const int b = (int)(rest % nblk), sl = (int)(rest / nblk);
        const int t0 = b * W, cnt = min(W, a.lens[sl] - t0);
        if (cnt <= 0) continue;
        const int64_t s = a.s_base + sl;
        const int hk = h % a.H_k;
        const Rsrc rg = rsrc(tin<DT>(a.g) + s * a.sg.seq + (int64_t)t0 * a.sg.tok + h * a.sg.head);
        const Rsrc rk = rsrc(tin<DT>(a.k) + s * a.sk.seq + (int64_t)t0 * a.sk.tok + hk * a.sk.head);
        const Rsrc rq = rsrc(tin<DT>(a.q) + s * a.sq.seq + (int64_t)t0 * a.sq.tok + hk * a.sq.head);
        float c[2][W], kv[2][W], qv[2][W];
        bool ok = true;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint32_t i = lane + 64 * n;
            float run = 1.f;
#pragma unroll
            for (int tt = 0; tt < W; ++tt) {
                float av = 1.f, kx = 0.f, qx = 0.f;
                if (tt < cnt) {
                    av = expf(bld<DT>(rg, (a.kda ? i : 0u) * ES, tt * gt));
                    kx = bld<DT>(rk, i * ES, tt * kt);
                    qx = bld<DT>(rq, i * ES, tt * qt);
                }
                run = tt == 0 ? av : run * av;
                c[n][tt] = run;
                kv[n][tt] = kx;
                qv[n][tt] = qx;
                ok = ok && run >= kLo && run <= kHi;
            }
        }
        const bool direct = __ballot(!ok) != 0;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int i = lane + 64 * n;
#pragma unroll
            for (int tt = 0; tt < W; ++tt) {
                const float cv = direct ? 1.f : c[n][tt];
                sm.kr[tt][i] = kv[n][tt] * rcp(cv);
                sm.kc[tt][i] = kv[n][tt] * cv;
                sm.qc[tt][i] = qv[n][tt] * cv;
            }
        }
        if (lane < W) {
            const Rsrc rb = rsrc(tin<DT>(a.beta) + s * a.sb.seq + (int64_t)t0 * a.sb.tok + h * a.sb.head);
            sm.bt[lane] = lane < cnt ? bld<DT>(rb, 0, lane * (uint32_t)a.sb.tok * ES) : 0.f;
        }
        __syncthreads();
        // Grams G[s][t] = kr_s . kc_t and kr_s . qc_t (D layout: s = 4 g4 + r, t = lm)
        f4 ga0 = zero4(), ga1 = zero4(), gb0 = zero4(), gb1 = zero4();
#pragma unroll
        for (int kb = 0; kb < S / 16; kb += 2) {
            const f4 ar0 = ld4(&sm.kr[lm][16 * kb + 4 * g4]), ar1 = ld4(&sm.kr[lm][16 * kb + 16 + 4 * g4]);
            const f4 bc0 = ld4(&sm.kc[lm][16 * kb + 4 * g4]), bc1 = ld4(&sm.kc[lm][16 * kb + 16 + 4 * g4]);
            const f4 bq0 = ld4(&sm.qc[lm][16 * kb + 4 * g4]), bq1 = ld4(&sm.qc[lm][16 * kb + 16 + 4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ga0 = mfma(ar0[x], bc0[x], ga0);
                gb0 = mfma(ar0[x], bq0[x], gb0);
                ga1 = mfma(ar1[x], bc1[x], ga1);
                gb1 = mfma(ar1[x], bq1[x], gb1);
            }
        }
        const f4 gA = ga0 + ga1, gB = gb0 + gb1;
        float *wm = a.wmat + ((s * nblk + b) * a.H_v + h) * (int64_t)MATF;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int sg = 4 * g4 + r, tt = lm;
            sm.am[sg][tt] = (!direct && sg < tt) ? gA[r] : 0.f;
            wm[sg * W + tt] = direct ? (sg == tt ? gB[r] : 0.f) : (sg <= tt ? gB[r] : 0.f);
        }
        __syncthreads();
        // rows of the unit upper triangular inverses: lane sg < 16 of Te, 16 + sg of Tb; the
        // matrix is read whole into registers first (broadcast LDS reads)
        if (lane < 2 * W) {
            const int sg = lane & 15;
            const bool tb = lane >= W;
            float v[W];
#pragma unroll
            for (int tt = 0; tt < W; ++tt) {
                float acc = 0.f;
#pragma unroll
                for (int rho = 0; rho < tt; ++rho) {
                    if (rho >= sg) {
                        const float l = tb ? sm.am[rho][tt] * sm.bt[tt] : sm.bt[rho] * sm.am[rho][tt];
                        acc = fmaf(v[rho], l, acc);
                    }
                }
                v[tt] = tt < sg ? 0.f : (tt == sg ? 1.f : -acc);
            }
            float *dst = wm + (tb ? 2 : 1) * W * W + sg * W;
#pragma unroll
            for (int tt = 0; tt < W; ++tt) dst[tt] = direct ? (tt == sg ? 1.f : 0.f) : v[tt];
        }
        if (lane == 0) a.wflag[(s * nblk + b) * a.H_v + h] = direct ? 1 : 0;
        __syncthreads();
    }
}

// ------------------------------------------------------------------ forward scan

// A workgroup owns a row quarter (32 rows) of a unit: two waves of 16 rows, each holding the
// state transposed as eight 16 x 16 accumulator tiles, tile ib: lane l register r holds
// M[j0 + l%16][16 ib + 4(l/16) + r].  Thread tid stages column tid of each block; the
// block's inputs are loaded into registers one block ahead.
struct alignas(16) FwdMfLds {
    float kc[W][SP], qc[W][SP];   // c.*k, c.*q   [token][column]
    float kr[S][KP];              // k./c         [column][token]
    float pv[S];                  // block product (scaled block) or the token's gates
};

template <int DT>
__global__ void __launch_bounds__(128, 2) fwd_mf_kernel(const Mf128Args a) {
    __shared__ FwdMfLds sm;
    constexpr uint32_t ES = sizeof(In<DT>);
    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int j0 = qb * QR + wv * 16;
    const int nblk = (a.T + W - 1) / W;
    const bool vec_state = (((uintptr_t)a.state0 | (uintptr_t)a.state_out) & 15) == 0;
    const In<DT> *gin = tin<DT>(a.g) + s * a.sg.seq + h * a.sg.head;
    const In<DT> *kin = tin<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qin = tin<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const In<DT> *vin = tin<DT>(a.v) + s * a.sv.seq + h * a.sv.head;
    const In<DT> *bin = tin<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
    float *yout = a.y ? a.y + s * a.sy.seq + h * a.sy.head : nullptr;
    float *eout = a.ebuf + (s * a.T * a.H_v + h) * S;
    const uint32_t gt = (uint32_t)a.sg.tok * ES, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES,
                   vt = (uint32_t)a.sv.tok * ES, bt = (uint32_t)a.sb.tok * ES, yt = (uint32_t)a.sy.tok * 4,
                   et = (uint32_t)(a.H_v * S) * 4;
    const uint32_t gcol = (a.kda ? (uint32_t)tid : 0u) * ES;

    f4 M[S / 16];
    {
        const float *p = a.state0 + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) {
            if (vec_state) M[ib] = ld4(p + 16 * ib);
            else M[ib] = f4{p[16 * ib], p[16 * ib + 1], p[16 * ib + 2], p[16 * ib + 3]};
        }
    }
    auto store_state = [&](float *base) {
        float *p = base + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) st4(p + 16 * ib, M[ib]);
    };
    float *snap = a.snap + unit * a.n_ck_max * S * S;

    // inputs of one block, loaded a block ahead: column tid of g, k, q for its 16 tokens; per
    // lane v and beta at (token 4(l/16) + r, row j0 + l%16) and the block matrices' operands
    struct Pre {
        float g[W], k[W], q[W];
        float v[4], b[4], te[4], bm[4];
        int dir;
    };
    auto prefetch = [&](Pre &P, int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        const float *wm = a.wmat + bi * MATF;
        P.dir = a.wflag[bi];
        const Rsrc rg = rsrc(gin + (int64_t)t0 * a.sg.tok), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                   rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rv = rsrc(vin + (int64_t)t0 * a.sv.tok),
                   rb = rsrc(bin + (int64_t)t0 * a.sb.tok), rw = rsrc(wm);
#pragma unroll
        for (int tt = 0; tt < W; ++tt) {
            const bool ok = tt < cnt;
            P.g[tt] = ok ? bld<DT>(rg, gcol, tt * gt) : 0.f;
            P.k[tt] = ok ? bld<DT>(rk, tid * ES, tt * kt) : 0.f;
            P.q[tt] = ok ? bld<DT>(rq, tid * ES, tt * qt) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t tt = 4 * g4 + r;
            const bool ok = (int)tt < cnt;
            P.v[r] = ok ? bld<DT>(rv, (j0 + lm) * ES + tt * vt, 0) : 0.f;
            P.b[r] = ok ? bld<DT>(rb, tt * bt, 0) : 0.f;
            P.te[r] = bldf(rw, (W * W + tt * W + lm) * 4, 0);
            P.bm[r] = bldf(rw, (tt * W + lm) * 4, 0);
        }
    };

    // one (sub)block of n tokens from token tw, its column data staged; vv, bb: v and beta,
    // teA, bmA: operands of Te^T and Bm^T
    auto block = [&](int tw, int n, const float (&vv)[4], const float (&bb)[4], const float (&teA)[4],
                     const float (&bmA)[4]) {
        // u and y against the start state: D[token][row]
        f4 u0 = zero4(), u1 = zero4(), y0 = zero4(), y1 = zero4();
#pragma unroll
        for (int ib = 0; ib < S / 16; ib += 2) {
            const f4 ak0 = ld4(&sm.kc[lm][16 * ib + 4 * g4]), aq0 = ld4(&sm.qc[lm][16 * ib + 4 * g4]);
            const f4 ak1 = ld4(&sm.kc[lm][16 * ib + 16 + 4 * g4]), aq1 = ld4(&sm.qc[lm][16 * ib + 16 + 4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                u0 = mfma(ak0[x], M[ib][x], u0);
                y0 = mfma(aq0[x], M[ib][x], y0);
                u1 = mfma(ak1[x], M[ib + 1][x], u1);
                y1 = mfma(aq1[x], M[ib + 1][x], y1);
            }
        }
        const f4 U = u0 + u1;
        f4 Y = y0 + y1;
        // e = (v - u0) Te, delta = beta e, y += Bm^T delta
        f4 E = zero4();
#pragma unroll
        for (int x = 0; x < 4; ++x) E = mfma(teA[x], vv[x] - U[x], E);
        float D[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) D[r] = bb[r] * E[r];
#pragma unroll
        for (int x = 0; x < 4; ++x) Y = mfma(bmA[x], D[x], Y);
        {
            const Rsrc re = rsrc(eout + (int64_t)tw * (a.H_v * S));
            const Rsrc ry = rsrc(yout ? yout + (int64_t)tw * a.sy.tok : eout);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t tt = 4 * g4 + r;
                if ((int)tt < n) {
                    if (yout) bst(ry, a.scale * Y[r], (j0 + lm) * 4 + tt * yt, 0);
                    bst(re, E[r], (j0 + lm) * 4 + tt * et, 0);
                }
            }
        }
        // M += delta (k./c)^T
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) {
            const f4 ar = ld4(&sm.kr[16 * ib + lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) M[ib] = mfma(ar[x], D[x], M[ib]);
        }
    };
    auto scale_state = [&]() {
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) M[ib] *= ld4(&sm.pv[16 * ib + 4 * g4]);
    };

    const int i = tid;   // staged column
    Pre P;
    if (L > 0) prefetch(P, 0);
    for (int b = 0; b * W < L; ++b) {
        const int t0 = b * W, cnt = min(W, L - t0);
        if (t0 % a.C == 0) store_state(snap + (int64_t)(t0 / a.C) * S * S);
        if (!P.dir) {
            float run = 1.f;
            float krow[W];
#pragma unroll
            for (int tt = 0; tt < W; ++tt) {
                const float av = tt < cnt ? expf(P.g[tt]) : 1.f;
                run = tt == 0 ? av : run * av;
                krow[tt] = P.k[tt] * rcp(run);
                sm.kc[tt][i] = P.k[tt] * run;
                sm.qc[tt][i] = P.q[tt] * run;
            }
#pragma unroll
            for (int tt = 0; tt < W; tt += 4) st4(&sm.kr[i][tt], f4{krow[tt], krow[tt + 1], krow[tt + 2], krow[tt + 3]});
            sm.pv[i] = run;
            const float vv[4] = {P.v[0], P.v[1], P.v[2], P.v[3]}, bb[4] = {P.b[0], P.b[1], P.b[2], P.b[3]};
            const float teA[4] = {P.te[0], P.te[1], P.te[2], P.te[3]}, bmA[4] = {P.bm[0], P.bm[1], P.bm[2], P.bm[3]};
            __syncthreads();
            if (t0 + W < L) prefetch(P, t0 + W);   // the registers are free again
            block(t0, cnt, vv, bb, teA, bmA);
            scale_state();
            __syncthreads();
        } else {   // token by token: each token a one-token block after its gates scale the state
            const int64_t bi = (s * nblk + b) * a.H_v + h;
            const float *wm = a.wmat + bi * MATF;
            const Rsrc rg = rsrc(gin + (int64_t)t0 * a.sg.tok), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                       rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rv = rsrc(vin + (int64_t)t0 * a.sv.tok),
                       rb = rsrc(bin + (int64_t)t0 * a.sb.tok);
            for (int tau = 0; tau < cnt; ++tau) {
                const float av = expf(bld<DT>(rg, gcol, tau * gt));
                const float kx = bld<DT>(rk, i * ES, tau * kt);
                const float qx = bld<DT>(rq, i * ES, tau * qt);
#pragma unroll
                for (int tt = 0; tt < W; ++tt) {
                    sm.kc[tt][i] = tt == 0 ? kx : 0.f;
                    sm.qc[tt][i] = tt == 0 ? qx : 0.f;
                }
#pragma unroll
                for (int tt = 0; tt < W; tt += 4) st4(&sm.kr[i][tt], f4{tt == 0 ? kx : 0.f, 0.f, 0.f, 0.f});
                sm.pv[i] = av;
                float vv[4], bb[4], teA[4], bmA[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = 4 * g4 + r;
                    vv[r] = tt == 0 ? bld<DT>(rv, (j0 + lm) * ES, tau * vt) : 0.f;
                    bb[r] = tt == 0 ? bld<DT>(rb, 0, tau * bt) : 0.f;
                    teA[r] = tt == lm ? 1.f : 0.f;
                    bmA[r] = (tt == 0 && lm == 0) ? wm[tau * (W + 1)] : 0.f;
                }
                __syncthreads();
                scale_state();
                block(t0 + tau, 1, vv, bb, teA, bmA);
                __syncthreads();
            }
            if (t0 + W < L) prefetch(P, t0 + W);
        }
    }
    if (yout) {
        for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += 128) {
            const int64_t t = L + idx / QR;
            yout[t * a.sy.tok + qb * QR + (int)(idx % QR)] = 0.f;
        }
    }
    if (a.state_out) {
        if (vec_state) {
            store_state(a.state_out + unit * S * S);
        } else {
            float *p = a.state_out + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
            for (int ib = 0; ib < S / 16; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) p[16 * ib + r] = M[ib][r];
        }
    }
}

// ------------------------------------------------------------------ backward

// A workgroup owns a row quarter (32 rows) of a unit; wave w owns its 32 rows at the 32
// columns 32w .. 32w + 31: four 16 x 16 tiles (jb, ib), lane l register r holding element
// [16 jb + 4(l/16) + r][16 ib + l%16] of the quarter's rows and the wave's columns.  The
// start state of a block (M) and the gradient X = dM diag(c) (Xt) are held so.  Blocks are
// walked from the last; a block's start state is the start of its 32-token stretch (a
// snapshot, or a stretch start the segment's first pass left in the workspace) replayed over
// at most one block.
constexpr int VS = 2 * W;      // tokens per stretch
constexpr int SCR_DD = 2 * W * (W + 4) - 512;   // dd0 partials at the scratch's end

struct alignas(16) BwdMfLds {
    float cc[4][32][KP], kk[4][32][KP], qq[4][32][KP];   // per wave: c, k, q [column][token]
    float pw[4][32];                                     // per wave: a token's gates (token by token)
    float sgy[W][RP], ee[W][RP], du[W][RP];              // scale gy, e, du of the quarter's rows
    float bt[W];
    float bm[W][W], tb[W][W];
    float scr[4][2 * W * (W + 4)];                       // per wave: transposes, partial sums
};
static_assert(2 * W * (W + 4) >= 16 * RP && 2 * W * (W + 4) >= 512, "scratch size");

template <int DT>
__global__ void __launch_bounds__(256, 2) bwd_mf_kernel(const Mf128Args a) {
    __shared__ BwdMfLds sm;
    constexpr uint32_t ES = sizeof(In<DT>);
    int ul, qb;
    map_block(blockIdx.x, gridDim.x, ul, qb);
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int C = a.C;
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int r0 = qb * QR;                 // first row of the quarter
    const int c0 = wv * 32;                 // first column of the wave
    const int nblk = (a.T + W - 1) / W;
    const float scale = a.scale;
    const bool kda = a.kda != 0;
    float *scr = sm.scr[wv];
    float (*cc)[KP] = sm.cc[wv];
    float (*kk)[KP] = sm.kk[wv];
    float (*qq)[KP] = sm.qq[wv];
    // bases of this (sequence, head) and byte strides per token
    const In<DT> *gin = tin<DT>(a.g) + s * a.sg.seq + h * a.sg.head;
    const In<DT> *kin = tin<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qin = tin<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const In<DT> *gyin = tin<DT>(a.gy) + s * a.sgy.seq + h * a.sgy.head + r0;
    const In<DT> *bin = tin<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
    const int64_t row0 = s * a.T * a.H_v + h;   // workspace row of token 0; token stride H_v
    const float *ein = a.ebuf + row0 * S + r0;
    float *dvout = a.dv + row0 * S + r0;
    float *pout = a.part + row0 * (NQ * 3 * S) + qb * (3 * S);
    float *pbout = a.pbuf + row0 * (2 * NQ) + 2 * qb;
    const uint32_t gt = (uint32_t)a.sg.tok * ES, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES,
                   gyt = (uint32_t)a.sgy.tok * ES, bt = (uint32_t)a.sb.tok * ES;
    const uint32_t et = (uint32_t)a.H_v * S * 4, pt = (uint32_t)a.H_v * (NQ * 3 * S) * 4,
                   pbt = (uint32_t)a.H_v * (2 * NQ) * 4;

    auto load_state = [&](const float *base, f4 (&Mr)[2][2]) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) Mr[jb][ib][r] = base[(16 * jb + 4 * g4 + r) * S + c0 + 16 * ib + lm];
    };
    auto save_state = [&](float *base, const f4 (&Mr)[2][2]) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) base[(16 * jb + 4 * g4 + r) * S + c0 + 16 * ib + lm] = Mr[jb][ib][r];
    };

    f4 Xt[2][2];
    if (a.dstate_out) {
        load_state(a.dstate_out + unit * S * S + (int64_t)r0 * S, Xt);
    } else {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) Xt[jb][ib] = zero4();
    }

    // operands of the wave's columns at (column 16 ib + l%16, tokens 4(l/16) .. + 3), read from
    // the staged block when used: k./c, c.*q, c.*k
    auto KR = [&](int ib) {
        const f4 cv = ld4(&cc[16 * ib + lm][4 * g4]), kv = ld4(&kk[16 * ib + lm][4 * g4]);
        return f4{kv[0] * rcp(cv[0]), kv[1] * rcp(cv[1]), kv[2] * rcp(cv[2]), kv[3] * rcp(cv[3])};
    };
    auto QC = [&](int ib) { return ld4(&qq[16 * ib + lm][4 * g4]) * ld4(&cc[16 * ib + lm][4 * g4]); };
    auto KC = [&](int ib) { return ld4(&kk[16 * ib + lm][4 * g4]) * ld4(&cc[16 * ib + lm][4 * g4]); };

    // ---- staging of a (sub)block: n tokens from tw; dir: one token, c = 1, its gates in pw
    auto stage = [&](int tw, int n, bool dir, int tau0, const float *wm) {
        {   // columns: lane holds column c0 + (lane & 31), tokens 8 (lane >> 5) .. + 7
            const int ic = lane & 31, hf = lane >> 5;
            const uint32_t i = c0 + ic;
            const Rsrc rg = rsrc(gin + (int64_t)tw * a.sg.tok), rk = rsrc(kin + (int64_t)tw * a.sk.tok),
                       rq = rsrc(qin + (int64_t)tw * a.sq.tok);
            const uint32_t gcol = (kda ? i : 0u) * ES;
            float av[8], kv[8], qv[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const uint32_t tt = 8 * hf + x;
                const bool valid = (int)tt < n;
                av[x] = valid ? expf(bld<DT>(rg, gcol + tt * gt, 0)) : 1.f;
                kv[x] = valid ? bld<DT>(rk, i * ES + tt * kt, 0) : 0.f;
                qv[x] = valid ? bld<DT>(rq, i * ES + tt * qt, 0) : 0.f;
            }
            float c[8];
            c[0] = av[0];
#pragma unroll
            for (int x = 1; x < 8; ++x) c[x] = c[x - 1] * av[x];
            const float c7 = __shfl(c[7], ic, 64);
            if (hf) {
                c[0] = c7 * av[0];
#pragma unroll
                for (int x = 1; x < 8; ++x) c[x] = c[x - 1] * av[x];
            }
            if (dir) {
                if (hf == 0) sm.pw[wv][ic] = av[0];
#pragma unroll
                for (int x = 0; x < 8; ++x) c[x] = 1.f;
            }
#pragma unroll
            for (int x = 0; x < 8; x += 4) {
                st4(&cc[ic][8 * hf + x], f4{c[x], c[x + 1], c[x + 2], c[x + 3]});
                st4(&kk[ic][8 * hf + x], f4{kv[x], kv[x + 1], kv[x + 2], kv[x + 3]});
                st4(&qq[ic][8 * hf + x], f4{qv[x], qv[x + 1], qv[x + 2], qv[x + 3]});
            }
        }
        {   // rows of the quarter: scale gy, e; beta; the block matrices
            const Rsrc rgy = rsrc(gyin + (int64_t)tw * a.sgy.tok), re = rsrc(ein + (int64_t)tw * (a.H_v * S));
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int idx = tid + 256 * x;
                const uint32_t tt = idx >> 5, j = idx & 31;
                const bool valid = (int)tt < n;
                sm.sgy[tt][j] = valid ? scale * bld<DT>(rgy, j * ES + tt * gyt, 0) : 0.f;
                sm.ee[tt][j] = valid ? bldf(re, j * 4 + tt * et, 0) : 0.f;
            }
            if (tid < W) sm.bt[tid] = tid < n ? bld<DT>(rsrc(bin + (int64_t)tw * a.sb.tok), tid * bt, 0) : 0.f;
            const Rsrc rw = rsrc(wm);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int idx = tid + 256 * x, m = idx >> 8, e = idx & 255, sg = e >> 4, tt = e & 15;
                float val;
                if (!dir) val = bldf(rw, ((m == 0 ? 0 : 2 * W * W) + e) * 4, 0);
                else if (m == 0) val = (sg == 0 && tt == 0) ? bldf(rw, tau0 * (W + 1) * 4, 0) : 0.f;
                else val = sg == tt ? 1.f : 0.f;
                if (m == 0) sm.bm[sg][tt] = val;
                else sm.tb[sg][tt] = val;
            }
        }
        __syncthreads();
    };
    // per-column factor of the wave's columns (block product, or the token's gates)
    auto col_factor = [&](int ib, bool dir) { return dir ? sm.pw[wv][16 * ib + lm] : cc[16 * ib + lm][W - 1]; };
    auto scale_cols = [&](f4 (&Z)[2][2], bool dir) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const float p = col_factor(ib, dir);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) Z[jb][ib] *= p;
        }
    };

    // ---- replay of a staged (sub)block: Mr from the block's start to its end
    auto replay = [&](f4 (&Mr)[2][2], bool dir) {
        if (dir) scale_cols(Mr, true);
        const f4 kr0 = KR(0), kr1 = KR(1);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int tt = 4 * g4 + x;
                const float dl = sm.bt[tt] * sm.ee[tt][16 * jb + lm];
                Mr[jb][0] = mfma(dl, kr0[x], Mr[jb][0]);
                Mr[jb][1] = mfma(dl, kr1[x], Mr[jb][1]);
            }
        if (!dir) scale_cols(Mr, false);
    };

    // column sum over the quarter's rows of X .* Mr, for the wave's columns 16 ib + l%16
    auto colsum_xm = [&](const f4 (&Mr)[2][2], float (&out)[2]) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            float v = 0.f;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(Xt[jb][ib][r], Mr[jb][ib][r], v);
            out[ib] = rows4_sum(v);
        }
    };

    // ---- walk of a staged (sub)block with start state Mb; n tokens from tw.  Phases: the row
    // Gram G1 = delta^T sgy; dd0 = X kr over the wave's columns (partials to the scratch); the
    // column sums P1 = M^T sgy (finished into dq) and P3 = X^T delta; after the partials, waves
    // 0 and 1 solve for dd of their 16 rows; after that, P2 = M^T du, G2 = delta^T du, the
    // update of X, and the outputs.
    auto walk = [&](const f4 (&Mb)[2][2], int tw, int n, bool dir) {
        if (!dir) scale_cols(Xt, false);   // X = dM diag(c) at the block's last token
        const float btl = sm.bt[lm];
        // G1[s][t] = delta_s . sgy_t (D layout s = 4(l/16) + r, t = l%16) and its transpose
        f4 g1 = zero4();
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const f4 sg4 = ld4(&sm.sgy[lm][16 * jb + 4 * g4]), e4 = ld4(&sm.ee[lm][16 * jb + 4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) g1 = mfma(btl * e4[x], sg4[x], g1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) scr[(4 * g4 + r) * (W + 4) + lm] = g1[r];
        const f4 g1t = ld4(&scr[lm * (W + 4) + 4 * g4]);
        fence();
        // dd0 = X kr (partial over the wave's columns), via X transposed through the scratch
        f4 dd0[2] = {zero4(), zero4()};
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) scr[(4 * g4 + r) * RP + 16 * ib + lm] = Xt[jb][ib][r];
            const f4 xt0 = ld4(&scr[lm * RP + 4 * g4]), xt1 = ld4(&scr[lm * RP + 16 + 4 * g4]);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int il = 16 * ib + 4 * g4 + x;
                    const float ar = kk[il][lm] * rcp(cc[il][lm]);
                    dd0[jb] = mfma(ar, ib ? xt1[x] : xt0[x], dd0[jb]);
                }
            fence();
        }
        st4(&scr[SCR_DD + lane * 4], dd0[0]);
        st4(&scr[SCR_DD + 256 + lane * 4], dd0[1]);
        fence();
        // P1 = M^T sgy + kr (G1 masked s <= t): dq = c P1, and the dg increment's first term
        float inc[2][4];
        float gsum[4] = {0.f, 0.f, 0.f, 0.f};
        const Rsrc rpo = rsrc(pout + (int64_t)tw * (pt / 4));
        {
            f4 p1[2] = {zero4(), zero4()};
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const f4 sg4 = ld4(&sm.sgy[lm][16 * jb + 4 * g4]);
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) p1[ib] = mfma(sg4[x], Mb[jb][ib][x], p1[ib]);
            }
            {
                const f4 kr0 = KR(0), kr1 = KR(1);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float wq = 4 * g4 + x <= lm ? g1[x] : 0.f;
                    p1[0] = mfma(wq, kr0[x], p1[0]);
                    p1[1] = mfma(wq, kr1[x], p1[1]);
                }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const f4 cv = ld4(&cc[16 * ib + lm][4 * g4]), qc = QC(ib);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = 4 * g4 + r;
                    inc[ib][r] = qc[r] * p1[ib][r];
                    if (tt < n) bst(rpo, cv[r] * p1[ib][r], (c0 + 16 * ib + lm) * 4 + tt * pt, 0);
                }
            }
        }
        fence();
        // P3 = X^T delta + qc (G1^T masked s >= t), the rest after G2
        f4 p3[2] = {zero4(), zero4()};
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const f4 e4 = ld4(&sm.ee[lm][16 * jb + 4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float dl = btl * e4[x];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) p3[ib] = mfma(dl, Xt[jb][ib][x], p3[ib]);
            }
        }
        {
            const f4 qc0 = QC(0), qc1 = QC(1);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float wk1 = 4 * g4 + x >= lm ? g1t[x] : 0.f;
                p3[0] = mfma(wk1, qc0[x], p3[0]);
                p3[1] = mfma(wk1, qc1[x], p3[1]);
            }
        }
        __syncthreads();   // dd0 partials
        if (wv < 2) {      // dd of row block jb = wv: Tb (dd0 + Bm sgy), then du, dv, dbeta
            const int jb = wv;
            f4 acc = ld4(&sm.scr[0][SCR_DD + jb * 256 + lane * 4]);
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) acc += ld4(&sm.scr[w2][SCR_DD + jb * 256 + lane * 4]);
            const f4 bm4 = ld4(&sm.bm[lm][4 * g4]), tb4 = ld4(&sm.tb[lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) acc = mfma(bm4[x], sm.sgy[4 * g4 + x][16 * jb + lm], acc);
            f4 dd = zero4();
#pragma unroll
            for (int x = 0; x < 4; ++x) dd = mfma(tb4[x], acc[x], dd);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * g4 + r;
                const float bv = sm.bt[tt];
                sm.du[tt][16 * jb + lm] = -bv * dd[r];
                const float pb = row16_sum(dd[r] * sm.ee[tt][16 * jb + lm]);
                if (tt < n) {
                    bst(rsrc(dvout + (int64_t)tw * (et / 4)), bv * dd[r], (16 * jb + lm) * 4 + tt * et, 0);
                    if (lm == 0) bst(rsrc(pbout + (int64_t)tw * (pbt / 4)), pb, jb * 4 + tt * pbt, 0);
                }
            }
        }
        __syncthreads();   // du
        // P2 = M^T du + kr (G2 masked s < t); G2 = delta^T du; P3 += kc (G2^T masked s > t)
        f4 p2[2] = {zero4(), zero4()}, g2 = zero4();
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const f4 du4 = ld4(&sm.du[lm][16 * jb + 4 * g4]), e4 = ld4(&sm.ee[lm][16 * jb + 4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) p2[ib] = mfma(du4[x], Mb[jb][ib][x], p2[ib]);
                g2 = mfma(btl * e4[x], du4[x], g2);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) scr[(4 * g4 + r) * (W + 4) + lm] = g2[r];
        const f4 g2t = ld4(&scr[lm * (W + 4) + 4 * g4]);
        {
            const f4 kr0 = KR(0), kr1 = KR(1), kc0 = KC(0), kc1 = KC(1);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int sg = 4 * g4 + x;
                const float wk3 = sg < lm ? g2[x] : 0.f, wk2 = sg > lm ? g2t[x] : 0.f;
                p2[0] = mfma(wk3, kr0[x], p2[0]);
                p2[1] = mfma(wk3, kr1[x], p2[1]);
                p3[0] = mfma(wk2, kc0[x], p3[0]);
                p3[1] = mfma(wk2, kc1[x], p3[1]);
            }
        }
        fence();
        // X += sgy qc^T + du kc^T
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const f4 qc = QC(ib), kc = KC(ib);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int tt = 4 * g4 + x;
                    Xt[jb][ib] = mfma(sm.sgy[tt][16 * jb + lm], qc[x], Xt[jb][ib]);
                    Xt[jb][ib] = mfma(sm.du[tt][16 * jb + lm], kc[x], Xt[jb][ib]);
                }
        }
        // dg at the block's first token: column sums of X .* Mb (X now the gradient before it)
        float dg0[2];
        colsum_xm(Mb, dg0);
        // dk = P3 / c + c P2; dg increments q.*dq - k.*(G^T delta - Mp^T du)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i = c0 + 16 * ib + lm;
            const f4 cv = ld4(&cc[16 * ib + lm][4 * g4]), kr = KR(ib), kc = KC(ib);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * g4 + r;
                const float c = cv[r], rc = rcp(c);
                const float dk = fmaf(rc, p3[ib][r], c * p2[ib][r]);
                float g = inc[ib][r] + fmaf(-kr[r], p3[ib][r], kc[r] * p2[ib][r]);
                if (tt == 0) g = dg0[ib];
                if (tt < n) {
                    bst(rpo, dk, (S + i) * 4 + tt * pt, 0);
                    if (kda) bst(rpo, g, (2 * S + i) * 4 + tt * pt, 0);
                }
                gsum[r] += g;
            }
        }
        if (!kda) {   // scalar gate: the wave's column sum per token
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gs = row16_sum(gsum[r]);
                const int tt = 4 * g4 + r;
                if (lm == 0 && tt < n) bst(rpo, gs, (2 * S + wv) * 4 + tt * pt, 0);
            }
        }
        if (dir) scale_cols(Xt, true);   // the gradient before the token's gates
        __syncthreads();   // row data and scratch are free for the next staging
    };

    // a whole block from Mr at its start to its end (token by token if flagged)
    auto replay_block = [&](f4 (&Mr)[2][2], int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        const float *wm = a.wmat + bi * MATF;
        const bool dir = a.wflag[bi] != 0;
        const int steps = dir ? cnt : 1;
        for (int k = 0; k < steps; ++k) {
            stage(dir ? t0 + k : t0, dir ? 1 : cnt, dir, k, wm);
            replay(Mr, dir);
            __syncthreads();
        }
    };
    // walk a whole block with start state M (token by token if flagged: each token's start
    // replayed from M)
    auto walk_block = [&](f4 (&M)[2][2], int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        const float *wm = a.wmat + bi * MATF;
        if (a.wflag[bi] == 0) {
            stage(t0, cnt, false, 0, wm);
            walk(M, t0, cnt, false);
            return;
        }
        for (int k = cnt - 1; k >= 0; --k) {
            f4 Mr[2][2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) Mr[jb][ib] = M[jb][ib];
            for (int sx = 0; sx < k; ++sx) {
                stage(t0 + sx, 1, true, sx, wm);
                replay(Mr, true);
                __syncthreads();
            }
            stage(t0 + k, 1, true, k, wm);
            scale_cols(Mr, true);
            walk(Mr, t0 + k, 1, true);
        }
    };

    const float *snapu = a.snap + unit * a.n_ck_max * S * S + (int64_t)r0 * S;
    float *vsb = a.vsbuf + ((unit * NQ + qb) * (int64_t)a.nvs_max) * (QR * S);
    const int nbk = (L + W - 1) / W;
    for (int b = nbk - 1; b >= 0; --b) {
        const int t0 = b * W, sg = t0 / C, ts = sg * C, te = min(ts + C, L);
        const int nvs = (te - ts + VS - 1) / VS;
        if (nvs > 1 && t0 + W >= te) {   // the segment's last block: its stretch starts first
            f4 M[2][2];
            load_state(snapu + (int64_t)sg * S * S, M);
            for (int t = ts; t < ts + (nvs - 1) * VS; t += W) {
                replay_block(M, t);
                if ((t + W - ts) % VS == 0) save_state(vsb + (int64_t)((t + W - ts) / VS) * (QR * S), M);
            }
        }
        const int vi = (t0 - ts) / VS, va = ts + vi * VS;
        f4 M[2][2];
        load_state(vi == 0 ? snapu + (int64_t)sg * S * S : vsb + (int64_t)vi * (QR * S), M);
        if (t0 != va) replay_block(M, va);
        if (b == nbk - 1) {   // final state: the start of the dg recursion after the last token
            f4 Mf[2][2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) Mf[jb][ib] = M[jb][ib];
            replay_block(Mf, t0);
            float hf[2];
            colsum_xm(Mf, hf);
            float *hp = a.hfin + (unit * NQ + qb) * (int64_t)S;
            if (kda) {
                if (g4 == 0) {
                    hp[c0 + lm] = hf[0];
                    hp[c0 + 16 + lm] = hf[1];
                }
            } else {
                const float hs = row16_sum(hf[0] + hf[1]);
                if (lane == 0) hp[wv] = hs;
            }
        }
        walk_block(M, t0);
    }
    save_state(a.dstate + unit * S * S + (int64_t)r0 * S, Xt);   // the gradient before token 0
    for (int64_t idx = tid; idx < (int64_t)(a.T - L) * QR; idx += 256) {
        const int64_t t = L + idx / QR;
        dvout[t * (a.H_v * S) + idx % QR] = 0.f;
    }
}

// ------------------------------------------------------------------ quarter / head sums

// dq, dk: sums over the quarters and the value heads of each key head (increasing order);
// dbeta: sum of the eight row-block partials; dg: per block, from its last token down, the
// next block's first-token value (after the sequence's last token: the final column sums)
// plus the quarters' increments, and at the block's first token the quarters' direct
// values.  A block processed token by token has every token as a first token.  The scalar
// gate sums the columns (the backward left per-wave sums in the first four slots).
template <int V>
__global__ void __launch_bounds__(256) combine_mf_kernel(const Mf128Args a) {
    const int64_t T = a.T, n = a.n_seqs_launch, Hk = a.H_k, Hv = a.H_v;
    const bool kda = a.kda != 0;
    const int64_t G = kda ? S : 1;
    const int64_t VG = kda ? V : 1;
    const int64_t nblk = (T + W - 1) / W;
    const int64_t n_qk = n * T * Hk * (S / V);
    const int64_t n_g = n * nblk * Hv * (G / VG);
    const int64_t n_b = n * T * Hv;
    const int64_t total = n_qk + n_g + n_b;
    const int64_t seq0 = a.s_base;
    auto ldv = [](const float *p, float (&x)[V]) {
        if constexpr (V == 4) {
            const f4 t = ld4(p);
            x[0] = t[0]; x[1] = t[1]; x[2] = t[2]; x[3] = t[3];
        } else {
            x[0] = *p;
        }
    };
    auto stv = [](float *p, const float (&x)[V]) {
        if constexpr (V == 4) st4(p, f4{x[0], x[1], x[2], x[3]});
        else *p = x[0];
    };
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
                for (int h = kh; h < Hv; h += (int)Hk) {
                    const float *pp = a.part + ((((seq0 + sl) * T + t) * Hv + h) * NQ) * (3 * S) + i;
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        float x[V], y[V];
                        ldv(pp + (qb * 3 + 0) * S, x);
                        ldv(pp + (qb * 3 + 1) * S, y);
#pragma unroll
                        for (int c = 0; c < V; ++c) q[c] += x[c], k[c] += y[c];
                    }
                }
            }
            const int64_t o = (((seq0 + sl) * T + t) * Hk + kh) * S + i;
            stv(a.dq + o, q);
            stv(a.dk + o, k);
        } else if (idx < n_qk + n_g) {
            const int64_t j = idx - n_qk;
            const int i = (int)(j % (G / VG)) * (int)VG;
            int64_t rest = j / (G / VG);
            const int h = (int)(rest % Hv);
            rest /= Hv;
            const int m = (int)(rest % nblk);
            const int sl = (int)(rest / nblk);
            const int t0 = m * W, L = a.lens[sl];
            const int cnt = max(0, min(W, L - t0));
            const bool dir = cnt > 0 && a.wflag[(((seq0 + sl) * nblk + m) * Hv + h)] != 0;
            auto part_sum = [&](int t, float (&g)[V]) {
                const int64_t rt = (((seq0 + sl) * T + t) * Hv + h) * NQ;
#pragma unroll
                for (int c = 0; c < V; ++c) g[c] = 0.f;
#pragma unroll
                for (int qb = 0; qb < NQ; ++qb) {
                    const float *pp = a.part + (rt + qb) * (3 * S) + 2 * S;
                    if (kda) {
                        float x[V];
                        ldv(pp + i, x);
#pragma unroll
                        for (int c = 0; c < V; ++c) g[c] += x[c];
                    } else {
#pragma unroll
                        for (int w2 = 0; w2 < 4; ++w2) g[0] += pp[w2];
                    }
                }
            };
            float carry[V];
#pragma unroll
            for (int c = 0; c < V; ++c) carry[c] = 0.f;
            if (cnt > 0) {
                if (t0 + W < L) {
                    part_sum(t0 + W, carry);
                } else {
                    const float *hf = a.hfin + ((seq0 + sl) * Hv + h) * NQ * S;
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        if (kda) {
                            float x[V];
                            ldv(hf + qb * S + i, x);
#pragma unroll
                            for (int c = 0; c < V; ++c) carry[c] += x[c];
                        } else {
#pragma unroll
                            for (int w2 = 0; w2 < 4; ++w2) carry[0] += hf[qb * S + w2];
                        }
                    }
                }
            }
            for (int tt = W - 1; tt >= 0; --tt) {
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
                        if (tt == 0 || dir) {
                            g[c] = p[c];
                            carry[c] = p[c];
                        } else {
                            carry[c] += p[c];
                            g[c] = carry[c];
                        }
                    }
                }
                float *dst = a.dg + (((seq0 + sl) * T + t) * Hv + h) * G + i;
                if (kda) stv(dst, g);
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
                const float *pp = a.pbuf + (((seq0 + sl) * T + t) * Hv + h) * (2 * NQ);
#pragma unroll
                for (int x = 0; x < 2 * NQ; ++x) b += pp[x];
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

template <template <int> class K>
const void *pick(int dt) {
    return dt == GDN_DTYPE_BF16 ? (const void *)K<GDN_DTYPE_BF16>::fn
           : dt == GDN_DTYPE_F16 ? (const void *)K<GDN_DTYPE_F16>::fn
                                 : (const void *)K<GDN_DTYPE_F32>::fn;
}
template <int DT>
struct PrepK {
    static constexpr auto fn = prep128_kernel<DT>;
};
template <int DT>
struct FwdK {
    static constexpr auto fn = fwd_mf_kernel<DT>;
};
template <int DT>
struct BwdK {
    static constexpr auto fn = bwd_mf_kernel<DT>;
};

}  // namespace

int mf128_stretch_tokens() { return VS; }

hipError_t launch_prep128(const Mf128Args &a, hipStream_t st) {
    const int64_t items = (int64_t)a.n_seqs_launch * ((a.T + W - 1) / W) * a.H_v;
    if (items <= 0) return hipSuccess;
    const int blocks = (int)std::min<int64_t>(items, 16384);
    return launch(pick<PrepK>(a.dtype), a, blocks, 64, st);
}

hipError_t launch_fwd_mf(const Mf128Args &a, hipStream_t st) {
    return launch(pick<FwdK>(a.dtype), a, a.n_seqs_launch * a.H_v * NQ, 128, st);
}

hipError_t launch_bwd_mf(const Mf128Args &a, hipStream_t st) {
    return launch(pick<BwdK>(a.dtype), a, a.n_seqs_launch * a.H_v * NQ, 256, st);
}

hipError_t launch_combine_mf(const Mf128Args &a, hipStream_t st) {
    auto a16 = [](const void *p) { return p == nullptr || ((uintptr_t)p & 15) == 0; };
    const bool vec = a16(a.part) && a16(a.hfin) && a16(a.dq) && a16(a.dk) && a16(a.dg);
    const int64_t V = vec ? 4 : 1, VG = a.kda ? V : 1, G = a.kda ? S : 1;
    const int64_t total = (int64_t)a.n_seqs_launch *
                          (a.T * (a.H_k * (S / V) + a.H_v) + (int64_t)((a.T + W - 1) / W) * a.H_v * (G / VG));
    if (total <= 0) return hipSuccess;
    const int blocks = (int)std::min<int64_t>((total + 255) / 256, 16384);
    return vec ? launch((const void *)combine_mf_kernel<4>, a, blocks, 256, st)
               : launch((const void *)combine_mf_kernel<1>, a, blocks, 256, st);
}

}  // namespace gdn
