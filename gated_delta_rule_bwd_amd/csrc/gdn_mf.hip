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
// One workgroup owns a unit.  Rows of M evolve independently in both directions ("metal:
// GATED_DELTA_NET_BACK", approval review: each row of the state is updated on its own), so the
// forward gives each of its eight waves 16 rows, and the backward's chain (dd = dM k and the
// update of dM) does the same; the backward's column sums (dq, dk, dg) take the columns of the
// state and of the transposed gradient instead, 16 per wave, so they are complete inside the
// workgroup.  Only dq and dk of key heads shared by several value heads are summed afterwards,
// over those value heads in increasing order.
//
// MFMA lane layout (16x16x4 f32): lane l supplies A[l%16][kappa] and B[kappa][l%16], and
// holds D[4(l/16) + r][l%16] in accumulator register r.  Every product below uses the
// contraction index kappa = 4(l/16) + s in its step s (within each block of 16), so a
// D-layout accumulator is directly the B operand of the next product.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int S = 128;
constexpr int W = 16;          // tokens per block
constexpr float kLo = 0x1p-60f, kHi = 0x1p60f;
constexpr int SP = S + 4;      // [token][column] LDS rows
constexpr int KP = W + 4;      // [column][token] LDS rows
constexpr int MATF = 3 * W * W;   // floats of block matrices: Bm, Te, Tb

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ void st4(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int as_i(float x) { return __builtin_bit_cast(int, x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), CTRL, 0xF, 0xF, true));
}
// the value of lane l - D in the same 16-lane row, 1 for the first D lanes of the row
template <int D>
__device__ __forceinline__ float row_shr(float v) {
    return as_f(__builtin_amdgcn_update_dpp(as_i(1.f), as_i(v), 0x110 + D, 0xF, 0xF, false));
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
// four consecutive elements (16 bytes of fp32 or 8 of a half type, aligned to that size)
template <int DT>
__device__ __forceinline__ f4 bld4(Rsrc r, uint32_t vbytes) {
    if constexpr (DT == GDN_DTYPE_F32) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, vbytes, 0, 0);
        return f4{as_f((int)v[0]), as_f((int)v[1]), as_f((int)v[2]), as_f((int)v[3])};
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vbytes, 0, 0);
        f4 o;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const unsigned short hb = (unsigned short)((x & 1) ? (v[x >> 1] >> 16) : (v[x >> 1] & 0xffffu));
            if constexpr (DT == GDN_DTYPE_BF16) o[x] = __builtin_bit_cast(float, (uint32_t)hb << 16);
            else o[x] = (float)__builtin_bit_cast(_Float16, hb);
        }
        return o;
    }
}
// A wave-uniform 32-bit value read through the constant address space, so it takes a scalar
// load (its wait does not drain the vector memory counter).  Only for data no kernel of the
// same launch writes.
__device__ __forceinline__ int32_t sload(const int32_t *p, int64_t i) {
    typedef const __attribute__((address_space(4))) int32_t *cptr;
    return ((cptr)(uintptr_t)p)[i];
}
template <int DT>
__device__ __forceinline__ const In<DT> *tin(const void *p) {
    return reinterpret_cast<const In<DT> *>(p);
}

// ------------------------------------------------------------------ block preparation

// Per block of every (sequence, value head): the running gate products c (written to cbuf for
// every token of the block), the flag of a block processed token by token (its cbuf rows then
// hold the gates a themselves), and the block matrices Bm (upper triangle of B with its
// diagonal), Te = (I + diag(beta) A)^-1 and Tb = (I + A diag(beta))^-1, A the strict upper
// triangle of the Gram A; a token-by-token block gets Bm = diag(k_t . q_t) and Te = Tb = I.
//
// One wave per block: lane l takes token l%16 and the columns 16 kb + 4(l/16) + x (kb < 8,
// x < 4).  c is a product scan over the 16 lanes of a row (the tokens of the block); the Grams
// are dense products of the lanes' own values (lane l supplies row l%16 of the left operand and
// column l%16 of the right one); the inverses of the unit triangular matrices use the
// nilpotent product form (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), N^16 = 0.
constexpr int PW = 4;   // waves (blocks) per workgroup of the preparation

// Z = X Y for 16 x 16 matrices held in the D layout, given X^T and Y
__device__ __forceinline__ f4 mm16(const f4 &xt, const f4 &y) {
    f4 z = zero4();
#pragma unroll
    for (int x = 0; x < 4; ++x) z = mfma(xt[x], y[x], z);
    return z;
}

template <int DT>
__global__ void __launch_bounds__(64 * PW) prep128_kernel(const Mf128Args a) {
    __shared__ float trs[PW][W][W + 1];   // per-wave transposes
    constexpr uint32_t ES = sizeof(In<DT>);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, lm = lane & 15, g4 = lane >> 4;
    float (*tr)[W + 1] = trs[wv];
    const int nblk = (a.T + W - 1) / W;
    const int G = a.kda ? S : 1;
    const bool kda = a.kda != 0;
    const int64_t items = (int64_t)a.n_seqs_launch * nblk * a.H_v;
    // rows whose starts are all aligned to four elements take vector loads
    auto aligned_rows = [&](const void *p, const gdn_strides &st) {
        return (((uintptr_t)p & (4 * ES - 1)) == 0) && st.seq % 4 == 0 && st.tok % 4 == 0 && st.head % 4 == 0;
    };
    const bool vec_g = aligned_rows(a.g, a.sg), vec_k = aligned_rows(a.k, a.sk), vec_q = aligned_rows(a.q, a.sq);
    // the transpose of a D-layout matrix, in the D layout: every lane's writes reach the LDS
    // before any lane reads (the wave barrier keeps the compiler from interleaving them; one
    // wave's LDS accesses complete in order)
    auto transpose = [&](const f4 &z) {
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < 4; ++r) tr[4 * g4 + r][lm] = z[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = tr[lm][4 * g4 + r];
        __builtin_amdgcn_wave_barrier();
        return o;
    };
    f4 eye;
#pragma unroll
    for (int r = 0; r < 4; ++r) eye[r] = 4 * g4 + r == lm ? 1.f : 0.f;
    // (I + N)^-1 for a strictly upper triangular N (D layout) and its transpose NT
    auto inverse = [&](const f4 &N, const f4 &NT) {
        const f4 n2 = mm16(NT, N), n2t = mm16(N, NT);
        const f4 n4 = mm16(n2t, n2), n4t = mm16(n2, n2t);
        const f4 n8 = mm16(n4t, n4);
        const f4 r1 = (eye - N) + mm16(eye - NT, n2), r1t = (eye - NT) + mm16(n2, eye - NT);
        const f4 r2 = r1 + mm16(r1t, n4), r2t = r1t + mm16(n4, r1t);
        return r2 + mm16(r2t, n8);
    };

    for (int64_t it = (int64_t)blockIdx.x * PW + wv; it < items; it += (int64_t)gridDim.x * PW) {
        const int h = (int)(it % a.H_v);
        const int64_t rest = it / a.H_v;
        const int b = (int)(rest % nblk), sl = (int)(rest / nblk);
        const int t0 = b * W, cnt = min(W, a.lens[sl] - t0);
        if (cnt <= 0) continue;
        const int64_t s = a.s_base + sl;
        const int hk = h % a.H_k;
        const bool ok = lm < cnt;
        const uint32_t tok = ok ? (uint32_t)lm : 0u;
        const Rsrc rg = rsrc(tin<DT>(a.g) + s * a.sg.seq + (int64_t)t0 * a.sg.tok + h * a.sg.head);
        const Rsrc rk = rsrc(tin<DT>(a.k) + s * a.sk.seq + (int64_t)t0 * a.sk.tok + hk * a.sk.head);
        const Rsrc rq = rsrc(tin<DT>(a.q) + s * a.sq.seq + (int64_t)t0 * a.sq.tok + hk * a.sq.head);
        const Rsrc rb = rsrc(tin<DT>(a.beta) + s * a.sb.seq + (int64_t)t0 * a.sb.tok + h * a.sb.head);
        const uint32_t gto = tok * (uint32_t)a.sg.tok * ES, kto = tok * (uint32_t)a.sk.tok * ES,
                       qto = tok * (uint32_t)a.sq.tok * ES;
        // the gates of token l%16 (column 16 (n / 4) + 4(l/16) + n % 4), and their running products
        // over the block's tokens
        auto column = [&](int n) { return (uint32_t)(16 * (n >> 2) + 4 * g4 + (n & 3)); };
        // four consecutive columns 16 kb + 4(l/16) .. of a row (vector loads when aligned)
        auto row4 = [&](Rsrc r, uint32_t rowb, bool vec, int kb) {
            const uint32_t o = rowb + (uint32_t)(16 * kb + 4 * g4) * ES;
            if (vec) return bld4<DT>(r, o);
            return f4{bld<DT>(r, o, 0), bld<DT>(r, o + ES, 0), bld<DT>(r, o + 2 * ES, 0), bld<DT>(r, o + 3 * ES, 0)};
        };
        auto gate = [&](int n) { return ok ? expf(bld<DT>(rg, gto + (kda ? column(n) : 0u) * ES, 0)) : 1.f; };
        float c[32];
        if (kda) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const f4 gv = ok ? row4(rg, gto, vec_g, kb) : zero4();
#pragma unroll
                for (int x = 0; x < 4; ++x) c[4 * kb + x] = ok ? expf(gv[x]) : 1.f;
            }
        } else {
            c[0] = gate(0);
        }
        const int nsc = kda ? 32 : 1;   // distinct columns of the scan
#pragma unroll
        for (int n = 0; n < 32; ++n) {   // lane l%16 takes the products with lanes l%16 - 1, - 2, - 4, - 8
            if (n < nsc) {
                c[n] *= row_shr<1>(c[n]);
                c[n] *= row_shr<2>(c[n]);
                c[n] *= row_shr<4>(c[n]);
                c[n] *= row_shr<8>(c[n]);
            }
        }
        if (!kda) {
#pragma unroll
            for (int n = 1; n < 32; ++n) c[n] = c[0];
        }
        bool bad = false;
#pragma unroll
        for (int n = 0; n < 32; ++n) bad = bad || (ok && !(c[n] >= kLo && c[n] <= kHi));
        const bool direct = __ballot(bad) != 0;
        {   // the running products (a token-by-token block: the gates) for the forward and backward
            float *cb = a.cbuf + ((s * a.T + t0 + tok) * a.H_v + h) * (int64_t)G;
            if (ok) {
                if (kda) {
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) {
                        const int n = 4 * kb;
                        st4(cb + 16 * kb + 4 * g4, direct ? f4{gate(n), gate(n + 1), gate(n + 2), gate(n + 3)}
                                                          : f4{c[n], c[n + 1], c[n + 2], c[n + 3]});
                    }
                } else if (g4 == 0) {
                    cb[0] = direct ? gate(0) : c[0];
                }
            }
        }
        // Grams GA[s][t] = kr_s . kc_t and GB[s][t] = kr_s . qc_t (D layout: s = 4(l/16) + r, t = l%16)
        f4 ga0 = zero4(), ga1 = zero4(), gb0 = zero4(), gb1 = zero4();
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const f4 k4 = ok ? row4(rk, kto, vec_k, kb) : zero4(), q4 = ok ? row4(rq, qto, vec_q, kb) : zero4();
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float cv = direct ? 1.f : c[4 * kb + x];
                const float kr = k4[x] * rcp(cv), kc = k4[x] * cv, qc = q4[x] * cv;
                if (kb & 1) {
                    ga1 = mfma(kr, kc, ga1);
                    gb1 = mfma(kr, qc, gb1);
                } else {
                    ga0 = mfma(kr, kc, ga0);
                    gb0 = mfma(kr, qc, gb0);
                }
            }
        }
        const f4 gA = ga0 + ga1, gB = gb0 + gb1;
        float bs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tt = 4 * g4 + r;
            bs[r] = tt < cnt ? bld<DT>(rb, tt * (uint32_t)a.sb.tok * ES, 0) : 0.f;
        }
        const float bl = ok ? bld<DT>(rb, lm * (uint32_t)a.sb.tok * ES, 0) : 0.f;
        f4 bm, ne, nb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int sg = 4 * g4 + r;
            const float as = (!direct && sg < lm) ? gA[r] : 0.f;
            bm[r] = direct ? (sg == lm ? gB[r] : 0.f) : (sg <= lm ? gB[r] : 0.f);
            ne[r] = bs[r] * as;   // diag(beta) A
            nb[r] = as * bl;      // A diag(beta)
        }
        const f4 te = inverse(ne, transpose(ne)), tb = inverse(nb, transpose(nb));
        float *wm = a.wmat + ((s * nblk + b) * a.H_v + h) * (int64_t)MATF;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = (4 * g4 + r) * W + lm;
            wm[o] = bm[r];
            wm[W * W + o] = direct ? eye[r] : te[r];
            wm[2 * W * W + o] = direct ? eye[r] : tb[r];
        }
        if (lane == 0) a.wflag[(s * nblk + b) * a.H_v + h] = direct ? 1 : 0;
    }
}

// ------------------------------------------------------------------ forward scan

constexpr int NW = 8;          // waves per workgroup, 16 rows each
constexpr int NT = 64 * NW;    // threads per workgroup

// A workgroup owns a unit (sequence, value head).  Wave w holds rows 16 w .. 16 w + 15 of the
// state transposed as eight 16 x 16 tiles: tile ib, lane l, register r holds
// M[16 w + l%16][16 ib + 4(l/16) + r].  Thread tid stages column tid % 128 of tokens
// 4 (tid / 128) .. + 3 of a block; the next block's inputs are loaded into registers while the
// current block is computed.
struct alignas(16) FwdLds {
    float kc[W][SP], qc[W][SP];   // c.*k, c.*q   [token][column]
    float kr[S][KP];              // k./c         [column][token]
    float pv[S];                  // block product per column (a token's gates)
};

template <int DT>
__global__ void __launch_bounds__(NT) fwd_mf_kernel(const Mf128Args a) {
    __shared__ FwdLds smb[2];   // staged blocks, alternately (one barrier per block)
    constexpr uint32_t ES = sizeof(In<DT>);
    const int ul = blockIdx.x;
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int j0 = wv * 16;
    const int ci = tid & (S - 1), tg = __builtin_amdgcn_readfirstlane(tid >> 7);   // staging: column ci, tokens 4 tg .. 4 tg + 3
    const int nblk = (a.T + W - 1) / W;
    const int G = a.kda ? S : 1;
    const bool vec_state = (((uintptr_t)a.state0 | (uintptr_t)a.state_out) & 15) == 0;
    const float *cin = a.cbuf + (s * a.T * a.H_v + h) * (int64_t)G;
    const In<DT> *kin = tin<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qin = tin<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const In<DT> *vin = tin<DT>(a.v) + s * a.sv.seq + h * a.sv.head;
    const In<DT> *bin = tin<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
    float *yout = a.y ? a.y + s * a.sy.seq + h * a.sy.head : nullptr;
    float *eout = a.ebuf + (s * a.T * a.H_v + h) * S;
    const uint32_t ct = (uint32_t)(a.H_v * G) * 4, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES,
                   vt = (uint32_t)a.sv.tok * ES, bt = (uint32_t)a.sb.tok * ES, yt = (uint32_t)a.sy.tok * 4,
                   et = (uint32_t)(a.H_v * S) * 4;
    const uint32_t ccol = (a.kda ? (uint32_t)ci : 0u) * 4;

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

    // inputs of one block: column ci of c, k, q at tokens 4 tg .. + 3; per lane v and beta at
    // (token 4(l/16) + r, row 16 w + l%16) and the operands of Te^T and Bm^T
    struct Pre {
        float c[4], k[4], q[4];
        float v[4], b[4], te[4], bm[4];
        int dir;
    };
    auto prefetch = [&](Pre &P, int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        P.dir = sload(a.wflag, bi);
        const Rsrc rc = rsrc(cin + (int64_t)t0 * (a.H_v * G)), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                   rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rv = rsrc(vin + (int64_t)t0 * a.sv.tok),
                   rb = rsrc(bin + (int64_t)t0 * a.sb.tok), rw = rsrc(a.wmat + bi * MATF);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t tt = 4 * tg + x;
            const bool ok = (int)tt < cnt;
            P.c[x] = ok ? bldf(rc, ccol, tt * ct) : 1.f;
            P.k[x] = ok ? bld<DT>(rk, ci * ES, tt * kt) : 0.f;
            P.q[x] = ok ? bld<DT>(rq, ci * ES, tt * qt) : 0.f;
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
    auto block = [&](const FwdLds &sm, int tw, int n, const float (&vv)[4], const float (&bb)[4],
                     const float (&teA)[4], const float (&bmA)[4]) {
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
    auto scale_state = [&](const FwdLds &sm) {
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) M[ib] *= ld4(&sm.pv[16 * ib + 4 * g4]);
    };

    // Each staging fills the buffer the previous block did not use; every wave left that buffer
    // before the barrier that followed the previous staging, so one barrier per block (per token
    // of a token-by-token block) orders the writes and the reads.
    Pre P;
    int cur = 0;
    if (L > 0) prefetch(P, 0);
    for (int b = 0; b * W < L; ++b) {
        const int t0 = b * W, cnt = min(W, L - t0);
        if (t0 % a.C == 0) store_state(snap + (int64_t)(t0 / a.C) * S * S);
        if (!P.dir) {
            FwdLds &sm = smb[cur];
            float krow[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int tt = 4 * tg + x;
                const float c = P.c[x];
                krow[x] = P.k[x] * rcp(c);
                sm.kc[tt][ci] = P.k[x] * c;
                sm.qc[tt][ci] = P.q[x] * c;
                if (tt == cnt - 1) sm.pv[ci] = c;
            }
            st4(&sm.kr[ci][4 * tg], f4{krow[0], krow[1], krow[2], krow[3]});
            const float vv[4] = {P.v[0], P.v[1], P.v[2], P.v[3]}, bb[4] = {P.b[0], P.b[1], P.b[2], P.b[3]};
            const float teA[4] = {P.te[0], P.te[1], P.te[2], P.te[3]}, bmA[4] = {P.bm[0], P.bm[1], P.bm[2], P.bm[3]};
            __syncthreads();
            if (t0 + W < L) prefetch(P, t0 + W);   // the registers are free again
            block(sm, t0, cnt, vv, bb, teA, bmA);
            scale_state(sm);
            cur ^= 1;
        } else {   // token by token: each token a one-token block after its gates scale the state
            const int64_t bi = (s * nblk + b) * a.H_v + h;
            const float *wm = a.wmat + bi * MATF;
            const Rsrc rc = rsrc(cin + (int64_t)t0 * (a.H_v * G)), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                       rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rv = rsrc(vin + (int64_t)t0 * a.sv.tok),
                       rb = rsrc(bin + (int64_t)t0 * a.sb.tok);
            for (int tau = 0; tau < cnt; ++tau) {
                FwdLds &sm = smb[cur];
                const float av = bldf(rc, ccol + tau * ct, 0);
                const float kx = bld<DT>(rk, ci * ES + tau * kt, 0);
                const float qx = bld<DT>(rq, ci * ES + tau * qt, 0);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int tt = 4 * tg + x;
                    sm.kc[tt][ci] = tt == 0 ? kx : 0.f;
                    sm.qc[tt][ci] = tt == 0 ? qx : 0.f;
                }
                st4(&sm.kr[ci][4 * tg], f4{tg == 0 ? kx : 0.f, 0.f, 0.f, 0.f});
                if (tg == 0) sm.pv[ci] = av;
                float vv[4], bb[4], teA[4], bmA[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = 4 * g4 + r;
                    vv[r] = tt == 0 ? bld<DT>(rv, (j0 + lm) * ES + tau * vt, 0) : 0.f;
                    bb[r] = tt == 0 ? bld<DT>(rb, tau * bt, 0) : 0.f;
                    teA[r] = tt == lm ? 1.f : 0.f;
                    bmA[r] = (tt == 0 && lm == 0) ? wm[tau * (W + 1)] : 0.f;
                }
                __syncthreads();
                scale_state(sm);
                block(sm, t0 + tau, 1, vv, bb, teA, bmA);
                cur ^= 1;
            }
            if (t0 + W < L) prefetch(P, t0 + W);
        }
    }
    if (yout) {
        for (int64_t idx = tid; idx < (int64_t)(a.T - L) * S; idx += NT) {
            const int64_t t = L + idx / S;
            yout[t * a.sy.tok + (int)(idx % S)] = 0.f;
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

// The Gram G1[s][t] = delta_s . (scale gy_t) over the 128 rows of every block of every unit
// (it needs only the forward's errors and the cotangent).  One wave per block; a block processed
// token by token keeps its diagonal (the one-token Grams).
template <int DT>
__global__ void __launch_bounds__(64) gram1_kernel(const Mf128Args a) {
    constexpr uint32_t ES = sizeof(In<DT>);
    const int lane = threadIdx.x, lm = lane & 15, g4 = lane >> 4;
    const int nblk = (a.T + W - 1) / W;
    const int64_t items = (int64_t)a.n_seqs_launch * nblk * a.H_v;
    const uint32_t gyt = (uint32_t)a.sgy.tok * ES;
    const bool vec_gy = (((uintptr_t)a.gy & (4 * ES - 1)) == 0) && a.sgy.seq % 4 == 0 && a.sgy.tok % 4 == 0 &&
                        a.sgy.head % 4 == 0;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int h = (int)(it % a.H_v);
        const int64_t rest = it / a.H_v;
        const int b = (int)(rest % nblk), sl = (int)(rest / nblk);
        const int t0 = b * W, cnt = min(W, a.lens[sl] - t0);
        if (cnt <= 0) continue;
        const int64_t s = a.s_base + sl;
        const bool ok = lm < cnt;
        const float *er = a.ebuf + ((s * a.T + t0 + (ok ? lm : 0)) * a.H_v + h) * S;
        const Rsrc rgy = rsrc(tin<DT>(a.gy) + s * a.sgy.seq + (int64_t)t0 * a.sgy.tok + h * a.sgy.head);
        const Rsrc rb = rsrc(tin<DT>(a.beta) + s * a.sb.seq + (int64_t)t0 * a.sb.tok + h * a.sb.head);
        const float bl = ok ? bld<DT>(rb, lm * (uint32_t)a.sb.tok * ES, 0) : 0.f;
        // A = delta^T (row s = l%16, rows j along the contraction), B = scale gy (column t = l%16)
        f4 g0 = zero4(), g1 = zero4();
#pragma unroll
        for (int kb = 0; kb < S / 16; ++kb) {
            const int j = 16 * kb + 4 * g4;
            const f4 e4 = ok ? ld4(er + j) : zero4();
            f4 y4 = zero4();
            if (ok) {
                const uint32_t o = j * ES + lm * gyt;
                y4 = vec_gy ? bld4<DT>(rgy, o)
                            : f4{bld<DT>(rgy, o, 0), bld<DT>(rgy, o + ES, 0), bld<DT>(rgy, o + 2 * ES, 0),
                                 bld<DT>(rgy, o + 3 * ES, 0)};
                y4 *= a.scale;
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if (kb % 2 == 0) g0 = mfma(bl * e4[x], y4[x], g0);
                else g1 = mfma(bl * e4[x], y4[x], g1);
            }
        }
        const f4 gsum = g0 + g1;
        float *dst = a.g1buf + ((s * nblk + b) * a.H_v + h) * (int64_t)(W * W);
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * g4 + r) * W + lm] = gsum[r];
    }
}

// A workgroup owns a unit.  Two layouts of the 128 x 128 matrices:
//  - rows, for the chain dd = dM k and the update of dM: wave w holds rows 16 w .. 16 w + 15 of
//    the gradient X = dM diag(c) transposed as eight tiles (tile ib, lane l, register r:
//    X[16 w + l%16][16 ib + 4(l/16) + r]);
//  - columns, for the column sums (dq, dk, dg) and the state replay: wave w holds columns
//    16 w .. 16 w + 15 of the state M as eight tiles (tile jb, lane l, register r:
//    M[16 jb + 4(l/16) + r][16 w + l%16]).
// The gradient reaches the column layout through a transpose in LDS once per block.  Column
// results are tiles P[i][t] (lane l, register r: column 16 w + 4(l/16) + r, token l%16).
//
// Per segment of C tokens the backward runs a fixed sequence of steps: replays of the segment's
// blocks from its snapshot, each leaving the next block's start state in the workspace; for the
// sequence's last segment, a replay of its last block (the final state, which starts the dg
// recursion); then walks of the blocks from the last, each from its saved start state.  The
// inputs of each step are loaded into registers during the previous step.
constexpr int GP = W + 4;   // row pitch of the per-wave 16 x 16 partials

struct alignas(16) BwdLds {
    float krT[W][SP];          // k./c        [token][column]
    float krI[S][KP];          // k./c        [column][token]
    float qcI[S][KP];          // c.*q        [column][token]
    float kcI[S][KP];          // c.*k        [column][token]
    float sgy[W][SP];          // scale gy    [token][row]; with ee, in replays: delta
    float ee[W][SP];           // delta = beta e  [token][row]
    float du[W][SP];           // e, then du  [token][row]
    float xt[S][SP];           // X after the fold [column][row]; in replays: the state
    float pv[S];               // fold factor per column (a token's gates)
    float bt[W];               // beta
    float bm[W][W], tb[W][W];  // Bm, Tb
    float g1[W][GP];           // G1 = delta^T scale gy, upper triangle with the diagonal
    float gp[NW][W][GP];       // per-wave partials of G2 = delta^T du, strict upper triangle, [s][t]
    float gpt[NW][W][GP];      // the same, [t][s]
    float pb[NW][W];           // per-wave partials of dbeta
    float gs[NW][W];           // per-wave partial sums of the scalar gate's dg
};

static_assert(2 * W * SP >= S * KP, "a replay's delta fits in sgy and ee");
static_assert(offsetof(BwdLds, ee) == offsetof(BwdLds, sgy) + sizeof(float) * W * SP, "sgy and ee adjacent");
static_assert(S * SP >= 32 * NT, "a replay's state fits in xt");

template <int DT>
__global__ void __launch_bounds__(NT) bwd_mf_kernel(const Mf128Args a) {
    __shared__ BwdLds sm;
    constexpr uint32_t ES = sizeof(In<DT>);
    const int ul = blockIdx.x;
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int C = a.C;
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int j0 = 16 * wv, i0 = 16 * wv;   // rows (row layout) and columns (column layout) of the wave
    const int ci = tid & (S - 1), tg = __builtin_amdgcn_readfirstlane(tid >> 7);   // staging: column/row ci, tokens 4 tg .. 4 tg + 3
    const int nblk = (a.T + W - 1) / W;
    const int G = a.kda ? S : 1;
    const float scale = a.scale;
    const bool kda = a.kda != 0;
    // during replays: the delta [row][token] in the space of sgy and ee, and the state handed from
    // one replay step to the next in the space of xt (each lane reads back only what it wrote)
    float (*dl)[KP] = reinterpret_cast<float (*)[KP]>(&sm.sgy[0][0]);
    float *lst = &sm.xt[0][0];
    // bases of this (sequence, head) and byte strides per token
    const float *cin = a.cbuf + (s * a.T * a.H_v + h) * (int64_t)G;
    const In<DT> *kin = tin<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qin = tin<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const In<DT> *gyin = tin<DT>(a.gy) + s * a.sgy.seq + h * a.sgy.head;
    const In<DT> *bin = tin<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
    const int64_t row0 = s * a.T * a.H_v + h;   // per-token workspace row of token 0; stride H_v
    const float *ein = a.ebuf + row0 * S;
    float *dvout = a.dv + row0 * S;
    float *dqout = (a.dq_part ? a.dq_part : a.dq) + row0 * S;   // direct when H_v == H_k
    float *dkout = (a.dk_part ? a.dk_part : a.dk) + row0 * S;
    float *dgout = a.dg + row0 * G;
    float *dbout = a.dbeta + row0;
    const bool vec_out = (((uintptr_t)dqout | (uintptr_t)dkout | (uintptr_t)dgout) & 15) == 0;
    const uint32_t ct = (uint32_t)(a.H_v * G) * 4, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES,
                   gyt = (uint32_t)a.sgy.tok * ES, bt = (uint32_t)a.sb.tok * ES, et = (uint32_t)a.H_v * S * 4;
    const uint32_t ccol = (kda ? (uint32_t)ci : 0u) * 4;

    // the column layout in memory (row-major [S][S]): one vector offset per lane, the row block
    // and register in the scalar offset
    const uint32_t vcol = ((4 * g4) * S + i0 + lm) * 4;
    auto load_cols = [&](const float *base, f4 (&Mc)[8]) {
        const Rsrc rs = rsrc(base);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Mc[jb][r] = bldf(rs, vcol + r * S * 4, 16 * jb * S * 4);
    };
    auto save_cols = [&](float *base, const f4 (&Mc)[8]) {
        const Rsrc rs = rsrc(base);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) bst(rs, Mc[jb][r], vcol + r * S * 4, 16 * jb * S * 4);
    };

    auto save_lds = [&](const f4 (&Mc)[8]) {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) lst[(4 * jb + r) * NT + tid] = Mc[jb][r];
    };
    auto load_lds = [&](f4 (&Mc)[8]) {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Mc[jb][r] = lst[(4 * jb + r) * NT + tid];
    };

    // the gradient in the row layout
    f4 X[8];
    if (a.dstate_out) {
        const float *p = a.dstate_out + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) X[ib] = f4{p[16 * ib], p[16 * ib + 1], p[16 * ib + 2], p[16 * ib + 3]};
    } else {
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) X[ib] = zero4();
    }
    // the dg recursion's carry per column (tile layout: column i0 + 4(l/16) + r)
    f4 carry = zero4();

    // inputs of a block, loaded one step ahead: column (and row) ci at tokens 4 tg .. + 3 of c,
    // k, q, gy, e and beta; one entry each of Bm, Tb and G1
    struct Pre {
        float c[4], k[4], q[4], gy[4], e[4], b[4];
        float m0, m1, m2;
        int dir;
    };
    auto prefetch = [&](Pre &P, int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        P.dir = sload(a.wflag, bi);
        const Rsrc rc = rsrc(cin + (int64_t)t0 * (a.H_v * G)), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                   rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rgy = rsrc(gyin + (int64_t)t0 * a.sgy.tok),
                   re = rsrc(ein + (int64_t)t0 * (a.H_v * S)), rb = rsrc(bin + (int64_t)t0 * a.sb.tok),
                   rw = rsrc(a.wmat + bi * MATF), rg1 = rsrc(a.g1buf + bi * (W * W));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t tt = 4 * tg + x;
            const bool ok = (int)tt < cnt;
            P.c[x] = ok ? bldf(rc, ccol, tt * ct) : 1.f;
            P.k[x] = ok ? bld<DT>(rk, ci * ES, tt * kt) : 0.f;
            P.q[x] = ok ? bld<DT>(rq, ci * ES, tt * qt) : 0.f;
            P.gy[x] = ok ? bld<DT>(rgy, ci * ES, tt * gyt) : 0.f;
            P.e[x] = ok ? bldf(re, ci * 4, tt * et) : 0.f;
            P.b[x] = ok ? bld<DT>(rb, 0, tt * bt) : 0.f;
        }
        const uint32_t m = tid & 255;
        P.m0 = bldf(rw, m * 4, 0);                  // Bm
        P.m1 = bldf(rw, (2 * W * W + m) * 4, 0);    // Tb
        P.m2 = bldf(rg1, m * 4, 0);                 // G1
    };
    // staging of a column-scaled block for a walk
    auto stage_walk = [&](const Pre &P, int cnt) {
        float kr[4], qc[4], kc[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int tt = 4 * tg + x;
            const float c = P.c[x];
            kr[x] = P.k[x] * rcp(c);
            qc[x] = P.q[x] * c;
            kc[x] = P.k[x] * c;
            sm.krT[tt][ci] = kr[x];
            sm.sgy[tt][ci] = scale * P.gy[x];
            sm.ee[tt][ci] = P.b[x] * P.e[x];   // delta
            sm.du[tt][ci] = P.e[x];            // e, until the walk replaces it by du
            if (tt == cnt - 1) sm.pv[ci] = c;
            if (ci == 0) sm.bt[tt] = P.b[x];
        }
        st4(&sm.krI[ci][4 * tg], f4{kr[0], kr[1], kr[2], kr[3]});
        st4(&sm.qcI[ci][4 * tg], f4{qc[0], qc[1], qc[2], qc[3]});
        st4(&sm.kcI[ci][4 * tg], f4{kc[0], kc[1], kc[2], kc[3]});
        if (tid < 256) {
            (&sm.bm[0][0])[tid] = P.m0;
            (&sm.tb[0][0])[tid] = P.m1;
            sm.g1[tid >> 4][tid & 15] = (tid >> 4) <= (tid & 15) ? P.m2 : 0.f;   // s <= t
        }
        __syncthreads();
    };
    // staging of a column-scaled block for a replay: k./c and delta [row][token]
    auto stage_replay = [&](const Pre &P, int cnt) {
        float kr[4], d[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int tt = 4 * tg + x;
            kr[x] = P.k[x] * rcp(P.c[x]);
            d[x] = P.b[x] * P.e[x];
            if (tt == cnt - 1) sm.pv[ci] = P.c[x];
        }
        st4(&sm.krI[ci][4 * tg], f4{kr[0], kr[1], kr[2], kr[3]});
        st4(&dl[ci][4 * tg], f4{d[0], d[1], d[2], d[3]});
        __syncthreads();
    };
    // staging of token t0 + tau of a token-by-token block (loaded directly) as a one-token block
    // with c = 1, the token's gates in pv
    auto stage_token = [&](int t0, int tau, bool walk) {
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        const Rsrc rc = rsrc(cin + (int64_t)t0 * (a.H_v * G)), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                   rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rgy = rsrc(gyin + (int64_t)t0 * a.sgy.tok),
                   re = rsrc(ein + (int64_t)t0 * (a.H_v * S)), rb = rsrc(bin + (int64_t)t0 * a.sb.tok);
        const float av = bldf(rc, ccol + tau * ct, 0);
        const float kx = bld<DT>(rk, ci * ES + tau * kt, 0);
        const float ex = bldf(re, ci * 4 + tau * et, 0);
        const float bx = bld<DT>(rb, tau * bt, 0);
        const f4 k4 = f4{tg == 0 ? kx : 0.f, 0.f, 0.f, 0.f};
        st4(&sm.krI[ci][4 * tg], k4);
        if (tg == 0) sm.pv[ci] = av;
        if (!walk) {
            st4(&dl[ci][4 * tg], f4{tg == 0 ? bx * ex : 0.f, 0.f, 0.f, 0.f});
        } else {
            const float qx = bld<DT>(rq, ci * ES + tau * qt, 0);
            const float gx = scale * bld<DT>(rgy, ci * ES + tau * gyt, 0);
            st4(&sm.qcI[ci][4 * tg], f4{tg == 0 ? qx : 0.f, 0.f, 0.f, 0.f});
            st4(&sm.kcI[ci][4 * tg], k4);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int tt = 4 * tg + x;
                sm.krT[tt][ci] = tt == 0 ? kx : 0.f;
                sm.sgy[tt][ci] = tt == 0 ? gx : 0.f;
                sm.ee[tt][ci] = tt == 0 ? bx * ex : 0.f;
                sm.du[tt][ci] = tt == 0 ? ex : 0.f;
                if (ci == 0) sm.bt[tt] = tt == 0 ? bx : 0.f;
            }
            if (tid < 256) {
                const int sg = tid >> 4, t2 = tid & 15;
                const float *wm = a.wmat + bi * MATF;
                const float *g1b = a.g1buf + bi * (W * W);
                sm.bm[sg][t2] = (sg == 0 && t2 == 0) ? wm[tau * (W + 1)] : 0.f;
                sm.tb[sg][t2] = sg == t2 ? 1.f : 0.f;
                sm.g1[sg][t2] = (sg == 0 && t2 == 0) ? g1b[tau * (W + 1)] : 0.f;
            }
        }
        __syncthreads();
    };

    // ---- replay of a staged (sub)block in the column layout (dir: the token's gates scale the
    // state first; otherwise the block product folds in at the end)
    auto replay = [&](f4 (&Mr)[8], bool dir) {
        const float p = sm.pv[i0 + lm];
        if (dir) {
#pragma unroll
            for (int jb = 0; jb < 8; ++jb) Mr[jb] *= p;
        }
        const f4 kb = ld4(&sm.krI[i0 + lm][4 * g4]);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
            const f4 d4 = ld4(&dl[16 * jb + lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) Mr[jb] = mfma(d4[x], kb[x], Mr[jb]);
        }
        if (!dir) {
#pragma unroll
            for (int jb = 0; jb < 8; ++jb) Mr[jb] *= p;
        }
    };
    // the column sums of Z .* Mr over all rows for column i0 + l%16, Z in the column layout read
    // from memory (row-major [S][S])
    auto colsum_mem = [&](const float *Z, const f4 (&Mr)[8]) {
        const Rsrc rz = rsrc(Z);
        float v = 0.f;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) v = fmaf(bldf(rz, vcol + r * S * 4, 16 * jb * S * 4), Mr[jb][r], v);
        return rows4_sum(v);
    };
    // a value per column i0 + l%16 into the tile layout (column i0 + 4(l/16) + r)
    auto to_tile = [&](float v) {
        f4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = __shfl(v, 4 * g4 + r);
        return o;
    };

    // ---- walk of a staged (sub)block with start state Mb (column layout); n tokens from tw.
    auto walk = [&](const f4 (&Mb)[8], int tw, int n, bool dir) {
        // ---- phase A.  Chain: X' = X diag(P), its transpose for the column sums, dd0^T = KR X'^T,
        // dd^T = Tb (dd0^T + Bm sgy^T), du = -beta dd, dv and the dbeta partials.
        if (!dir) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) X[ib] *= ld4(&sm.pv[16 * ib + 4 * g4]);
        }
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.xt[16 * ib + 4 * g4 + r][j0 + lm] = X[ib][r];
        f4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int ib = 0; ib < 8; ib += 2) {
            const f4 a0 = ld4(&sm.krT[lm][16 * ib + 4 * g4]), a1 = ld4(&sm.krT[lm][16 * ib + 16 + 4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                d0 = mfma(a0[x], X[ib][x], d0);
                d1 = mfma(a1[x], X[ib + 1][x], d1);
            }
        }
        f4 rhs = d0 + d1;
        float sgB[4];   // sgy^T operand: scale gy at (token 4(l/16) + x, row 16 w + l%16)
#pragma unroll
        for (int x = 0; x < 4; ++x) sgB[x] = sm.sgy[4 * g4 + x][j0 + lm];
        {
            const f4 bm4 = ld4(&sm.bm[lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) rhs = mfma(bm4[x], sgB[x], rhs);
        }
        f4 dd = zero4();
        {
            const f4 tb4 = ld4(&sm.tb[lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) dd = mfma(tb4[x], rhs[x], dd);
        }
        float duv[4];   // du^T (token 4(l/16) + r, row 16 w + l%16), the B operand of the update
        {
            const Rsrc rdv = rsrc(dvout + (int64_t)tw * (a.H_v * S));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * g4 + r;
                const float bv = sm.bt[tt];
                duv[r] = -bv * dd[r];
                const float pbv = row16_sum(dd[r] * sm.du[tt][j0 + lm]);   // e, read before du replaces it
                sm.du[tt][j0 + lm] = duv[r];
                if (lm == 0) sm.pb[wv][tt] = pbv;
                if (tt < n) bst(rdv, bv * dd[r], (j0 + lm) * 4 + tt * et, 0);
            }
        }
        // Column part: P1 = M^T sgy against the block start (dq's dense part); its share of dg at
        // the block's first token; then P1 += KR^T (G1 masked s <= t).
        f4 p1, dgacc;
        {
            f4 pa = zero4(), pb = zero4();
#pragma unroll
            for (int jb = 0; jb < 8; jb += 2) {
                const f4 b0 = ld4(&sm.sgy[lm][16 * jb + 4 * g4]), b1 = ld4(&sm.sgy[lm][16 * jb + 16 + 4 * g4]);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    pa = mfma(Mb[jb][x], b0[x], pa);
                    pb = mfma(Mb[jb + 1][x], b1[x], pb);
                }
            }
            p1 = pa + pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) dgacc[r] = sm.qcI[i0 + 4 * g4 + r][lm] * p1[r];
            const f4 kr4 = ld4(&sm.krI[i0 + lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) p1 = mfma(kr4[x], sm.g1[4 * g4 + x][lm], p1);
        }
        __syncthreads();   // X' transposed, du, dbeta partials
        // ---- phase B.  Column part: P3 = X'^T delta, P2 = M^T du, the G2 partial over the wave's
        // rows, the column sums of X' .* M.  Chain: X = X' + sgy qc^T + du kc^T.
        f4 p3, p2, dg0;
        {
            f4 p3a = zero4(), p3b = zero4(), p2a = zero4(), p2b = zero4();
            float xa = 0.f, xb = 0.f;
#pragma unroll
            for (int jb = 0; jb < 8; jb += 2) {
                const f4 x0 = ld4(&sm.xt[i0 + lm][16 * jb + 4 * g4]), x1 = ld4(&sm.xt[i0 + lm][16 * jb + 16 + 4 * g4]);
                const f4 e0 = ld4(&sm.ee[lm][16 * jb + 4 * g4]), e1 = ld4(&sm.ee[lm][16 * jb + 16 + 4 * g4]);
                const f4 u0 = ld4(&sm.du[lm][16 * jb + 4 * g4]), u1 = ld4(&sm.du[lm][16 * jb + 16 + 4 * g4]);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    p3a = mfma(x0[x], e0[x], p3a);
                    p3b = mfma(x1[x], e1[x], p3b);
                    p2a = mfma(Mb[jb][x], u0[x], p2a);
                    p2b = mfma(Mb[jb + 1][x], u1[x], p2b);
                    xa = fmaf(x0[x], Mb[jb][x], xa);
                    xb = fmaf(x1[x], Mb[jb + 1][x], xb);
                }
            }
            p3 = p3a + p3b;
            p2 = p2a + p2b;
            // dg at the block's first token: the column sums of X .* M with X after the update,
            // = sum(X' .* M) + sum_t (qc_t P1 + kc_t P2) over the dense parts
            const f4 xm4 = to_tile(rows4_sum(xa + xb));
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dg0[r] = xm4[r] + row16_sum(dgacc[r] + sm.kcI[i0 + 4 * g4 + r][lm] * p2[r]);
            const f4 qc4 = ld4(&sm.qcI[i0 + lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) p3 = mfma(qc4[x], sm.g1[lm][4 * g4 + x], p3);   // QC^T (G1^T, s >= t)
        }
        {   // G2 partial over rows 16 w ..: delta^T (row s = l%16) times du (column t = l%16)
            const f4 e4 = ld4(&sm.ee[lm][j0 + 4 * g4]), u4 = ld4(&sm.du[lm][j0 + 4 * g4]);
            f4 g2p = zero4();
#pragma unroll
            for (int x = 0; x < 4; ++x) g2p = mfma(e4[x], u4[x], g2p);
#pragma unroll
            for (int r = 0; r < 4; ++r) g2p[r] = 4 * g4 + r < lm ? g2p[r] : 0.f;   // s < t
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.gp[wv][4 * g4 + r][lm] = g2p[r];
            st4(&sm.gpt[wv][lm][4 * g4], g2p);
        }
        if (wv == 0 && lane < W) {   // dbeta: the eight row-block partials in order
            float b = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) b += sm.pb[w2][lane];
            if (lane < n) dbout[(int64_t)(tw + lane) * a.H_v] = b;
        }
        __syncthreads();   // G2 partials
        // ---- phase C.  The G2 corrections, outputs, the dg recursion.
        {
            f4 g2v = zero4(), g2t = zero4();   // G2[4(l/16) + r][l%16] and G2[l%16][4(l/16) + r]
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                g2v += ld4(&sm.gpt[w2][lm][4 * g4]);
                g2t += ld4(&sm.gp[w2][lm][4 * g4]);
            }
            const f4 kr4 = ld4(&sm.krI[i0 + lm][4 * g4]), kc4 = ld4(&sm.kcI[i0 + lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                p3 = mfma(kc4[x], g2t[x], p3);    // KC^T (G2^T, s > t)
                p2 = mfma(kr4[x], g2v[x], p2);    // KR^T (G2, s < t)
            }
        }
        // the chain: X = X' + sgy qc^T + du kc^T
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            const f4 qa = ld4(&sm.qcI[16 * ib + lm][4 * g4]), ka = ld4(&sm.kcI[16 * ib + lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                X[ib] = mfma(qa[x], sgB[x], X[ib]);
                X[ib] = mfma(ka[x], duv[x], X[ib]);
            }
        }
        // dq = c P1, dk = P3 / c + c P2, dg increments q.*dq - k.*(P3 / c) + k.*(c P2)
        f4 cv = f4{1.f, 1.f, 1.f, 1.f};
        if (!dir) {
            const float *cp = cin + (int64_t)(tw + (lm < n ? lm : 0)) * (a.H_v * G);
#pragma unroll
            for (int r = 0; r < 4; ++r) cv[r] = cp[kda ? i0 + 4 * g4 + r : 0];
        }
        f4 dq4, dk4, inc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * g4 + r;
            const float c = cv[r], rc = rcp(c);
            dq4[r] = c * p1[r];
            dk4[r] = fmaf(rc, p3[r], c * p2[r]);
            inc[r] = sm.qcI[i][lm] * p1[r] - sm.krI[i][lm] * p3[r] + sm.kcI[i][lm] * p2[r];
        }
        // suffix sums of the increments over the block's tokens (lanes l%16 upwards)
#pragma unroll
        for (int d = 1; d < W; d <<= 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float o = __shfl_down(inc[r], d, W);
                inc[r] += (lm + d < W) ? o : 0.f;
            }
        }
        f4 dgv;
#pragma unroll
        for (int r = 0; r < 4; ++r) dgv[r] = lm == 0 ? dg0[r] : carry[r] + inc[r];
        carry = dg0;
        if (lm < n) {
            const int64_t o = (int64_t)(tw + lm) * (a.H_v * S) + i0 + 4 * g4;
            if (vec_out) {
                st4(dqout + o, dq4);
                st4(dkout + o, dk4);
                if (kda) st4(dgout + o, dgv);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dqout[o + r] = dq4[r];
                    dkout[o + r] = dk4[r];
                    if (kda) dgout[o + r] = dgv[r];
                }
            }
        }
        if (!kda) {   // scalar gate: the wave's column sum per token
            const float gsv = rows4_sum(dgv[0] + dgv[1] + dgv[2] + dgv[3]);
            if (g4 == 0) sm.gs[wv][lm] = gsv;
        }
        if (dir) {   // the gradient before the token's gates
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) X[ib] *= ld4(&sm.pv[16 * ib + 4 * g4]);
        }
        __syncthreads();   // row data and scratch are free for the next staging
        if (!kda && wv == 0 && lane < n) {
            float g = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) g += sm.gs[w2][lane];
            dgout[(int64_t)(tw + lane) * a.H_v] = g;
        }
    };

    // ---- the step sequence
    const float *snapu = a.snap + unit * a.n_ck_max * S * S;
    float *bsb = a.vsbuf + unit * (int64_t)a.nbs * (S * S);   // block starts of the segment
    const int n_ck = (L + C - 1) / C;
    auto seg_nb = [&](int sg) { return (min(sg * C + C, L) - sg * C + W - 1) / W; };
    auto n_steps = [&](int sg) { return 2 * seg_nb(sg) - 1 + (sg == n_ck - 1 ? 1 : 0); };
    // step k of segment sg: 0 replay block bb (saving the next block's start), 1 replay the last
    // block (final state), 2 walk block bb
    auto step_info = [&](int sg, int k, int &kind, int &bb) {
        const int nb = seg_nb(sg), fin = sg == n_ck - 1 ? 1 : 0;
        if (k < nb - 1) {
            kind = 0;
            bb = k;
        } else if (fin && k == nb - 1) {
            kind = 1;
            bb = nb - 1;
        } else {
            kind = 2;
            bb = nb - 1 - (k - (nb - 1) - fin);
        }
    };
    auto block_start = [&](int sg, int bb) -> const float * {
        return bb == 0 ? snapu + (int64_t)sg * S * S : bsb + (int64_t)bb * (S * S);
    };
    auto final_sums = [&](const f4 (&Mf)[8]) {   // the dg recursion's start after the last token
        if (a.dstate_out) carry = to_tile(colsum_mem(a.dstate_out + unit * S * S, Mf));
    };

    Pre P;
    f4 M[8];
    int sg = n_ck - 1, k = 0;
    if (L > 0) prefetch(P, sg * C);   // the segment's first step handles its block 0
    while (sg >= 0) {
        int kind, bb;
        step_info(sg, k, kind, bb);
        const int t0 = sg * C + bb * W, cnt = min(W, L - t0);
        int nsg = sg, nk = k + 1;
        if (nk == n_steps(sg)) {
            nsg = sg - 1;
            nk = 0;
        }
        int nt0 = -1;
        if (nsg >= 0) {
            int nkind, nbb;
            step_info(nsg, nk, nkind, nbb);
            nt0 = nsg * C + nbb * W;
        }
        const bool dir = P.dir != 0;
        // a column-scaled block is staged from the registers loaded during the previous step,
        // which then take the next step's inputs
        if (!dir) {
            if (kind == 2) stage_walk(P, cnt);
            else stage_replay(P, cnt);
        }
        if (nt0 >= 0) prefetch(P, nt0);
        if (kind != 2) {
            // replay: the block as one column-scaled block, or token by token, from the snapshot or
            // from the state the previous replay step left in LDS
            if (bb == 0) load_cols(block_start(sg, 0), M);
            else load_lds(M);
            const int nsub = dir ? cnt : 1;
            for (int u = 0; u < nsub; ++u) {
                if (dir) stage_token(t0, u, false);
                replay(M, dir);
                __syncthreads();
            }
            if (kind == 0) {
                save_cols(bsb + (int64_t)(bb + 1) * (S * S), M);   // for the walk of block bb + 1
                save_lds(M);                                        // for the next replay step
            } else {
                final_sums(M);
            }
        } else {
            // walk: the block as one column-scaled block, or its tokens from the last, each from
            // its own start state replayed from the block start
            const int nsub = dir ? cnt : 1;
            for (int u = 0; u < nsub; ++u) {
                const int tau = cnt - 1 - u;
                load_cols(block_start(sg, bb), M);
                if (dir) {
                    for (int sx = 0; sx < tau; ++sx) {
                        stage_token(t0, sx, false);
                        replay(M, true);
                        __syncthreads();
                    }
                    stage_token(t0, tau, true);
                    const float p = sm.pv[i0 + lm];
#pragma unroll
                    for (int jb = 0; jb < 8; ++jb) M[jb] *= p;
                }
                walk(M, dir ? t0 + tau : t0, dir ? 1 : cnt, dir);
            }
        }
        sg = nsg;
        k = nk;
    }
    {   // the gradient before token 0
        float *p = a.dstate + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) p[16 * ib + r] = X[ib][r];
    }
    for (int64_t idx = tid; idx < (int64_t)(a.T - L) * S; idx += NT) {   // padded tokens
        const int64_t row = (int64_t)(L + idx / S) * a.H_v;
        const int i = (int)(idx % S);
        dvout[row * S + i] = 0.f;
        dqout[row * S + i] = 0.f;
        dkout[row * S + i] = 0.f;
        if (kda) dgout[row * S + i] = 0.f;
        else if (i == 0) dgout[row] = 0.f;
        if (i == 0) dbout[row] = 0.f;
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
struct Gram1K {
    static constexpr auto fn = gram1_kernel<DT>;
};
template <int DT>
struct BwdK {
    static constexpr auto fn = bwd_mf_kernel<DT>;
};

int block_items(const Mf128Args &a) {
    const int64_t items = (int64_t)a.n_seqs_launch * ((a.T + W - 1) / W) * a.H_v;
    return (int)std::min<int64_t>(items, 16384);
}

}  // namespace

hipError_t launch_prep128(const Mf128Args &a, hipStream_t st) {
    const int64_t items = (int64_t)a.n_seqs_launch * ((a.T + W - 1) / W) * a.H_v;
    const int blocks = (int)std::min<int64_t>((items + PW - 1) / PW, 16384);
    return launch(pick<PrepK>(a.dtype), a, blocks, 64 * PW, st);
}

hipError_t launch_fwd_mf(const Mf128Args &a, hipStream_t st) {
    return launch(pick<FwdK>(a.dtype), a, a.n_seqs_launch * a.H_v, NT, st);
}

hipError_t launch_bwd_mf(const Mf128Args &a, hipStream_t st) {
    hipError_t e = launch(pick<Gram1K>(a.dtype), a, block_items(a), 64, st);
    if (e != hipSuccess) return e;
    return launch(pick<BwdK>(a.dtype), a, a.n_seqs_launch * a.H_v, NT, st);
}

}  // namespace gdn
