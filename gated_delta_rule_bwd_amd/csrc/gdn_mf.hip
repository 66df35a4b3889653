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
// by an exact telescoping identity, from its value at each checkpoint segment's first token,
// taken directly as a column sum of the gradient times the segment's snapshot.
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
// workgroup.  dq and dk of a key head shared by several value heads are summed by the column
// pass itself: one workgroup takes the value heads of the key head in increasing order.  The
// host runs both directions over pieces of the token axis (the state or gradient carried
// between launches), the column sums of a piece beside the chain of the next on a second
// stream.
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
// [column][token] LDS arrays with the token quads of a column rotated by bits 4-5 of the column,
// so that writes of four columns of one token spread over the banks; a quad stays contiguous
__device__ __forceinline__ int cti(int col, int t) { return col * KP + 4 * ((t >> 2) ^ ((col >> 4) & 3)) + (t & 3); }
__device__ __forceinline__ int ctq(int col, int q) { return col * KP + 4 * (q ^ ((col >> 4) & 3)); }

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
// the value of lane l + D in the same 16-lane row, 0 for the last D lanes of the row
template <int D>
__device__ __forceinline__ float row_shl0(float v) {
    return as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x100 + D, 0xF, 0xF, false));
}
// the value of lane l - D in the same 16-lane row, 0 for the first D lanes of the row
template <int D>
__device__ __forceinline__ float row_shr0(float v) {
    return as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x110 + D, 0xF, 0xF, false));
}
// the value of the last lane of the 16-lane row, in every lane of the row (row_newbcast:15)
__device__ __forceinline__ float row_bcast15(float v) {
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), 0x15F, 0xF, 0xF, false));
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
// four consecutive elements at byte offset o: one vector load when every row start is aligned
// to four elements, else four loads
template <int DT>
__device__ __forceinline__ f4 ld4v(Rsrc r, uint32_t o, bool vec) {
    constexpr uint32_t ES = sizeof(In<DT>);
    if (vec) return bld4<DT>(r, o);
    return f4{bld<DT>(r, o, 0), bld<DT>(r, o + ES, 0), bld<DT>(r, o + 2 * ES, 0), bld<DT>(r, o + 3 * ES, 0)};
}

// Loads issued one block ahead keep the input's own bits and are widened where they are staged:
// a widening right at the load would make the wave wait for that load there.
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
template <int DT>
struct RawT {
    using one = float;
    using four = f4;
};
template <>
struct RawT<GDN_DTYPE_F16> {
    using one = unsigned short;
    using four = u2;
};
template <>
struct RawT<GDN_DTYPE_BF16> {
    using one = unsigned short;
    using four = u2;
};
template <int DT>
using Raw = typename RawT<DT>::one;
template <int DT>
using Raw4 = typename RawT<DT>::four;
template <int DT>
__device__ __forceinline__ Raw<DT> rld(Rsrc r, uint32_t vbytes, uint32_t sbytes) {
    if constexpr (DT == GDN_DTYPE_F32) return bld<DT>(r, vbytes, sbytes);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, vbytes, sbytes, 0);
}
template <int DT>
__device__ __forceinline__ float widen(Raw<DT> x) {
    if constexpr (DT == GDN_DTYPE_F32) return x;
    else if constexpr (DT == GDN_DTYPE_BF16) return __builtin_bit_cast(float, (uint32_t)x << 16);
    else return (float)__builtin_bit_cast(_Float16, x);
}
// four elements as ld4v; the unaligned form packs four loads (it waits for them)
template <int DT>
__device__ __forceinline__ Raw4<DT> rld4v(Rsrc r, uint32_t o, bool vec) {
    if constexpr (DT == GDN_DTYPE_F32) {
        return ld4v<DT>(r, o, vec);
    } else {
        if (vec) return __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
        uint32_t h[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) h[x] = __builtin_amdgcn_raw_buffer_load_b16(r, o + 2 * x, 0, 0);
        return u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
}
template <int DT>
__device__ __forceinline__ f4 widen4(Raw4<DT> v) {
    if constexpr (DT == GDN_DTYPE_F32) {
        return v;
    } else {
        f4 o;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            o[x] = widen<DT>((unsigned short)((x & 1) ? (v[x >> 1] >> 16) : (v[x >> 1] & 0xffffu)));
        return o;
    }
}
__device__ __forceinline__ bool rows_aligned(const void *p, const gdn_strides &st, uint32_t es) {
    return (((uintptr_t)p & (4 * es - 1)) == 0) && st.seq % 4 == 0 && st.tok % 4 == 0 && st.head % 4 == 0;
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
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lm = lane & 15, g4 = lane >> 4;
    float (*tr)[W + 1] = trs[wv];
    const int nblk = (a.T + W - 1) / W;
    const int G = a.kda ? S : 1;
    const bool kda = a.kda != 0;
    const int b_lo = a.t_lo / W, nbp = min(nblk, (a.t_hi + W - 1) / W) - b_lo;   // the launch's blocks
    const int64_t items = (int64_t)a.n_seqs_launch * nbp * a.H_v;
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
        const int b = b_lo + (int)(rest % nbp), sl = (int)(rest / nbp);
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

constexpr int NW = 8;          // waves per workgroup of the column pass, 16 rows (columns) each
constexpr int NT = 64 * NW;    // its threads

// A workgroup owns R = 16 NWC rows of a unit (sequence, value head): all 128 (NWC = 8), or one of
// two halves when the launch has too few units to fill the chip with whole units (the rows of
// the state evolve independently).  Wave w holds rows j0 = R slab + 16 w .. + 15 of the state
// transposed as eight 16 x 16 tiles: tile ib, lane l, register r holds
// M[j0 + l%16][16 ib + 4(l/16) + r].  Thread tid stages column tid % 128 of tokens
// TPT (tid / 128) .. + TPT - 1 of a block; the next block's inputs are loaded into registers while
// the current block is computed.
struct alignas(16) FwdLds {
    float kc[W][SP], qc[W][SP];   // c.*k, c.*q   [token][column]
    float kr[S][KP];              // k./c         [column][token]
    float pv[S];                  // block product per column (a token's gates)
};

template <int DT, int NWC>
__global__ void __launch_bounds__(64 * NWC) fwd_mf_kernel(const Mf128Args a) {
    constexpr int NTC = 64 * NWC, NSL = NW / NWC, TPT = W * S / NTC;
    __shared__ FwdLds smb[2];   // staged blocks, alternately (one barrier per block)
    constexpr uint32_t ES = sizeof(In<DT>);
    const int ul = blockIdx.x / NSL, slab = blockIdx.x % NSL;
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int j0 = 16 * (NWC * slab + wv);
    const int ci = tid & (S - 1), tg = __builtin_amdgcn_readfirstlane(tid >> 7);   // staging: column ci, tokens TPT tg ..
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

    // the state entering the launch's tokens: state0 at the sequence's start, else the carry
    const bool from_carry = a.t_lo > 0;
    const int t_end = min(L, a.t_hi);   // the launch's last token (exclusive) of this sequence
    f4 M[S / 16];
    {
        const float *p = (from_carry ? a.carry : a.state0) + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) {
            if (vec_state || from_carry) M[ib] = ld4(p + 16 * ib);
            else M[ib] = f4{p[16 * ib], p[16 * ib + 1], p[16 * ib + 2], p[16 * ib + 3]};
        }
    }
    auto store_state = [&](float *base) {
        float *p = base + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < S / 16; ++ib) st4(p + 16 * ib, M[ib]);
    };
    float *snap = a.snap + unit * a.n_ck_max * S * S;

    // inputs of one block: column ci of c, k, q at tokens TPT tg .. (tokens past the end load the
    // last one, replaced when staged); per lane v and beta at (token 4(l/16) + r, row j0 + l%16)
    // and the operands of Te^T and Bm^T
    struct Pre {
        float c[TPT];
        Raw<DT> k[TPT], q[TPT];
        Raw<DT> v[4], b[4];
        float te[4], bm[4];
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
        for (int x = 0; x < TPT; ++x) {
            const uint32_t tt = (uint32_t)min(TPT * tg + x, cnt - 1);
            P.c[x] = bldf(rc, ccol, tt * ct);
            P.k[x] = rld<DT>(rk, ci * ES, tt * kt);
            P.q[x] = rld<DT>(rq, ci * ES, tt * qt);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t tt = (uint32_t)min(4 * g4 + r, cnt - 1);
            P.v[r] = rld<DT>(rv, (j0 + lm) * ES + tt * vt, 0);
            P.b[r] = rld<DT>(rb, tt * bt, 0);
            P.te[r] = bldf(rw, (W * W + (4 * g4 + r) * W + lm) * 4, 0);
            P.bm[r] = bldf(rw, ((4 * g4 + r) * W + lm) * 4, 0);
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
    if (a.t_lo < t_end) prefetch(P, a.t_lo);
    for (int b = a.t_lo / W; b * W < t_end; ++b) {
        const int t0 = b * W, cnt = min(W, L - t0);
        if (t0 % a.C == 0) store_state(snap + (int64_t)(t0 / a.C) * S * S);
        if (!P.dir) {
            FwdLds &sm = smb[cur];
            float krow[TPT];
#pragma unroll
            for (int x = 0; x < TPT; ++x) {
                const int tt = TPT * tg + x;
                const bool ok = tt < cnt;   // tokens past the end: c = 1 and zeros
                const float c = ok ? P.c[x] : 1.f, k = ok ? widen<DT>(P.k[x]) : 0.f;
                krow[x] = k * rcp(c);
                sm.kc[tt][ci] = k * c;
                sm.qc[tt][ci] = ok ? widen<DT>(P.q[x]) * c : 0.f;
                if (tt == cnt - 1) sm.pv[ci] = c;
            }
#pragma unroll
            for (int x = 0; x < TPT; x += 4)
                st4(&sm.kr[ci][TPT * tg + x], f4{krow[x], krow[x + 1], krow[x + 2], krow[x + 3]});
            float vv[4], bb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = 4 * g4 + r < cnt;
                vv[r] = ok ? widen<DT>(P.v[r]) : 0.f;
                bb[r] = ok ? widen<DT>(P.b[r]) : 0.f;
            }
            const float teA[4] = {P.te[0], P.te[1], P.te[2], P.te[3]}, bmA[4] = {P.bm[0], P.bm[1], P.bm[2], P.bm[3]};
            __syncthreads();
            if (t0 + W < t_end) prefetch(P, t0 + W);   // the registers are free again
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
                for (int x = 0; x < TPT; ++x) {
                    const int tt = TPT * tg + x;
                    sm.kc[tt][ci] = tt == 0 ? kx : 0.f;
                    sm.qc[tt][ci] = tt == 0 ? qx : 0.f;
                }
#pragma unroll
                for (int x = 0; x < TPT; x += 4) st4(&sm.kr[ci][TPT * tg + x], f4{tg == 0 && x == 0 ? kx : 0.f, 0.f, 0.f, 0.f});
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
            if (t0 + W < t_end) prefetch(P, t0 + W);
        }
    }
    if (yout) {   // padded tokens of the launch: the workgroup's rows
        constexpr int R = 16 * NWC;
        const int p0 = max(L, a.t_lo), p1 = min(a.T, a.t_hi);
        for (int64_t idx = tid; idx < (int64_t)max(0, p1 - p0) * R; idx += NTC) {
            const int64_t t = p0 + idx / R;
            yout[t * a.sy.tok + 16 * NWC * slab + (int)(idx % R)] = 0.f;
        }
    }
    if (a.t_hi < a.T) {   // the state after the launch's tokens, for the next launch
        store_state(a.carry + unit * S * S);
    } else if (a.state_out) {
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

// The backward runs as two passes over the blocks.
//
// Pass 1, the chain (one workgroup per unit, or per row slab).  The rows of the state gradient
// evolve independently, and its recurrence (dd = dM k, then the update of dM) reads no state, so
// this pass walks the blocks of a sequence from the last in the row layout and never replays the
// state.  Wave w holds rows 16 w .. 16 w + 15 of the gradient X = dM diag(c) transposed as eight
// tiles (tile ib, lane l, register r: X[16 w + l%16][16 ib + 4(l/16) + r]).  Per block: the fold
// X' = X diag(P) (P the block's gate product); dd^T = Tb (KR X'^T + Bm sgy^T); dv = beta dd
// (which also hands du = -dv to pass 2); dbeta = dd . e; the block's Grams over the rows
// G1 = delta^T sgy and G2 = delta^T du for pass 2; X = X' + sgy qc^T + du kc^T; and
// P3 = X'^T delta, the column sums of the gradient against the block's deltas, from the gradient
// entering the block transposed through LDS.  At a checkpoint segment's first token: dg there.
//
// Pass 2, the column sums (one workgroup per checkpoint segment of a (sequence, key head), all in
// parallel; inside it the value heads of the key head one after the other, adding dq and dk).
// Wave w holds columns 16 w .. 16 w + 15 of the state M as eight tiles (tile jb, lane l,
// register r: M[16 jb + 4(l/16) + r][16 w + l%16]).  Starting from the segment's snapshot, per
// block: the column sums against the block's start state (dq, the dense part of dk besides P3,
// the increments of dg), then the replay to the next block's start.  Column results are tiles
// P[i][t] (lane l, register r: column 16 w + 4(l/16) + r, token l%16).
//
// The chain stages each block into one LDS buffer and takes two barriers per block (after the
// staging; after the step, before the gradient entering the next step is written for P3); the
// column pass stages block b + 1 while block b may still be read, in the other of two LDS
// buffers, so one barrier per block suffices.  Results the waves combine (dbeta, the Grams, the
// scalar gate's dg) are summed after a later barrier.
constexpr int GP = W + 4;   // row pitch of the per-wave 16 x 16 partials

template <int NWC>
struct alignas(16) ChainLds {
    static constexpr int RP = 16 * NWC + 4;   // row pitch of the workgroup's rows
    float krT[W][SP];          // k./c        [token][column]
    float sgy[W][RP];          // scale gy    [token][row of the workgroup]
    float er[W][RP];           // e           [token][row of the workgroup]
    float qcI[S][KP];          // c.*q        [column][token]
    float kcI[S][KP];          // c.*k        [column][token]
    float pv[S];               // fold factor per column (a token's gates)
    float bt[W];               // beta
    float bm[W][W], tb[W][W];  // Bm, Tb
    float pb[NWC][W];          // per-wave partials of dbeta
    float p1[NWC][W][GP];      // per-wave partials of G1 [s][t]
    float p2[NWC][W][GP];      // per-wave partials of G2 [s][t]
    float anp[NWC][S];         // per-wave partials of dg at a segment's first token
};

// The chain's workgroup owns 16 NWC rows of a unit (all, or one of NSL = 8 / NWC slabs: the rows
// are independent); its sums over rows (dbeta, G1, G2) are written per slab, and the column pass
// adds the slabs in order.
template <int DT, int NWC>
__global__ void __launch_bounds__(64 * NWC) chain_kernel(const Mf128Args a) {
    constexpr int NTC = 64 * NWC, NSL = NW / NWC, R = 16 * NWC;
    __shared__ ChainLds<NWC> sm;       // the staged block (two barriers per block)
    __shared__ float dut[NWC][W][GP];   // each wave's du, [token][row], for its Grams
    __shared__ f4 tT[R * S / 4];        // the gradient entering the step, for P3 (transposed reads)
    constexpr uint32_t ES = sizeof(In<DT>);
    const int ul = blockIdx.x / NSL, slab = blockIdx.x % NSL;
    const int sl = ul / a.H_v, h = ul % a.H_v;
    const int64_t s = a.s_base + sl;
    const int hk = h % a.H_k;
    const int L = a.lens[sl];
    const int64_t unit = s * a.H_v + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int jl = 16 * wv, r0 = R * slab, j0 = r0 + jl;   // the wave's rows: local and in the state
    const int nblk = (a.T + W - 1) / W;
    const int G = a.kda ? S : 1;
    const int nsl = a.nslab;
    const float scale = a.scale;
    const float *cin = a.cbuf + (s * a.T * a.H_v + h) * (int64_t)G;
    const In<DT> *kin = tin<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qin = tin<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const In<DT> *gyin = tin<DT>(a.gy) + s * a.sgy.seq + h * a.sgy.head + r0;
    const In<DT> *bin = tin<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
    const int64_t row0 = s * a.T * a.H_v + h;   // per-token workspace row of token 0; stride H_v
    const float *ein = a.ebuf + row0 * S + r0;
    float *dvout = a.dv + row0 * S;
    const bool vec_dv = ((uintptr_t)a.dv & 15) == 0;
    const int64_t prow0 = (s * a.pb_T - a.pb_t0) * a.H_v + h;   // piece-buffer row of token 0; stride H_v
    float *dbout = NSL > 1 ? a.dbp + prow0 * nsl + slab : a.dbeta + row0;   // stride H_v nsl per token
    const int64_t dbt = NSL > 1 ? (int64_t)a.H_v * nsl : a.H_v;
    float *p3out = a.p3buf + prow0 * S;                              // token stride H_v S
    float *ancu = a.anc + unit * (int64_t)a.n_ck_max * S;
    const int64_t gbase = ((s * (a.pb_T / W) - a.pb_t0 / W) * a.H_v + h) * nsl + slab;   // block b at b H_v nsl W^2
    float *g1u = a.g1buf + gbase * (W * W);
    float *g2u = a.g2buf + gbase * (W * W);
    const uint32_t ct = (uint32_t)(a.H_v * G) * 4, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES,
                   gyt = (uint32_t)a.sgy.tok * ES, bt = (uint32_t)a.sb.tok * ES, et = (uint32_t)a.H_v * S * 4;

    // the gradient entering the launch's tokens (walking backwards): dstate_out after the
    // sequence's end, else the carry from the launch of the later tokens
    const bool from_carry = a.t_hi < a.T;
    f4 X[8];
    if (from_carry) {
        const float *p = a.carry + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) X[ib] = ld4(p + 16 * ib);
    } else if (a.dstate_out) {
        const float *p = a.dstate_out + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) X[ib] = f4{p[16 * ib], p[16 * ib + 1], p[16 * ib + 2], p[16 * ib + 3]};
    } else {
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) X[ib] = zero4();
    }

    // inputs of a block, loaded one block ahead (tokens past the end load the last one, replaced
    // when staged): thread (tk = tid / 32 + v NTC / 32, cg = tid % 32) takes columns 4 cg .. + 3
    // of token tk of c, k and q and that token's beta; thread (tr, rq) rows 4 rq .. + 3 of the
    // workgroup at token tr of gy and e; entries of Bm and Tb
    constexpr int TPV = S * W / (4 * NTC);
    const int cg = tid & 31, tk0 = tid >> 5;
    const int rq = tid % (R / 4), tr = tid / (R / 4);
    const bool vk = rows_aligned(a.k, a.sk, ES), vq = rows_aligned(a.q, a.sq, ES), vgy = rows_aligned(a.gy, a.sgy, ES);
    struct Pre {
        f4 c[TPV];
        Raw4<DT> k[TPV], q[TPV];
        Raw<DT> b[TPV];
        Raw4<DT> gy;
        f4 e;
        float m0, m1;
        int dir;
    };
    auto prefetch = [&](Pre &P, int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        P.dir = sload(a.wflag, bi);
        const Rsrc rc = rsrc(cin + (int64_t)t0 * (a.H_v * G)), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                   rq_ = rsrc(qin + (int64_t)t0 * a.sq.tok), rgy = rsrc(gyin + (int64_t)t0 * a.sgy.tok),
                   re = rsrc(ein + (int64_t)t0 * (a.H_v * S)), rb = rsrc(bin + (int64_t)t0 * a.sb.tok),
                   rw = rsrc(a.wmat + bi * MATF);
#pragma unroll
        for (int v = 0; v < TPV; ++v) {
            const uint32_t tt = (uint32_t)min(tk0 + v * (NTC / 32), cnt - 1);
            if (a.kda) P.c[v] = ld4v<GDN_DTYPE_F32>(rc, tt * ct + 16 * cg, true);
            else P.c[v] = f4{1.f, 1.f, 1.f, 1.f} * bldf(rc, tt * ct, 0);
            P.k[v] = rld4v<DT>(rk, tt * kt + 4 * cg * ES, vk);
            P.q[v] = rld4v<DT>(rq_, tt * qt + 4 * cg * ES, vq);
            P.b[v] = rld<DT>(rb, tt * bt, 0);
        }
        {
            const uint32_t tt = (uint32_t)min(tr, cnt - 1);
            P.gy = rld4v<DT>(rgy, tt * gyt + 4 * rq * ES, vgy);
            P.e = ld4v<GDN_DTYPE_F32>(re, tt * et + 16 * rq, true);
        }
        const uint32_t m = tid & 255;
        P.m0 = bldf(rw, m * 4, 0);                  // Bm
        P.m1 = bldf(rw, (2 * W * W + m) * 4, 0);    // Tb
    };
    // staging of a column-scaled block
    auto stage = [&](ChainLds<NWC> &sm, const Pre &P, int cnt) {
        float *qcI = &sm.qcI[0][0], *kcI = &sm.kcI[0][0];
#pragma unroll
        for (int v = 0; v < TPV; ++v) {
            const int tt = tk0 + v * (NTC / 32);
            const bool ok = tt < cnt;   // tokens past the end: c = 1 and zeros
            const f4 c = ok ? P.c[v] : f4{1.f, 1.f, 1.f, 1.f}, k = ok ? widen4<DT>(P.k[v]) : zero4();
            const f4 qc = ok ? widen4<DT>(P.q[v]) * c : zero4(), kc = k * c;
            st4(&sm.krT[tt][4 * cg], f4{k[0] * rcp(c[0]), k[1] * rcp(c[1]), k[2] * rcp(c[2]), k[3] * rcp(c[3])});
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                qcI[cti(4 * cg + x, tt)] = qc[x];
                kcI[cti(4 * cg + x, tt)] = kc[x];
            }
            if (tt == cnt - 1) st4(&sm.pv[4 * cg], c);
            if (cg == 0) sm.bt[tt] = ok ? widen<DT>(P.b[v]) : 0.f;
        }
        {
            const bool ok = tr < cnt;
            st4(&sm.sgy[tr][4 * rq], ok ? widen4<DT>(P.gy) * scale : zero4());
            st4(&sm.er[tr][4 * rq], ok ? P.e : zero4());
        }
        if (tid < 256) {
            (&sm.bm[0][0])[tid] = P.m0;
            (&sm.tb[0][0])[tid] = P.m1;
        }
    };
    // staging of token t0 + tau of a token-by-token block (loaded directly) as a one-token block
    // with c = 1, the token's gates in pv
    auto stage_token = [&](ChainLds<NWC> &sm, int t0, int tau) {
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        const int64_t t = t0 + tau;
        float *qcI = &sm.qcI[0][0], *kcI = &sm.kcI[0][0];
        const bool z = tk0 == 0;   // threads of token slot 0 load the token; the others zero
#pragma unroll
        for (int v = 0; v < TPV; ++v) {
            const int tt = tk0 + v * (NTC / 32);
            f4 k = zero4(), q = zero4();
            if (z && v == 0) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    k[x] = (float)kin[t * a.sk.tok + 4 * cg + x];
                    q[x] = (float)qin[t * a.sq.tok + 4 * cg + x];
                }
                f4 av;
#pragma unroll
                for (int x = 0; x < 4; ++x) av[x] = cin[t * (a.H_v * G) + (a.kda ? 4 * cg + x : 0)];
                st4(&sm.pv[4 * cg], av);
            }
            st4(&sm.krT[tt][4 * cg], k);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                qcI[cti(4 * cg + x, tt)] = q[x];
                kcI[cti(4 * cg + x, tt)] = k[x];
            }
            if (cg == 0) sm.bt[tt] = (z && v == 0) ? (float)bin[t * a.sb.tok] : 0.f;
        }
        {
            f4 gy = zero4(), e = zero4();
            if (tr == 0) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    gy[x] = scale * (float)gyin[t * a.sgy.tok + 4 * rq + x];
                    e[x] = ein[t * (a.H_v * S) + 4 * rq + x];
                }
            }
            st4(&sm.sgy[tr][4 * rq], gy);
            st4(&sm.er[tr][4 * rq], e);
        }
        if (tid < 256) {
            const int sg = tid >> 4, t2 = tid & 15;
            sm.bm[sg][t2] = (sg == 0 && t2 == 0) ? a.wmat[bi * MATF + tau * (W + 1)] : 0.f;
            sm.tb[sg][t2] = sg == t2 ? 1.f : 0.f;
        }
    };

    // ---- one step of the chain on a staged (sub)block of n tokens from tw: the fold and X'
    // (saved to xs when given), then, once the next block's inputs are in flight, the rest
    // The gradient entering a step is written to tT after the barrier that ends the step before:
    // tile (row tile, column tile) at 256 (8 rt + ct), element (rho, sigma) of a tile at
    // (16 rho + sigma) ^ (((rho >> 1) & 7) << 2), so that a lane's four columns of a row stay one
    // 16-byte write and the column reads (one element per lane, four rows per lane) spread over
    // the banks.
    auto swz = [](int rho, int sigma) { return (16 * rho + sigma) ^ (((rho >> 1) & 7) << 2); };
    auto save_T = [&]() {
        float *base = reinterpret_cast<float *>(tT) + 256 * 8 * wv + swz(lm, 4 * g4);
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) st4(base + 256 * ib, X[ib]);
    };
    auto fold = [&](const ChainLds<NWC> &sm) {
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) X[ib] *= ld4(&sm.pv[16 * ib + 4 * g4]);
    };
    // P3 = X'^T delta of a step over the workgroup's rows, X' = X diag(pv) the folded gradient
    // (pv = 1 for a token-by-token step): diag(pv) (X^T delta) with X from tT.  Wave w takes
    // the column tiles CT w .. CT w + CT - 1, each a contraction over the workgroup's NWC row tiles;
    // lane l, register r: column 16 ct + 4(l/16) + r, token l%16.  Two row slabs add their halves
    // into a zeroed buffer (two terms: the order does not change the sum).
    constexpr int CT = 8 / NWC;
    f4 xa[CT][NWC];
    auto p3_load = [&]() {
        const float *tf = reinterpret_cast<const float *>(tT);
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int rt = 0; rt < NWC; ++rt)
#pragma unroll
                for (int x = 0; x < 4; ++x) xa[c][rt][x] = tf[256 * (8 * rt + CT * wv + c) + swz(4 * g4 + x, lm)];
    };
    auto p3_finish = [&](const ChainLds<NWC> &sm, int tw, int n, bool fold_pv) {
        f4 dP[NWC];
#pragma unroll
        for (int rt = 0; rt < NWC; ++rt) dP[rt] = ld4(&sm.er[lm][16 * rt + 4 * g4]) * sm.bt[lm];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const int ct = CT * wv + c;
            f4 acc = zero4();
#pragma unroll
            for (int rt = 0; rt < NWC; ++rt)
#pragma unroll
                for (int x = 0; x < 4; ++x) acc = mfma(xa[c][rt][x], dP[rt][x], acc);
            if (fold_pv) acc *= ld4(&sm.pv[16 * ct + 4 * g4]);
            if (lm < n) {
                float *o = p3out + (int64_t)(tw + lm) * (a.H_v * S) + 16 * ct + 4 * g4;
                if constexpr (NSL == 1) {
                    st4(o, acc);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) unsafeAtomicAdd(o + r, acc[r]);
                }
            }
        }
    };
    // dg at a segment's first token: the column sums of the gradient there times the segment's
    // snapshot, over the wave's rows (summed over the waves after the next barrier)
    bool anc_pend = false;
    int anc_sg = 0;
    auto anchor_part = [&](ChainLds<NWC> &sm, int sgi) {
        const float *ms = a.snap + (unit * a.n_ck_max + sgi) * (int64_t)(S * S) + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            f4 v = X[ib] * ld4(ms + 16 * ib);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = row16_sum(v[r]);
            if (lm == 0) st4(&sm.anp[wv][16 * ib + 4 * g4], v);
        }
        anc_pend = true;
        anc_sg = sgi;
    };
    // mid(): work that needs no result of the step (the step's P3), placed after dd so that the
    // loads of tT it waits for have had the dd products' time to arrive
    auto step = [&](ChainLds<NWC> &sm, int tw, int n, bool dir, auto &&mid) {
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
        float sgB[4];   // sgy^T operand: scale gy at (token 4(l/16) + x, row j0 + l%16)
#pragma unroll
        for (int x = 0; x < 4; ++x) sgB[x] = sm.sgy[4 * g4 + x][jl + lm];
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
        float duv[4];   // du^T (token 4(l/16) + r, row j0 + l%16), the B operand of the update
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tt = 4 * g4 + r;
            duv[r] = -sm.bt[tt] * dd[r];
            const float pbv = row16_sum(dd[r] * sm.er[tt][jl + lm]);
            if (lm == 0) sm.pb[wv][tt] = pbv;
            dut[wv][tt][lm] = duv[r];
        }
        mid();
        // X = X' + sgy qc^T + du kc^T
        const float *qcI = &sm.qcI[0][0], *kcI = &sm.kcI[0][0];
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            const f4 qa = ld4(qcI + ctq(16 * ib + lm, g4)), ka = ld4(kcI + ctq(16 * ib + lm, g4));
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                X[ib] = mfma(qa[x], sgB[x], X[ib]);
                X[ib] = mfma(ka[x], duv[x], X[ib]);
            }
        }
        if (dir) {   // the gradient before the token's gates
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) X[ib] *= ld4(&sm.pv[16 * ib + 4 * g4]);
        }
        // the Grams over the wave's rows: delta^T (row s = l%16, the wave's rows along the
        // contraction) times scale gy and du (column t = l%16)
        {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            const f4 e4 = ld4(&sm.er[lm][jl + 4 * g4]) * sm.bt[lm];
            const f4 y4 = ld4(&sm.sgy[lm][jl + 4 * g4]), u4 = ld4(&dut[wv][lm][4 * g4]);
            // dv = beta dd = -du: token l%16, rows j0 + 4(l/16) ..
            if (lm < n) {
                float *o = dvout + (int64_t)(tw + lm) * (a.H_v * S) + j0 + 4 * g4;
                if (vec_dv) {
                    st4(o, -u4);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = -u4[r];
                }
            }
            f4 q1 = zero4(), q2 = zero4();
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                q1 = mfma(e4[x], y4[x], q1);
                q2 = mfma(e4[x], u4[x], q2);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sm.p1[wv][4 * g4 + r][lm] = q1[r];
                sm.p2[wv][4 * g4 + r][lm] = q2[r];
            }
        }
    };
    // the previous step's dbeta and Grams over the workgroup's rows: the per-wave partials in
    // order, once every wave has passed the barrier after this step's staging
    int pend_t0 = 0, pend_tau = -1, pend_n = 0;
    auto flush = [&](const ChainLds<NWC> &sp) {
        if (anc_pend) {
            for (int col = tid; col < S; col += NTC) {
                float g = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NWC; ++w2) g += sp.anp[w2][col];
                if constexpr (NSL == 1) ancu[(int64_t)anc_sg * S + col] = g;
                else unsafeAtomicAdd(&ancu[(int64_t)anc_sg * S + col], g);
            }
            anc_pend = false;
        }
        if (pend_n == 0) return;
        if (wv == 0 && lane < pend_n) {
            float b = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NWC; ++w2) b += sp.pb[w2][lane];
            dbout[(int64_t)(pend_t0 + (pend_tau < 0 ? lane : pend_tau)) * dbt] = b;
        }
        const int64_t gb = (int64_t)(pend_t0 / W) * a.H_v * nsl * (W * W);
        if (pend_tau < 0) {   // G1 keeps s <= t, G2 s < t
            for (int e = tid; e < 2 * W * W; e += NTC) {
                const int m = e & 255, sr = m >> 4, tc = m & 15;
                float g = 0.f;
                if (e < 256) {
#pragma unroll
                    for (int w2 = 0; w2 < NWC; ++w2) g += sp.p1[w2][sr][tc];
                    g1u[gb + m] = sr <= tc ? g : 0.f;
                } else {
#pragma unroll
                    for (int w2 = 0; w2 < NWC; ++w2) g += sp.p2[w2][sr][tc];
                    g2u[gb + m] = sr < tc ? g : 0.f;
                }
            }
        } else if (tid == 0) {   // a one-token block: its G1 on the diagonal
            float g = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NWC; ++w2) g += sp.p1[w2][0][0];
            g1u[gb + pend_tau * (W + 1)] = g;
        }
    };

    // Per step: staging, barrier, P3 and the step (all waves read the staged block and tT), barrier,
    // then the sums over the waves (flush) and the gradient entering the next step into tT.
    Pre P;
    const int nb = min((L + W - 1) / W, (a.t_hi + W - 1) / W), b_lo = a.t_lo / W;   // the launch's blocks
    save_T();   // the gradient entering the last block
    if (nb > b_lo) prefetch(P, (nb - 1) * W);
    for (int b = nb - 1; b >= b_lo; --b) {
        const int t0 = b * W, cnt = min(W, L - t0);
        const bool dir = P.dir != 0;
        if (!dir) {
            stage(sm, P, cnt);
            __syncthreads();
            p3_load();
            fold(sm);
            if (b > b_lo) prefetch(P, t0 - W);
            step(sm, t0, cnt, false, [&] { p3_finish(sm, t0, cnt, true); });
            if (t0 % a.C == 0) anchor_part(sm, t0 / a.C);
            pend_t0 = t0;
            pend_tau = -1;
            pend_n = cnt;
            __syncthreads();
            flush(sm);
            save_T();
        } else {
            if (b > b_lo) prefetch(P, t0 - W);
            for (int u = 0; u < cnt; ++u) {
                const int tau = cnt - 1 - u;
                stage_token(sm, t0, tau);
                __syncthreads();
                p3_load();
                step(sm, t0 + tau, 1, true, [&] { p3_finish(sm, t0 + tau, 1, false); });
                if (tau == 0 && t0 % a.C == 0) anchor_part(sm, t0 / a.C);
                pend_t0 = t0;
                pend_tau = tau;
                pend_n = 1;
                __syncthreads();
                flush(sm);
                save_T();
            }
        }
    }
    if (a.t_lo > 0) {   // the gradient before the launch's tokens, for the next launch
        float *p = a.carry + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) st4(p + 16 * ib, X[ib]);
    } else {   // the gradient before token 0
        float *p = a.dstate + unit * S * S + (int64_t)(j0 + lm) * S + 4 * g4;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) p[16 * ib + r] = X[ib][r];
    }
    const int pad0 = max(L, a.t_lo), pad1 = min(a.T, a.t_hi);   // padded tokens of the launch
    for (int64_t idx = tid; idx < (int64_t)max(0, pad1 - pad0) * R; idx += NTC) {
        const int64_t row = (int64_t)(pad0 + idx / R) * a.H_v;
        const int i = (int)(idx % R);
        dvout[row * S + r0 + i] = 0.f;
        if (slab == 0 && i == 0) a.dbeta[row0 + row] = 0.f;
    }
}

struct alignas(16) ColLds {
    float krI[S][KP];          // k./c        [column][token]; token by token: q and k of the gradient's update
    float qcI[S][KP];          // c.*q        [column][token]
    float kcI[S][KP];          // c.*k        [column][token]
    float cI[S][KP];           // c           [column][token]
    float dl[S][KP];           // delta       [row][token]; token by token: scale gy and du of the update
    float sgy[W][SP];          // scale gy    [token][row]
    float du[W][SP];           // du          [token][row]
    float pv[S];               // fold factor per column (a token's gates)
    float g1[W][GP];           // G1 = delta^T scale gy, [s][t], s <= t
    float g2[W][GP];           // G2 = delta^T du, [s][t], s < t
    float g2t[W][GP];          // G2 transposed
    float gs[NW][W];           // per-wave partial sums of the scalar gate's dg
};

template <int DT>
__global__ void __launch_bounds__(NT) colsum_kernel(const Mf128Args a) {
    __shared__ ColLds smb[2];
    constexpr uint32_t ES = sizeof(In<DT>);
    // one workgroup per (sequence, key head, segment): the value heads hk, hk + H_k, .. of the
    // key head one after the other, each adding its dq and dk to the key head's sums
    const int groups = a.n_seqs_launch * a.H_k;
    const int gl = blockIdx.x % groups, sg = a.t_lo / a.C + blockIdx.x / groups;
    const int sl = gl / a.H_k, hk = gl % a.H_k;
    const int64_t s = a.s_base + sl;
    const int L = a.lens[sl];
    const int C = a.C;
    const int nrep = a.H_v / a.H_k;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lm = lane & 15, g4 = lane >> 4;
    const int i0 = 16 * wv;   // the wave's columns
    const int ci = tid & (S - 1), tg = __builtin_amdgcn_readfirstlane(tid >> 7);   // staging: column/row ci, tokens 4 tg .. 4 tg + 3
    const int nblk = (a.T + W - 1) / W;
    const int G = a.kda ? S : 1;
    const float scale = a.scale;
    const bool kda = a.kda != 0;
    const In<DT> *kin = tin<DT>(a.k) + s * a.sk.seq + hk * a.sk.head;
    const In<DT> *qin = tin<DT>(a.q) + s * a.sq.seq + hk * a.sq.head;
    const int64_t qkt = (int64_t)a.H_k * S;     // token stride of dq and dk
    float *dqout = a.dq + (s * a.T * a.H_k + hk) * S;
    float *dkout = a.dk + (s * a.T * a.H_k + hk) * S;
    const bool vec_out = (((uintptr_t)a.dq | (uintptr_t)a.dk | (uintptr_t)a.dg) & 15) == 0;
    const bool vec_dv = ((uintptr_t)a.dv & 15) == 0;
    const uint32_t ct = (uint32_t)(a.H_v * G) * 4, kt = (uint32_t)a.sk.tok * ES, qt = (uint32_t)a.sq.tok * ES,
                   gyt = (uint32_t)a.sgy.tok * ES, bt = (uint32_t)a.sb.tok * ES, et = (uint32_t)a.H_v * S * 4;
    const int nsl = a.nslab;
    const int ts = sg * C;

    // the value head in progress (set at the top of each head's pass)
    int rep = 0, h = hk;
    int64_t unit = 0, row0 = 0;   // row0: per-token workspace row of token 0; stride H_v
    const float *cin = nullptr, *ein = nullptr, *dvin = nullptr;
    const In<DT> *gyin = nullptr, *bin = nullptr;
    float *dgout = nullptr;
    auto set_head = [&](int r) {
        rep = r;
        h = hk + r * a.H_k;
        unit = s * a.H_v + h;
        row0 = s * a.T * a.H_v + h;
        cin = a.cbuf + row0 * (int64_t)G;
        gyin = tin<DT>(a.gy) + s * a.sgy.seq + h * a.sgy.head;
        bin = tin<DT>(a.beta) + s * a.sb.seq + h * a.sb.head;
        ein = a.ebuf + row0 * S;
        dvin = a.dv + row0 * S;
        dgout = a.dg + row0 * G;
    };
    // padded tokens of the segment's span: dg of every value head, dq and dk of the key head
    {
        const int64_t p0 = max((int64_t)L, (int64_t)ts), p1 = min((int64_t)a.T, (int64_t)ts + C);
        for (int64_t idx = tid; idx < (p1 - p0) * S; idx += NT) {
            const int64_t t = p0 + idx / S;
            const int i = (int)(idx % S);
            dqout[t * qkt + i] = 0.f;
            dkout[t * qkt + i] = 0.f;
            for (int r = 0; r < nrep; ++r) {
                const int64_t row = (s * a.T + t) * a.H_v + hk + r * a.H_k;
                if (kda) a.dg[row * S + i] = 0.f;
                else if (i == 0) a.dg[row] = 0.f;
            }
        }
    }
    if (ts >= L) return;
    const int nb = (min(ts + C, L) - ts + W - 1) / W;

    // a 128 x 128 row-major [S][S] matrix (a snapshot) in the column layout
    const uint32_t vcol = ((4 * g4) * S + i0 + lm) * 4;
    auto load_cols = [&](const float *base, f4 (&Mc)[8]) {
        const Rsrc rs = rsrc(base);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Mc[jb][r] = bldf(rs, vcol + r * S * 4, 16 * jb * S * 4);
    };

    // inputs of a block, loaded one block ahead (tokens past the end load the last one, replaced
    // when staged): thread (tk = tid / 32, cg = tid % 32) takes columns (rows) 4 cg .. + 3 of token
    // tk of c, k, q, gy, e and dv and that token's beta; one entry of each slab's G1 and G2
    const int cg = tid & 31, tk = tid >> 5;
    const bool vk = rows_aligned(a.k, a.sk, ES), vq = rows_aligned(a.q, a.sq, ES), vgy = rows_aligned(a.gy, a.sgy, ES);
    struct Pre {
        f4 c, e, dv;
        Raw4<DT> k, q, gy;
        Raw<DT> b;
        float m1[2], m2[2];   // the chain's slabs (at most two)
        int dir;
    };
    auto prefetch = [&](Pre &P, int t0) {
        const int cnt = min(W, L - t0);
        const int64_t bi = (s * nblk + t0 / W) * a.H_v + h;
        P.dir = sload(a.wflag, bi);
        const Rsrc rc = rsrc(cin + (int64_t)t0 * (a.H_v * G)), rk = rsrc(kin + (int64_t)t0 * a.sk.tok),
                   rq = rsrc(qin + (int64_t)t0 * a.sq.tok), rgy = rsrc(gyin + (int64_t)t0 * a.sgy.tok),
                   re = rsrc(ein + (int64_t)t0 * (a.H_v * S)), rb = rsrc(bin + (int64_t)t0 * a.sb.tok),
                   rdv = rsrc(dvin + (int64_t)t0 * (a.H_v * S));
        const uint32_t tt = (uint32_t)min(tk, cnt - 1);
        if (kda) P.c = ld4v<GDN_DTYPE_F32>(rc, tt * ct + 16 * cg, true);
        else P.c = f4{1.f, 1.f, 1.f, 1.f} * bldf(rc, tt * ct, 0);
        P.k = rld4v<DT>(rk, tt * kt + 4 * cg * ES, vk);
        P.q = rld4v<DT>(rq, tt * qt + 4 * cg * ES, vq);
        P.gy = rld4v<DT>(rgy, tt * gyt + 4 * cg * ES, vgy);
        P.e = ld4v<GDN_DTYPE_F32>(re, tt * et + 16 * cg, true);
        P.dv = ld4v<GDN_DTYPE_F32>(rdv, tt * et + 16 * cg, vec_dv);
        P.b = rld<DT>(rb, tt * bt, 0);
        const int64_t gb = ((s * (a.pb_T / W) + (t0 - a.pb_t0) / W) * a.H_v + h) * nsl * (W * W) + (tid & 255);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t o = gb + min(k, nsl - 1) * (W * W);
            P.m1[k] = a.g1buf[o];
            P.m2[k] = a.g2buf[o];
        }
    };
    auto stage = [&](ColLds &sm, const Pre &P, int cnt) {
        const bool ok = tk < cnt;   // tokens past the end: c = 1 and zeros
        const f4 c = ok ? P.c : f4{1.f, 1.f, 1.f, 1.f}, k = ok ? widen4<DT>(P.k) : zero4();
        const f4 qc = ok ? widen4<DT>(P.q) * c : zero4(), kc = k * c, d = ok ? P.e * widen<DT>(P.b) : zero4();
        float *krI = &sm.krI[0][0], *qcI = &sm.qcI[0][0], *kcI = &sm.kcI[0][0], *cI = &sm.cI[0][0], *dl = &sm.dl[0][0];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int o = cti(4 * cg + x, tk);
            krI[o] = k[x] * rcp(c[x]);
            qcI[o] = qc[x];
            kcI[o] = kc[x];
            cI[o] = c[x];
            dl[o] = d[x];
        }
        st4(&sm.sgy[tk][4 * cg], ok ? widen4<DT>(P.gy) * scale : zero4());
        st4(&sm.du[tk][4 * cg], ok ? -P.dv : zero4());
        if (tk == cnt - 1) st4(&sm.pv[4 * cg], c);
        if (tid < 256) {   // the slabs' partials in order
            const float g1 = nsl > 1 ? P.m1[0] + P.m1[1] : P.m1[0], g2 = nsl > 1 ? P.m2[0] + P.m2[1] : P.m2[0];
            sm.g1[tid >> 4][tid & 15] = g1;
            sm.g2[tid >> 4][tid & 15] = g2;
            sm.g2t[tid & 15][tid >> 4] = g2;
        }
    };
    // token t0 + tau of a token-by-token block as a one-token block with c = 1 (loaded directly)
    auto stage_token = [&](ColLds &sm, int t0, int tau) {
        const int64_t t = t0 + tau;
        const float av = cin[t * (a.H_v * G) + (kda ? ci : 0)];
        const float kx = (float)kin[t * a.sk.tok + ci];
        const float qx = (float)qin[t * a.sq.tok + ci];
        const float gx = scale * (float)gyin[t * a.sgy.tok + ci];
        const float dx = (float)bin[t * a.sb.tok] * ein[t * (a.H_v * S) + ci];
        const float ux = -dvin[t * (a.H_v * S) + ci];
        const bool z = tg == 0;
        st4(&sm.krI[0][0] + ctq(ci, tg), f4{z ? kx : 0.f, 0.f, 0.f, 0.f});
        st4(&sm.qcI[0][0] + ctq(ci, tg), f4{z ? qx : 0.f, 0.f, 0.f, 0.f});
        st4(&sm.kcI[0][0] + ctq(ci, tg), f4{z ? kx : 0.f, 0.f, 0.f, 0.f});
        st4(&sm.cI[0][0] + ctq(ci, tg), f4{1.f, 1.f, 1.f, 1.f});
        st4(&sm.dl[0][0] + ctq(ci, tg), f4{z ? dx : 0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int tt = 4 * tg + x;
            sm.sgy[tt][ci] = tt == 0 ? gx : 0.f;
            sm.du[tt][ci] = tt == 0 ? ux : 0.f;
        }
        if (z) sm.pv[ci] = av;
        if (tid < 256) {
            const int sr = tid >> 4, t2 = tid & 15;
            float g = 0.f;
            if (sr == 0 && t2 == 0)
                for (int k = 0; k < nsl; ++k)
                    g += a.g1buf[(((s * (a.pb_T / W) + (t0 - a.pb_t0) / W) * a.H_v + h) * nsl + k) * (W * W) + tau * (W + 1)];
            sm.g1[sr][t2] = g;
            sm.g2[sr][t2] = 0.f;
            sm.g2t[sr][t2] = 0.f;
        }
    };
    // Z += A B^T over the staged token slots for the column layout: A = dl [row][slot], B = krI
    // [column][slot]
    auto rank_update = [&](const ColLds &sm, f4 (&Z)[8]) {
        const f4 kb = ld4(&sm.krI[0][0] + ctq(i0 + lm, g4));
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
            const f4 d4 = ld4(&sm.dl[0][0] + ctq(16 * jb + lm, g4));
#pragma unroll
            for (int x = 0; x < 4; ++x) Z[jb] = mfma(d4[x], kb[x], Z[jb]);
        }
    };

    // ---- the column sums of a staged (sub)block of n tokens from tw with start state M and
    // gradient X' at its end (column layout); then the state's replay to the block's end (dir: the
    // token's gates have scaled M already; otherwise the block product folds in at the end)
    f4 M[8];
    f4 dgrun;                     // dg at the next token, per column (i0 + 4(l/16) + r)
    const float *p3in = nullptr;   // the chain's P3 of the value head
    // (replay: the state after this (sub)block is needed; not after the segment's last token)
    auto block = [&](ColLds &sm, int tw, int n, bool dir, bool replay) {
        // the earlier value heads' dq and dk of the block's tokens (zero for the first head) and
        // the chain's P3 = X'^T delta, loaded first so that the products below cover their latency
        f4 pq = zero4(), pk = zero4(), p3 = zero4();
        if (lm < n) {
            const int64_t oq = (int64_t)(tw + lm) * qkt + i0 + 4 * g4;
            p3 = ld4(p3in + (int64_t)(tw + lm) * (a.H_v * S) + i0 + 4 * g4);
            if (rep > 0) {
                if (vec_out) {
                    pq = ld4(dqout + oq);
                    pk = ld4(dkout + oq);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pq[r] = dqout[oq + r];
                        pk[r] = dkout[oq + r];
                    }
                }
            }
        }
        // P1 = M^T sgy (dq's dense part), then P1 += KR^T G1
        f4 p1, p2, krv;
        {
            f4 pa = zero4(), pb = zero4();
#pragma unroll
            for (int jb = 0; jb < 8; jb += 2) {
                const f4 b0 = ld4(&sm.sgy[lm][16 * jb + 4 * g4]), b1 = ld4(&sm.sgy[lm][16 * jb + 16 + 4 * g4]);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    pa = mfma(M[jb][x], b0[x], pa);
                    pb = mfma(M[jb + 1][x], b1[x], pb);
                }
            }
            p1 = pa + pb;
            const f4 kr4 = ld4(&sm.krI[0][0] + ctq(i0 + lm, g4));
#pragma unroll
            for (int x = 0; x < 4; ++x) p1 = mfma(kr4[x], sm.g1[4 * g4 + x][lm], p1);
        }
        // P2 = M^T du; the rank-16 corrections of P2 and P3 through the block's Grams
        {
            f4 p2a = zero4(), p2b = zero4();
#pragma unroll
            for (int jb = 0; jb < 8; jb += 2) {
                const f4 u0 = ld4(&sm.du[lm][16 * jb + 4 * g4]), u1 = ld4(&sm.du[lm][16 * jb + 16 + 4 * g4]);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    p2a = mfma(M[jb][x], u0[x], p2a);
                    p2b = mfma(M[jb + 1][x], u1[x], p2b);
                }
            }
            p2 = p2a + p2b;
#pragma unroll
            for (int r = 0; r < 4; ++r) krv[r] = (&sm.krI[0][0])[cti(i0 + 4 * g4 + r, lm)];
            const f4 qc4 = ld4(&sm.qcI[0][0] + ctq(i0 + lm, g4)), kr4 = ld4(&sm.krI[0][0] + ctq(i0 + lm, g4)),
                     kc4 = ld4(&sm.kcI[0][0] + ctq(i0 + lm, g4));
            const f4 g1t = f4{sm.g1[lm][4 * g4], sm.g1[lm][4 * g4 + 1], sm.g1[lm][4 * g4 + 2], sm.g1[lm][4 * g4 + 3]};
            const f4 g2v = ld4(&sm.g2t[lm][4 * g4]), g2t = ld4(&sm.g2[lm][4 * g4]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                p3 = mfma(qc4[x], g1t[x], p3);    // QC^T (G1^T, s >= t)
                p3 = mfma(kc4[x], g2t[x], p3);    // KC^T (G2^T, s > t)
                p2 = mfma(kr4[x], g2v[x], p2);    // KR^T (G2, s < t)
            }
        }
        // the replay: M += delta kr^T, then the block product
        if (replay) {
            rank_update(sm, M);
            if (!dir) {
                const float p = sm.pv[i0 + lm];
#pragma unroll
                for (int jb = 0; jb < 8; ++jb) M[jb] *= p;
            }
        }
        // dq = c P1, dk = P3 / c + c P2, dg increments q.*dq - k.*(P3 / c) + k.*(c P2)
        f4 dq4, dk4, inc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * g4 + r;
            const float c = (&sm.cI[0][0])[cti(i, lm)], rc = rcp(c);
            dq4[r] = c * p1[r];
            dk4[r] = fmaf(rc, p3[r], c * p2[r]);
            inc[r] = (&sm.qcI[0][0])[cti(i, lm)] * p1[r] - krv[r] * p3[r] + (&sm.kcI[0][0])[cti(i, lm)] * p2[r];
        }
        // dg_t = dg at the segment's first token - the increments of the earlier tokens: an
        // exclusive prefix sum over the block's tokens (lanes l%16 upwards) from the running value
        f4 dgv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = inc[r];
            v += row_shr0<1>(v);
            v += row_shr0<2>(v);
            v += row_shr0<4>(v);
            v += row_shr0<8>(v);
            dgv[r] = dgrun[r] - (v - inc[r]);
            dgrun[r] -= row_bcast15(v);
        }
        if (lm < n) {
            const int64_t o = (int64_t)(tw + lm) * (a.H_v * S) + i0 + 4 * g4;
            const int64_t oq = (int64_t)(tw + lm) * qkt + i0 + 4 * g4;
            if (vec_out) {
                st4(dqout + oq, pq + dq4);
                st4(dkout + oq, pk + dk4);
                if (kda) st4(dgout + o, dgv);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dqout[oq + r] = pq[r] + dq4[r];
                    dkout[oq + r] = pk[r] + dk4[r];
                    if (kda) dgout[o + r] = dgv[r];
                }
            }
        }
        if (!kda) {   // scalar gate: the wave's column sum per token
            const float gsv = rows4_sum(dgv[0] + dgv[1] + dgv[2] + dgv[3]);
            if (g4 == 0) sm.gs[wv][lm] = gsv;
        }
    };
    // the scalar gate's dg of the previous step: the eight per-wave sums in order, once every
    // wave has passed the barrier after this step's staging
    int pend_tw = 0, pend_n = 0;
    auto flush = [&](const ColLds &sp) {
        if (!kda && wv == 0 && lane < pend_n) {
            float g = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) g += sp.gs[w2][lane];
            dgout[(int64_t)(pend_tw + lane) * a.H_v] = g;
        }
    };

    int cur = 0;
    for (int r = 0; r < nrep; ++r) {
        set_head(r);
        if (nsl > 1) {   // dbeta of the segment's tokens: the chain's slabs in order
            for (int t = ts + tid; t < min(ts + C, L); t += NT) {
                const int64_t rw = row0 + (int64_t)t * a.H_v, pr = (s * a.pb_T + t - a.pb_t0) * a.H_v + h;
                float b = 0.f;
                for (int k = 0; k < nsl; ++k) b += a.dbp[pr * nsl + k];
                a.dbeta[rw] = b;
            }
        }
        load_cols(a.snap + (unit * a.n_ck_max + sg) * (int64_t)(S * S), M);
        dgrun = ld4(a.anc + (unit * a.n_ck_max + sg) * (int64_t)S + i0 + 4 * g4);
        p3in = a.p3buf + ((s * a.pb_T - a.pb_t0) * a.H_v + h) * S;
        Pre P;
        prefetch(P, ts);
        pend_n = 0;
        for (int bb = 0; bb < nb; ++bb) {
            const int t0 = ts + bb * W, cnt = min(W, L - t0);
            const bool dir = P.dir != 0;
            // a column-scaled block in one step; a token-by-token block one token per step
            const int nsub = dir ? cnt : 1;
            for (int tau = 0; tau < nsub; ++tau) {
                ColLds &sm = smb[cur];
                if (!dir) stage(sm, P, cnt);
                else stage_token(sm, t0, tau);
                if (tau == 0 && bb + 1 < nb) prefetch(P, t0 + W);
                __syncthreads();
                flush(smb[cur ^ 1]);
                if (dir) {
                    const float p = sm.pv[i0 + lm];
#pragma unroll
                    for (int jb = 0; jb < 8; ++jb) M[jb] *= p;
                }
                block(sm, dir ? t0 + tau : t0, dir ? 1 : cnt, dir, bb + 1 < nb || (dir && tau + 1 < nsub));
                pend_tw = dir ? t0 + tau : t0;
                pend_n = dir ? 1 : cnt;
                cur ^= 1;
            }
        }
        __syncthreads();
        flush(smb[cur ^ 1]);
    }
}

// p[0 .. n) = 0 (n a multiple of 4, p 16-byte aligned); a kernel rather than a memset, so that a
// captured graph records no memset node
__global__ void __launch_bounds__(256) zero_kernel(float *p, int64_t n) {
    for (int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); i < n; i += 4 * (int64_t)gridDim.x * 256)
        st4(p + i, zero4());
}
hipError_t launch_zero(float *p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int blocks = (int)std::min<int64_t>((n / 4 + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
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
    static constexpr auto fn = fwd_mf_kernel<DT, NW>;
};
template <int DT>
struct FwdK2 {
    static constexpr auto fn = fwd_mf_kernel<DT, NW / 2>;
};
template <int DT>
struct ChainK {
    static constexpr auto fn = chain_kernel<DT, NW>;
};
template <int DT>
struct ChainK2 {
    static constexpr auto fn = chain_kernel<DT, NW / 2>;
};
template <int DT>
struct ColK {
    static constexpr auto fn = colsum_kernel<DT>;
};

}  // namespace

hipError_t launch_prep128(const Mf128Args &a, hipStream_t st) {
    const int nblk = (a.T + W - 1) / W;
    const int64_t items = (int64_t)a.n_seqs_launch * (std::min(nblk, (a.t_hi + W - 1) / W) - a.t_lo / W) * a.H_v;
    const int blocks = (int)std::min<int64_t>((items + PW - 1) / PW, 16384);
    return launch(pick<PrepK>(a.dtype), a, blocks, 64 * PW, st);
}

hipError_t launch_fwd_mf(const Mf128Args &a, hipStream_t st) {
    const int units = a.n_seqs_launch * a.H_v;
    if (a.nslab == 2) return launch(pick<FwdK2>(a.dtype), a, 2 * units, NT / 2, st);
    return launch(pick<FwdK>(a.dtype), a, units, NT, st);
}

hipError_t launch_zero_anc(const Mf128Args &a, hipStream_t st) {
    // the two slabs of a unit add their segment dg into zeros
    if (a.nslab != 2) return hipSuccess;
    const int64_t units = (int64_t)a.n_seqs_launch * a.H_v;
    return launch_zero(a.anc + (int64_t)a.s_base * a.H_v * a.n_ck_max * S, units * a.n_ck_max * S, st);
}

hipError_t launch_zero_p3_all(const Mf128Args &a, hipStream_t st) {
    // the launch's sequences of the piece buffer's P3
    const int64_t units = (int64_t)a.n_seqs_launch * a.H_v;
    return launch_zero(a.p3buf + (int64_t)a.s_base * a.pb_T * a.H_v * S, units * a.pb_T * S, st);
}

hipError_t launch_zero_p3(const Mf128Args &a, hipStream_t st) {
    // the two slabs of a unit add their P3 into zeros
    return a.nslab == 2 ? launch_zero_p3_all(a, st) : hipSuccess;
}

hipError_t launch_chain(const Mf128Args &a, hipStream_t st) {
    const int units = a.n_seqs_launch * a.H_v;
    return a.nslab == 2 ? launch(pick<ChainK2>(a.dtype), a, 2 * units, NT / 2, st)
                        : launch(pick<ChainK>(a.dtype), a, units, NT, st);
}

hipError_t launch_colsum(const Mf128Args &a, hipStream_t st) {
    const int segs = (std::min(a.t_hi, a.T) + a.C - 1) / a.C - a.t_lo / a.C;
    return launch(pick<ColK>(a.dtype), a, a.n_seqs_launch * a.H_k * segs, NT, st);
}

}  // namespace gdn
