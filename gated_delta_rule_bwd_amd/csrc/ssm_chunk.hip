// ssm_chunk.hip -- gfx950 forward and backward of the selective scan with one decay per head
// (the Mamba-2 branch; page "S1-24: chunked attention", the SSM_SCAN_BACK commit notes and the
// n_group fold) in 32-token chunks on the fp32 matrix cores (v_mfma_f32_16x16x4f32).
//
// Per (sequence, head) and chunk of tokens t = 0..31 with steps d_t, log-decays l_t = d_t A and
// partial sums L_t = l_0 + ... + l_t, the state after token t is
//   s_t = e^{L_t} s_in + sum_{u <= t} e^{L_t - L_u} d_u x_u B_u^T,
// a closed form of the per-token recurrence, so its gradients are dense products over the chunk
// given the state s_in before the chunk (saved by the forward) and the gradient dS of the state
// after it.  With the gradient of s_u
//   G_u = sum_{t >= u} e^{L_t - L_u} gy_t C_t^T + w_u dS,   w_u = e^{L_31 - L_u},
// the outputs are dx_u = d_u G_u B_u, dB_u = d_u G_u^T x_u, dC_t = s_t^T gy_t and the gradient of
// the log-decay dl_u = <G_u, s_u> - d_u x_u . G_u B_u (ddt = A dl + x . G B, times softplus').
// With the Grams CB[t][u] = C_t . B_u, GX[t][u] = gy_t . x_u and the decay matrix
// D[t][u] = e^{L_t - L_u} for u <= t (0 above the diagonal):
//   G B = (D.CB)^T gy + diag(w) B dS^T
//   dB  = diag(d) (D.GX)^T C + diag(d w) x dS
//   dC  = (D.GX) diag(d) B + diag(e^L) gy s_in
//   dl_u = sum_{t >= u} Y_t + e^{L_31} <dS, s_in> + sum_{v < u <= t} Z[t][v] + sum_{v < u} R_v
// where Y_t = e^{L_t} C_t . (gy s_in)_t, Z = (D.GX) diag(d) . CB and R_v = d_v w_v x_v . (dS B_v):
// the terms of <G_u, s_u> in which token u's own decay takes part.  The chunk-end gradients come
// from a first pass that walks each head's chunks backwards, dS <- e^{L_31} dS + gy^T diag(e^L) C.
// The forward reads the closed form the other way: a pass walks the chunks forwards,
// s <- e^{L_31} s + (diag(d w) x)^T B, saving the state before each chunk, and then per chunk
// y = (D.CB) diag(d) x + diag(e^L) C s_in^T.
//
// Matrix-core operands: for a product over K = 16 q + 4 g + i (q: a 16-wide slice, g = lane / 16,
// i < 4), lane l supplies A[l % 16][K] and B[K][l % 16] in the i-th of four products, so an
// operand whose K runs along a row is one float4 per lane; D[4 (l / 16) + r][l % 16] is in
// register r.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gdn_internal.h"
#include "ssm_common.h"

namespace gdn {
namespace {

constexpr int Q = 32;            // tokens per chunk
constexpr int QW = Q / 8;        // 8-token windows of the forward's saved states per chunk

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ void st4(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }
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
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
// Inclusive prefix and suffix sums over lanes 0..31 (lanes 32..63 receive no meaningful value).
__device__ __forceinline__ float scan32(float v, int lane) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}
__device__ __forceinline__ float scan32_suffix(float v, int lane) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_down(v, o, 64);
        if (lane + o < 32) v += u;
    }
    return v;
}
// (the whole vector is bit-cast: bit-casting its elements one by one made this compiler load
// only the first dword)
__device__ __forceinline__ f4 bld4(Rsrc r, uint32_t vbytes, uint32_t sbytes) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, vbytes, sbytes, 0));
}

// Four consecutive floats; one 16-byte load when the address allows it.
__device__ __forceinline__ f4 ld4u(const float *p, bool vec) {
    return vec ? ld4(p) : f4{p[0], p[1], p[2], p[3]};
}

// ---- pass 1: the state gradient after every chunk ---------------------------------------
// One wave per (sequence, head, 16 rows of P, 64 columns of N) walks the chunks backwards and
// keeps its 16 x 64 slice of dS in four accumulator tiles: dsq[c] is the gradient of the state
// after chunk c, and after chunk 0 the gradient of the initial state is d_s0.  Column l % 16 of
// tile j is state 64 nh + 4 (l % 16) + j, so a lane reads the four states of its C operand, and
// writes its four tiles' values of a row, as one float4.  The chunks' inputs are loaded two
// chunks ahead.
template <int P, int N>
__global__ void __launch_bounds__(64) ssm_dsq_kernel(const SsmArgs a) {
    const int lane = threadIdx.x, ar = lane & 15, kg = lane >> 4;
    int64_t b = blockIdx.x;
    const int nh = (int)(b % (N / 64));
    b /= N / 64;
    const int pt = (int)(b % (P / 16));
    b /= P / 16;
    const int64_t T = a.T, H = a.H, G = a.G;
    const int64_t h = b % H, s = b / H, g = h / (H / G), unit = s * H + h;
    const int nc = (a.T + Q - 1) / Q;
    const float Ah = a.A[h];
    const int prow = 16 * pt + 4 * kg;   // rows of the lane's accumulator registers
    const int ncol = 64 * nh + 4 * ar;   // its four states (one per tile)
    f4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const f4 v = a.gs ? ld4(a.gs + (unit * P + prow + r) * N + ncol) : zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j][r] = v[j];
    }
    struct Ld {
        f4 c[8];
        float gy[8], dt;
    };
    // a chunk inside the sequence loads from wave-uniform token bases with fixed lane offsets
    // (lane rows 4 kg tokens down); the last one clamps its tokens to the sequence (masked at use)
    const int64_t HP = H * P, GN = G * N;
    const float *const gyb = a.gy + s * T * HP + h * P + 16 * pt, *const cb = a.C + s * T * GN + g * N + 64 * nh;
    const float *const dtb = a.dt + s * T * H + h;
    const uint32_t HP4 = (uint32_t)HP * 4, GN4 = (uint32_t)GN * 4, H4 = (uint32_t)H * 4;
    auto load = [&](int c, Ld &L) {
        // tokens past the end read the last one (masked at use)
        const int t0 = c * Q, last = a.T - 1 - t0;
        const Rsrc rg = rsrc(gyb + t0 * HP), rc = rsrc(cb + t0 * GN), rd = rsrc(dtb + t0 * H);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t tl = (uint32_t)min(16 * q + 4 * kg + i, last);
                L.gy[4 * q + i] = bld(rg, tl * HP4 + 4 * ar, 0);
                L.c[4 * q + i] = bld4(rc, tl * GN4 + 16 * ar, 0);
            }
        L.dt = bld(rd, (uint32_t)min(lane & 31, last) * H4, 0);
    };
    float *dsq = a.dsq + unit * nc * (int64_t)(P * N);
    auto step = [&](int c, const Ld &L) {
        float *o = dsq + (int64_t)c * P * N;
#pragma unroll
        for (int r = 0; r < 4; ++r) st4(o + (prow + r) * N + ncol, f4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]});
        const bool ok = lane < Q && c * Q + lane < a.T;
        const float l = ok ? ssm_step(L.dt, a.softplus) * Ah : 0.f;
        const float e = __expf(scan32(l, lane));
        const float elast = __shfl(e, Q - 1, 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= elast;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int kt = 16 * (k >> 2) + 4 * kg + (k & 3);
            const float ek = __shfl(e, kt, 64);   // every lane takes part in the shuffle
            // a token past the end adds nothing (its C is finite: a clamped in-range row)
            const float av = c * Q + kt < a.T ? L.gy[k] * ek : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = mfma(av, L.c[k][j], acc[j]);
        }
    };
    Ld L0, L1, L2;
    if (nc > 0) load(nc - 1, L0);
    if (nc > 1) load(nc - 2, L1);
    for (int c = nc - 1; c >= 0; c -= 3) {
        if (c >= 2) load(c - 2, L2);
        step(c, L0);
        if (c < 1) break;
        if (c >= 3) load(c - 3, L0);
        step(c - 1, L1);
        if (c < 2) break;
        if (c >= 4) load(c - 4, L1);
        step(c - 2, L2);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        st4(a.ds0 + (unit * P + prow + r) * N + ncol, f4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]});
}

// ---- pass 2: the chunks' gradients ------------------------------------------------------
// LDS rows are padded by 4 floats: the four row groups of a scalar operand read then fall in
// distinct banks, and so do the 16 rows of a float4 operand read.
struct ChunkLds {
    float Bc[Q][132], Cc[Q][132];            // the chunk's B and C rows of the group (0 past T)
    float xs[Q][68], gys[Q][68];             // the head's x and gy rows
    float M1T[Q][36], WdT[Q][36], Wd[Q][36]; // (D.CB)^T, ((D.GX) diag(d))^T, (D.GX) diag(d)
    float dS[64][132], sin[64][132];         // gradient after the chunk, state before it
    float sc[2][5][Q];                       // by head parity: d, L, e^L, w, softplus'
    float xgb[4][Q], rr[4][Q], yy[4][Q];     // per-wave-group parts of x.GB, R, Y
    float rowz[2][Q], colz[2][Q];            // strict row / column sums of Z per 16-wide tile
    float k0[2][8];                          // <dS, s_in> per wave, by head parity
};

// One workgroup of eight waves per (sequence, chunk, group, head slice) walks the slice's heads
// in increasing order and sums their dB and dC in its accumulators; the slices' sums are added
// by the combine kernel.  Wave w owns row tile ui = w & 1 (16 tokens) and column group
// grp = w >> 1 (16 elements of P in G B, 32 states of N in dB and dC); waves 0-2 also own the
// three nonzero 16 x 16 tiles of the chunk's Grams.  Per head: stage the head's rows in LDS, one
// barrier; Grams and the products with dS and s_in, one barrier; the products with the masked
// Grams and the row sums, one barrier; wave 0 then finishes ddt while the others stage the next
// head.
template <int P, int N>
__global__ void __launch_bounds__(512) ssm_chunk_kernel(const SsmArgs a) {
    static_assert(P == 64 && N == 128, "tile assignment of this kernel");
    __shared__ ChunkLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ar = lane & 15, kg = lane >> 4;
    const int64_t T = a.T, H = a.H, G = a.G;
    const int nc = (a.T + Q - 1) / Q;
    int64_t b = blockIdx.x;
    const int hsl = (int)(b % a.hgs);
    b /= a.hgs;
    const int64_t g = b % G;
    b /= G;
    const int c = (int)(b % nc);
    const int64_t s = b / nc;
    const int t0 = c * Q;
    const int Hg = a.H / a.G, hper = (Hg + a.hgs - 1) / a.hgs;
    const int h_lo = (int)g * Hg + std::min(Hg, hsl * hper);
    const int h_hi = (int)g * Hg + std::min(Hg, (hsl + 1) * hper);
    const int ui = wv & 1, grp = wv >> 1;
    const bool vec = (((uintptr_t)a.x | (uintptr_t)a.gy) & 15) == 0;

    // the chunk's B and C rows, and the tile sums no Gram tile writes
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int e = tid + 512 * m, row = e >> 5, c4 = e & 31;
        const int t = t0 + row;
        const bool ok = t < a.T;
        const int64_t off = ((s * T + (ok ? t : T - 1)) * G + g) * N + 4 * c4;
        const f4 bv = ld4(a.B + off), cv = ld4(a.C + off);
        st4(&sm.Bc[row][4 * c4], ok ? bv : zero4());
        st4(&sm.Cc[row][4 * c4], ok ? cv : zero4());
    }
    if (tid < 16) {
        sm.rowz[1][tid] = 0.f;
        sm.colz[0][16 + tid] = 0.f;
    }

    struct Pf {
        f4 x, gy, ds[4], si[4];
        float dt;
    };
    auto fetch = [&](int64_t h, Pf &F) {
        {
            const int row = tid >> 4, c4 = tid & 15;
            const int64_t off = ((s * T + std::min(t0 + row, a.T - 1)) * H + h) * P + 4 * c4;
            F.x = ld4u(a.x + off, vec);    // rows past the end are zeroed when staged
            F.gy = ld4u(a.gy + off, vec);
        }
        const float *dsp = a.dsq + ((s * H + h) * nc + c) * (int64_t)(P * N);
        const float *sip = a.ck + (s * H + h) * P * (int64_t)a.nck * N + (int64_t)(c * QW / a.ckw) * N;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 512 * m, p = e >> 5, c4 = e & 31;
            F.ds[m] = ld4(dsp + p * N + 4 * c4);
            F.si[m] = ld4(sip + (int64_t)p * a.nck * N + 4 * c4);
        }
        F.dt = a.dt[(s * T + std::min(t0 + (lane & 31), a.T - 1)) * H + h];
    };
    auto put = [&](const Pf &F, int par, float Ah) {
        {
            const int row = tid >> 4, c4 = tid & 15;
            const bool ok = t0 + row < a.T;
            st4(&sm.xs[row][4 * c4], ok ? F.x : zero4());
            st4(&sm.gys[row][4 * c4], ok ? F.gy : zero4());
        }
        float k0 = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 512 * m, p = e >> 5, c4 = e & 31;
            st4(&sm.dS[p][4 * c4], F.ds[m]);
            st4(&sm.sin[p][4 * c4], F.si[m]);
#pragma unroll
            for (int i = 0; i < 4; ++i) k0 = fmaf(F.ds[m][i], F.si[m][i], k0);
        }
        k0 = wave_sum(k0);
        if (lane == 0) sm.k0[par][wv] = k0;
        if (wv == 0) {
            const bool ok = lane < Q && t0 + lane < a.T;
            const float d = ok ? ssm_step(F.dt, a.softplus) : 0.f;
            const float L = scan32(d * Ah, lane);
            const float last = __shfl(L, Q - 1, 64);
            if (lane < Q) {
                sm.sc[par][0][lane] = d;
                sm.sc[par][1][lane] = L;
                sm.sc[par][2][lane] = __expf(L);
                sm.sc[par][3][lane] = __expf(last - L);
                sm.sc[par][4][lane] = a.softplus ? 1.f / (1.f + expf(-F.dt)) : 1.f;
            }
        }
    };

    f4 dBa[2] = {zero4(), zero4()}, dCa[2] = {zero4(), zero4()}, cb = zero4();
    const int ti = wv > 0 ? 1 : 0, tj = wv > 1 ? 1 : 0;   // Gram tile of waves 0-2
    Pf F;
    if (h_lo < h_hi) fetch(h_lo, F);
    for (int h = h_lo; h < h_hi; ++h) {
        const int par = (h - h_lo) & 1;
        const float Ah = a.A[h];
        put(F, par, Ah);
        __syncthreads();
        if (h + 1 < h_hi) fetch(h + 1, F);
        const float(*sc)[Q] = sm.sc[par];

        // ---- Grams, decay masks and the products with dS and s_in
        if (wv < 3) {
            if (h == h_lo) {   // CB is common to the slice's heads
#pragma unroll
                for (int q = 0; q < N / 16; ++q) {
                    const f4 af = ld4(&sm.Cc[16 * ti + ar][16 * q + 4 * kg]);
                    const f4 bf = ld4(&sm.Bc[16 * tj + ar][16 * q + 4 * kg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) cb = mfma(af[i], bf[i], cb);
                }
            }
            f4 gx = zero4();
#pragma unroll
            for (int q = 0; q < P / 16; ++q) {
                const f4 af = ld4(&sm.gys[16 * ti + ar][16 * q + 4 * kg]);
                const f4 bf = ld4(&sm.xs[16 * tj + ar][16 * q + 4 * kg]);
#pragma unroll
                for (int i = 0; i < 4; ++i) gx = mfma(af[i], bf[i], gx);
            }
            const int u = 16 * tj + ar;
            const float du = sc[0][u], lu = sc[1][u];
            f4 m1, wd;
            float cz = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ti + 4 * kg + r;
                const float dm = u <= t ? __expf(sc[1][t] - lu) : 0.f;
                m1[r] = dm * cb[r];
                wd[r] = dm * gx[r] * du;
                sm.Wd[t][u] = wd[r];
                const float z = u < t ? wd[r] * cb[r] : 0.f;
                const float zr = row16_sum(z);
                if (ar == 0) sm.rowz[tj][t] = zr;
                cz += z;
            }
            st4(&sm.M1T[u][16 * ti + 4 * kg], m1);
            st4(&sm.WdT[u][16 * ti + 4 * kg], wd);
            cz += __shfl_xor(cz, 16, 64);
            cz += __shfl_xor(cz, 32, 64);
            if (kg == 0) sm.colz[ti][u] = cz;
        }
        f4 gbe = zero4();   // (B dS^T)[u][p]
#pragma unroll
        for (int q = 0; q < N / 16; ++q) {
            const f4 af = ld4(&sm.Bc[16 * ui + ar][16 * q + 4 * kg]);
            const f4 bf = ld4(&sm.dS[16 * grp + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) gbe = mfma(af[i], bf[i], gbe);
        }
        {   // dB += diag(d w) x dS
            const int u = 16 * ui + ar;
            const float f = sc[0][u] * sc[3][u];
#pragma unroll
            for (int q = 0; q < P / 16; ++q) {
                const f4 af = ld4(&sm.xs[u][16 * q + 4 * kg]) * f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = 16 * q + 4 * kg + i;
#pragma unroll
                    for (int j = 0; j < 2; ++j) dBa[j] = mfma(af[i], sm.dS[p][32 * grp + 16 * j + ar], dBa[j]);
                }
            }
        }
        f4 dci[2] = {zero4(), zero4()};   // (gy s_in)[t][n]
#pragma unroll
        for (int q = 0; q < P / 16; ++q) {
            const f4 af = ld4(&sm.gys[16 * ui + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 16 * q + 4 * kg + i;
#pragma unroll
                for (int j = 0; j < 2; ++j) dci[j] = mfma(af[i], sm.sin[p][32 * grp + 16 * j + ar], dci[j]);
            }
        }
        __syncthreads();

        // ---- products with the masked Grams (K limited to the nonzero tiles)
        f4 gbi = zero4();   // ((D.CB)^T gy)[u][p]
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (q < ui) continue;
            const f4 af = ld4(&sm.M1T[16 * ui + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) gbi = mfma(af[i], sm.gys[16 * q + 4 * kg + i][16 * grp + ar], gbi);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {   // dB += (D.GX diag(d))^T C
            if (q < ui) continue;
            const f4 af = ld4(&sm.WdT[16 * ui + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * q + 4 * kg + i;
#pragma unroll
                for (int j = 0; j < 2; ++j) dBa[j] = mfma(af[i], sm.Cc[t][32 * grp + 16 * j + ar], dBa[j]);
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {   // dC += (D.GX diag(d)) B
            if (q > ui) continue;
            const f4 af = ld4(&sm.Wd[16 * ui + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = 16 * q + 4 * kg + i;
#pragma unroll
                for (int j = 0; j < 2; ++j) dCa[j] = mfma(af[i], sm.Bc[u][32 * grp + 16 * j + ar], dCa[j]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {   // dx, and the rows' x . G B and R
            const int u = 16 * ui + 4 * kg + r;
            const float du = sc[0][u];
            const float ge = sc[3][u] * gbe[r], gb = gbi[r] + ge;
            if (t0 + u < a.T) a.dx[((s * T + t0 + u) * H + h) * P + 16 * grp + ar] = du * gb;
            const float xv = sm.xs[u][16 * grp + ar];
            const float s1 = row16_sum(xv * gb), s2 = row16_sum(xv * ge);
            if (ar == 0) {
                sm.xgb[grp][u] = s1;
                sm.rr[grp][u] = du * s2;
            }
        }
        {   // dC += diag(e^L) gy s_in, and the rows' Y
            float yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ui + 4 * kg + r;
                    const float v = dci[j][r] * sc[2][t];
                    dCa[j][r] += v;
                    yv[r] = fmaf(sm.Cc[t][32 * grp + 16 * j + ar], v, yv[r]);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ys = row16_sum(yv[r]);
                if (ar == 0) sm.yy[grp][16 * ui + 4 * kg + r] = ys;
            }
        }
        __syncthreads();

        // ---- ddt of the head's tokens (wave 0; the others go on to stage the next head)
        if (wv == 0) {
            const int u = lane & 31;
            const float xgb = ((sm.xgb[0][u] + sm.xgb[1][u]) + sm.xgb[2][u]) + sm.xgb[3][u];
            const float R = ((sm.rr[0][u] + sm.rr[1][u]) + sm.rr[2][u]) + sm.rr[3][u];
            const float Y = ((sm.yy[0][u] + sm.yy[1][u]) + sm.yy[2][u]) + sm.yy[3][u];
            const float dz = (sm.colz[0][u] + sm.colz[1][u]) - (sm.rowz[0][u] + sm.rowz[1][u]);
            float k0 = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) k0 += sm.k0[par][w];
            k0 *= sc[2][Q - 1];
            const float ysuf = scan32_suffix(Y, lane);
            float ze = __shfl_up(scan32(dz, lane), 1, 64), re = __shfl_up(scan32(R, lane), 1, 64);
            if (lane == 0) ze = re = 0.f;
            const float dl = ((ysuf + k0) + ze) + re;
            const float dd = fmaf(Ah, dl, xgb) * sc[4][u];
            if (lane < Q && t0 + lane < a.T) a.ddt[(s * T + t0 + lane) * H + h] = dd;
        }
    }

    // the slice's dB and dC (zero for a slice without heads)
    const int64_t plane = (int64_t)a.n_seqs * T * G * N;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * ui + 4 * kg + r;
        if (t < a.T) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t o = ((s * T + t) * G + g) * N + 32 * grp + 16 * j + ar;
                a.cpart[2 * hsl * plane + o] = dBa[j][r];
                a.cpart[(2 * hsl + 1) * plane + o] = dCa[j][r];
            }
        }
    }
}

// ---- pass 3: dB and dC, the head slices added in increasing order ------------------------
__global__ void __launch_bounds__(256) ssm_chunk_combine_kernel(const SsmArgs a) {
    const int64_t plane = (int64_t)a.n_seqs * a.T * a.G * a.N, n4 = plane / 4;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < 2 * n4;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int which = idx >= n4;
        const int64_t o = 4 * (idx - which * n4);
        f4 acc = zero4();
        for (int j = 0; j < a.hgs; ++j) acc += ld4(a.cpart + (2 * j + which) * plane + o);
        float *dst = (which ? a.dC : a.dB) + o;   // the packed gradient: 4-byte alignment only
        dst[0] = acc[0]; dst[1] = acc[1]; dst[2] = acc[2]; dst[3] = acc[3];
    }
}

// ---- forward: the state before every chunk, then the chunks' outputs --------------------
// Pass 1: one wave per (sequence, head, 16 rows of P, 64 states) walks the chunks in order with
// its slice of the state in four accumulator tiles, saves the state before every chunk (for the
// output pass and the backward) and updates s <- e^{L_31} s + (diag(d w) x)^T B over the chunk
// (w_u = e^{L_31 - L_u}); after the last chunk it is the final state.  Tokens past the end have
// step 0, so they add nothing.  The lane layout is that of the chunk-end gradient pass.
template <int P, int N>
__global__ void __launch_bounds__(64) ssm_fst_kernel(const SsmArgs a) {
    const int lane = threadIdx.x, ar = lane & 15, kg = lane >> 4;
    int64_t b = blockIdx.x;
    const int nh = (int)(b % (N / 64));
    b /= N / 64;
    const int pt = (int)(b % (P / 16));
    b /= P / 16;
    const int64_t T = a.T, H = a.H, G = a.G;
    const int64_t h = b % H, s = b / H, g = h / (H / G), unit = s * H + h;
    const int nc = (a.T + Q - 1) / Q;
    const float Ah = a.A[h];
    const int prow = 16 * pt + 4 * kg;
    const int ncol = 64 * nh + 4 * ar;
    f4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const f4 v = ld4(a.s0 + (unit * P + prow + r) * N + ncol);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j][r] = v[j];
    }
    struct Ld {
        f4 b[8];
        float x[8], dt;
    };
    // as in the chunk-end pass: uniform token bases with fixed lane offsets inside the sequence,
    // clamped tokens (step 0 past the end) in its last chunk
    const int64_t HP = H * P, GN = G * N;
    const float *const xb = a.x + s * T * HP + h * P + 16 * pt, *const bb = a.B + s * T * GN + g * N + 64 * nh;
    const float *const dtb = a.dt + s * T * H + h;
    const uint32_t HP4 = (uint32_t)HP * 4, GN4 = (uint32_t)GN * 4, H4 = (uint32_t)H * 4;
    auto load = [&](int c, Ld &L) {
        // tokens past the end read the last one (their step is 0)
        const int t0 = c * Q, last = a.T - 1 - t0;
        const Rsrc rx = rsrc(xb + t0 * HP), rb = rsrc(bb + t0 * GN), rd = rsrc(dtb + t0 * H);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t tl = (uint32_t)min(16 * q + 4 * kg + i, last);
                L.x[4 * q + i] = bld(rx, tl * HP4 + 4 * ar, 0);
                L.b[4 * q + i] = bld4(rb, tl * GN4 + 16 * ar, 0);
            }
        L.dt = bld(rd, (uint32_t)min(lane & 31, last) * H4, 0);
    };
    float *ckp = a.ck + unit * P * (int64_t)a.nck * N;
    auto step = [&](int c, const Ld &L) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st4(ckp + ((int64_t)(prow + r) * a.nck + c * QW / a.ckw) * N + ncol,
                f4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]});
        const bool ok = lane < Q && c * Q + lane < a.T;
        const float d = ok ? ssm_step(L.dt, a.softplus) : 0.f;
        const float lam = scan32(d * Ah, lane);
        const float last = __shfl(lam, Q - 1, 64);
        const float dw = d * __expf(last - lam);
        const float elast = __expf(last);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= elast;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float av = L.x[k] * __shfl(dw, 16 * (k >> 2) + 4 * kg + (k & 3), 64);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = mfma(av, L.b[k][j], acc[j]);
        }
    };
    Ld L0, L1, L2;
    if (nc > 0) load(0, L0);
    if (nc > 1) load(1, L1);
    for (int c = 0; c < nc; c += 3) {
        if (c + 2 < nc) load(c + 2, L2);
        step(c, L0);
        if (c + 1 >= nc) break;
        if (c + 3 < nc) load(c + 3, L0);
        step(c + 1, L1);
        if (c + 2 >= nc) break;
        if (c + 4 < nc) load(c + 4, L1);
        step(c + 2, L2);
    }
    if (a.s_out) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st4(a.s_out + (unit * P + prow + r) * N + ncol, f4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]});
    }
}

// Pass 2: one 512-thread workgroup per (sequence, chunk, group, head slice); per head
//   y = (D.CB) diag(d) x + diag(e^L) C s_in^T,
// wave w owning the 16 x 16 tile (tokens 16 (w & 1), elements 16 (w >> 1)) of y; CB is formed
// once per chunk on waves 0-2 (its B rows' LDS then holds the head's d x and D.CB).
struct FwdLds {
    float Cc[Q][132];
    float sin[64][132];
    union {
        float Bc[Q][132];
        struct {
            float xs[Q][68];       // d_u x_u
            float M1[Q][36];       // (D.CB)[t][u]
        } hd;
    } u;
    float L[Q], eL[Q];
};

template <int P, int N>
__global__ void __launch_bounds__(512) ssm_chunk_fwd_kernel(const SsmArgs a) {
    static_assert(P == 64 && N == 128, "tile assignment of this kernel");
    __shared__ FwdLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, ar = lane & 15, kg = lane >> 4;
    const int64_t T = a.T, H = a.H, G = a.G;
    const int nc = (a.T + Q - 1) / Q;
    int64_t b = blockIdx.x;
    const int hsl = (int)(b % a.hgs);
    b /= a.hgs;
    const int64_t g = b % G;
    b /= G;
    const int c = (int)(b % nc);
    const int64_t s = b / nc;
    const int t0 = c * Q;
    const int Hg = a.H / a.G, hper = (Hg + a.hgs - 1) / a.hgs;
    const int h_lo = (int)g * Hg + std::min(Hg, hsl * hper);
    const int h_hi = (int)g * Hg + std::min(Hg, (hsl + 1) * hper);
    if (h_lo >= h_hi) return;
    const int ti = wv & 1, pj = wv >> 1;
    const bool vec = ((uintptr_t)a.x & 15) == 0;

#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int e = tid + 512 * m, row = e >> 5, c4 = e & 31;
        const bool ok = t0 + row < a.T;
        const int64_t off = ((s * T + std::min(t0 + row, a.T - 1)) * G + g) * N + 4 * c4;
        const f4 bv = ld4(a.B + off), cv = ld4(a.C + off);
        st4(&sm.u.Bc[row][4 * c4], ok ? bv : zero4());
        st4(&sm.Cc[row][4 * c4], ok ? cv : zero4());
    }
    __syncthreads();
    const int gi = wv > 0 ? 1 : 0, gj = wv > 1 ? 1 : 0;   // CB tile of waves 0-2
    f4 cb = zero4();
    if (wv < 3) {
#pragma unroll
        for (int q = 0; q < N / 16; ++q) {
            const f4 af = ld4(&sm.Cc[16 * gi + ar][16 * q + 4 * kg]);
            const f4 bf = ld4(&sm.u.Bc[16 * gj + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) cb = mfma(af[i], bf[i], cb);
        }
    }
    __syncthreads();   // the B rows' LDS is the heads' from here on

    struct Pf {
        f4 x, si[4];
        float dt, dtl;
    };
    auto fetch = [&](int64_t h, Pf &F) {
        const int row = tid >> 4, c4 = tid & 15;
        const int64_t tc = std::min(t0 + row, a.T - 1);
        F.x = ld4u(a.x + ((s * T + tc) * H + h) * P + 4 * c4, vec);
        F.dt = a.dt[(s * T + tc) * H + h];
        F.dtl = a.dt[(s * T + std::min(t0 + (lane & 31), a.T - 1)) * H + h];
        const float *sip = a.ck + (s * H + h) * P * (int64_t)a.nck * N + (int64_t)(c * QW / a.ckw) * N;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 512 * m, p = e >> 5, c4b = e & 31;
            F.si[m] = ld4(sip + (int64_t)p * a.nck * N + 4 * c4b);
        }
    };
    Pf F;
    fetch(h_lo, F);
    for (int h = h_lo; h < h_hi; ++h) {
        const float Ah = a.A[h];
        {
            const int row = tid >> 4, c4 = tid & 15;
            const bool ok = t0 + row < a.T;
            const float d = ok ? ssm_step(F.dt, a.softplus) : 0.f;
            st4(&sm.u.hd.xs[row][4 * c4], F.x * d);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = tid + 512 * m, p = e >> 5, c4b = e & 31;
                st4(&sm.sin[p][4 * c4b], F.si[m]);
            }
            if (wv == 0) {
                const bool okl = lane < Q && t0 + lane < a.T;
                const float dl = okl ? ssm_step(F.dtl, a.softplus) : 0.f;
                const float L = scan32(dl * Ah, lane);
                if (lane < Q) {
                    sm.L[lane] = L;
                    sm.eL[lane] = __expf(L);
                }
            }
        }
        __syncthreads();
        if (h + 1 < h_hi) fetch(h + 1, F);
        if (wv < 3) {   // D.CB on the three nonzero tiles
            const int u = 16 * gj + ar;
            const float lu = sm.L[u];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * gi + 4 * kg + r;
                sm.u.hd.M1[t][u] = u <= t ? __expf(sm.L[t] - lu) * cb[r] : 0.f;
            }
        }
        __syncthreads();
        f4 yi = zero4(), ye = zero4();
#pragma unroll
        for (int q = 0; q < 2; ++q) {   // (D.CB) (d x): u below the tile's last token
            if (q > ti) continue;
            const f4 af = ld4(&sm.u.hd.M1[16 * ti + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) yi = mfma(af[i], sm.u.hd.xs[16 * q + 4 * kg + i][16 * pj + ar], yi);
        }
#pragma unroll
        for (int q = 0; q < N / 16; ++q) {   // C s_in^T
            const f4 af = ld4(&sm.Cc[16 * ti + ar][16 * q + 4 * kg]);
            const f4 bf = ld4(&sm.sin[16 * pj + ar][16 * q + 4 * kg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) ye = mfma(af[i], bf[i], ye);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * ti + 4 * kg + r;
            if (t0 + t < a.T) a.y[((s * T + t0 + t) * H + h) * P + 16 * pj + ar] = fmaf(sm.eL[t], ye[r], yi[r]);
        }
        __syncthreads();
    }
}

}  // namespace

// The chunk walks address 32 tokens of a head's rows and of a group's B/C rows with 32-bit byte
// offsets from the chunk's first token, so a token's stride stays at most 2^24 floats.
bool ssm_chunked(int P, int N, int aps, int64_t H, int64_t G) {
    return aps == 0 && P == 64 && N == 128 && H * P <= (int64_t(1) << 24) && G * N <= (int64_t(1) << 24);
}

hipError_t launch_ssm_chunk_fwd(const SsmArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.n_seqs * a.H;
    if (units <= 0) return hipSuccess;
    if (!ssm_chunked(a.P, a.N, a.aps, a.H, a.G) || a.hgs < 1 || a.H % a.G != 0 || QW % a.ckw != 0)
        return hipErrorInvalidValue;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    hipError_t e = hipLaunchKernel((const void *)ssm_fst_kernel<64, 128>, dim3((unsigned)(units * (64 / 16) * (128 / 64))),
                                   dim3(64), params, 0, st);
    const int64_t nc = (a.T + Q - 1) / Q;
    const int64_t nwg = (int64_t)a.n_seqs * nc * a.G * a.hgs;
    if (e == hipSuccess && a.y && nwg > 0)
        e = hipLaunchKernel((const void *)ssm_chunk_fwd_kernel<64, 128>, dim3((unsigned)nwg), dim3(512), params, 0, st);
    return e;
}

hipError_t launch_ssm_chunk_bwd(const SsmArgs &a, hipStream_t st) {
    const int64_t units = (int64_t)a.n_seqs * a.H;
    if (units <= 0) return hipSuccess;
    if (!ssm_chunked(a.P, a.N, a.aps, a.H, a.G) || a.hgs < 1 || a.H % a.G != 0 || QW % a.ckw != 0)
        return hipErrorInvalidValue;
    void *params[] = {const_cast<SsmArgs *>(&a)};
    hipError_t e = hipLaunchKernel((const void *)ssm_dsq_kernel<64, 128>, dim3((unsigned)(units * (64 / 16) * (128 / 64))),
                                   dim3(64), params, 0, st);
    const int64_t nc = (a.T + Q - 1) / Q;
    const int64_t nwg = (int64_t)a.n_seqs * nc * a.G * a.hgs;
    if (e == hipSuccess && nwg > 0)
        e = hipLaunchKernel((const void *)ssm_chunk_kernel<64, 128>, dim3((unsigned)nwg), dim3(512), params, 0, st);
    const int64_t n4 = (int64_t)a.n_seqs * a.T * a.G * a.N / 4;
    if (e == hipSuccess && n4 > 0) {
        const int64_t blocks = std::min<int64_t>((2 * n4 + 255) / 256, 65535);
        e = hipLaunchKernel((const void *)ssm_chunk_combine_kernel, dim3((unsigned)blocks), dim3(256), params, 0, st);
    }
    return e;
}

}  // namespace gdn
