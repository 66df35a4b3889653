// ssm_conv.hip -- gfx950 kernels of the short causal depthwise convolution upstream of the
// gated delta rule and of its backward with respect to the input (page "S1-24: chunked
// attention -- the kernel-free long-context path", the commit notes on SSM_CONV_BACK).
//
// Layouts (channels innermost, so a token's channels are contiguous):
//   sx, d_sx [n_seqs][d_conv - 1 + T][d_inner]  (carried state rows first)
//   c        [d_inner][d_conv]
//   y, dy    [n_seqs][T][d_inner]
//   y[s][t][i]    = sum_j sx[s][t + j][i] c[i][j]
//   d_sx[s][u][i] = sum over taps j with 0 <= u - j < T of dy[s][u - j][i] c[i][j]
// The backward is computed as that gather (one owner per output element, taps in increasing
// j, no atomics), which equals the page's scatter term by term.  Both kernels are HBM-bound:
// a thread owns V consecutive channels of R consecutive rows and keeps the d_conv - 1 rows
// its window needs beyond them in registers (vector loads and stores of V = 4 channels when
// every row start is 16-byte aligned).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int RR = 8;     // rows per thread

template <int V>
__device__ __forceinline__ void ld(const float *p, float (&x)[V]) {
    if constexpr (V == 4) {
        const float4 t = *reinterpret_cast<const float4 *>(p);
        x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else {
        x[0] = *p;
    }
}
// Outputs are written once and not read back by the kernel: nontemporal stores keep them from
// displacing the input rows that neighbouring row blocks re-read through L2 (the loads stay
// ordinary for that reason).
typedef float f4v __attribute__((ext_vector_type(4)));
template <int V>
__device__ __forceinline__ void st(float *p, const float (&x)[V]) {
    if constexpr (V == 4) __builtin_nontemporal_store(f4v{x[0], x[1], x[2], x[3]}, reinterpret_cast<f4v *>(p));
    else __builtin_nontemporal_store(x[0], p);
}

// Forward: out = y (rows_out = T), in = sx (rows_in = T + K - 1), out[r] = sum_j in[r + j] w[j].
// Backward: out = d_sx (rows_out = T + K - 1), in = dy (rows_in = T),
// out[r] = sum_j in[r - j] w[j] over the rows r - j that exist.
template <int V, int K, bool BWD>
__global__ void __launch_bounds__(256) conv_kernel(const ConvArgs a) {
    constexpr int OFF = BWD ? K - 1 : 0;   // first input row of a thread's window, relative
    const int64_t groups = a.d_inner / V;
    const int64_t rblocks = (a.rows_out + RR - 1) / RR;
    const int64_t total = (int64_t)a.n_seqs * rblocks * groups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t gi = idx % groups, rest = idx / groups;
        const int64_t rb = rest % rblocks, s = rest / rblocks;
        const int i = (int)gi * V;
        const int r0 = (int)rb * RR;
        // taps of the V channels
        float w[K][V];
#pragma unroll
        for (int c = 0; c < V; ++c)
#pragma unroll
            for (int j = 0; j < K; ++j) w[j][c] = a.w[(int64_t)(i + c) * K + j];
        const float *in = a.in + s * a.in_seq + i;
        float *out = a.out + s * a.out_seq + i;
        // the input rows the R outputs read: r0 - OFF .. r0 - OFF + R + K - 2; rows outside
        // the input contribute nothing (loads clamped to a valid row, then zeroed: no branch)
        float x[RR + K - 1][V];
#pragma unroll
        for (int m = 0; m < RR + K - 1; ++m) {
            const int row = r0 - OFF + m;
            const bool in_range = row >= 0 && row < a.rows_in;
            if (a.rows_in > 0) ld<V>(in + (int64_t)min(max(row, 0), a.rows_in - 1) * a.in_tok, x[m]);
#pragma unroll
            for (int c = 0; c < V; ++c) x[m][c] = in_range ? x[m][c] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < RR; ++m) {
            const int r = r0 + m;
            if (r >= a.rows_out) break;
            float y[V];
#pragma unroll
            for (int c = 0; c < V; ++c) {
                float acc = 0.f;
                // forward: taps j in increasing order read rows r + j; backward: tap j reads
                // row r - j, i.e. x[m + K - 1 - j]; both sum j = 0 .. K - 1 in order
#pragma unroll
                for (int j = 0; j < K; ++j) acc = fmaf(BWD ? x[m + K - 1 - j][c] : x[m + j][c], w[j][c], acc);
                y[c] = acc;
            }
            st<V>(out + (int64_t)r * a.out_tok, y);
        }
    }
}

template <int V, bool BWD>
hipError_t launch_k(const ConvArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.n_seqs * ((a.rows_out + RR - 1) / RR) * (a.d_inner / V);
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65535) blocks = 65535;
    void *params[] = {const_cast<ConvArgs *>(&a)};
    const void *fn = nullptr;
    switch (a.d_conv) {
#define GDN_K(k) case k: fn = (const void *)conv_kernel<V, k, BWD>; break;
        GDN_K(1) GDN_K(2) GDN_K(3) GDN_K(4) GDN_K(5) GDN_K(6) GDN_K(7) GDN_K(8)
#undef GDN_K
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), params, 0, st);
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, bool bwd, hipStream_t st) {
    const bool vec = a.d_inner % 4 == 0 && ((uintptr_t)a.in & 15) == 0 && ((uintptr_t)a.out & 15) == 0 &&
                     a.in_seq % 4 == 0 && a.in_tok % 4 == 0 && a.out_seq % 4 == 0 && a.out_tok % 4 == 0;
    if (bwd) return vec ? launch_k<4, true>(a, st) : launch_k<1, true>(a, st);
    return vec ? launch_k<4, false>(a, st) : launch_k<1, false>(a, st);
}

}  // namespace gdn
