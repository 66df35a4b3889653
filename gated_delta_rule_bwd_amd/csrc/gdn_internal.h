// gdn_internal.h -- argument blocks shared by the host side of the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Sequences handled by one launch; their lengths travel in the kernel argument block.
constexpr int kMaxSeqsPerLaunch = 256;
// Pieces of the token axis in the pipelined head-128 passes.
constexpr int kMaxPieces = 16;

// Arguments of the forward scan (also used, with y == nullptr, as the checkpoint pass
// of the backward).
struct FwdArgs {
    const float *q, *k, *v, *g, *beta, *state0;
    float *y;          // nullptr: do not write y
    float *state_out;  // nullptr: do not write the final state
    float *snap;       // [unit][n_ck_max][S][S] snapshots (state before tokens 0, C, 2C, ...)
    gdn_strides sq, sk, sv, sg, sb, sy;
    int32_t s_base;    // first sequence of this launch
    int32_t T, H_k, H_v, C, n_ck_max;
    float scale;
    int32_t dtype;     // always fp32 here (half inputs are widened first)
    int32_t lens[kMaxSeqsPerLaunch];
};

// Arguments of the backward walk.
struct BwdArgs {
    const float *q, *k, *v, *g, *beta, *gy, *dstate_out;
    const float *snap;  // [unit][n_ck_max][S][S]
    float *segbuf;      // S < 128: [unit][C][S][S] decayed previous state Mp of each segment token
    float *ebuf_seg;    // S < 128: [unit][C][S] prediction errors v - u of the current segment
    float *dq, *dk;     // direct outputs (H_v == H_k) or per-value-head partials
    int64_t dqk_head;   // head count of the dq/dk arrays (H_k direct, H_v for partials)
    float *dv, *dg, *dbeta, *dstate;
    gdn_strides sq, sk, sv, sg, sb, sgy;
    int32_t s_base;
    int32_t T, H_k, H_v, C, n_ck_max;
    float scale;
    int32_t dtype;      // always fp32 here
    int32_t lens[kMaxSeqsPerLaunch];
};

// Sum of the value heads of each key head (fixed increasing order) for dq and dk.
struct CombineArgs {
    const float *dq_part, *dk_part;  // [n_seqs][T][H_v][S] (S: the key width)
    float *dq, *dk;                  // [n_seqs][T][H_k][S]
    int32_t n_seqs, T, H_k, H_v, S;
};

// Exact widening of a strided half-precision per-token tensor [n][T][H][W] (IEEE binary16,
// or bfloat16 when bf16 != 0) into a contiguous fp32 copy.
struct WidenArgs {
    const uint16_t *src;
    gdn_strides st;
    float *dst;
    int64_t n, T, H, W;
    int32_t bf16;
};

hipError_t launch_widen(const WidenArgs &a, hipStream_t st);

// Short causal depthwise convolution (forward) or its input gradient (backward), over
// channel-innermost rows; in/out row counts and strides in floats (see ssm_conv.hip).
struct ConvArgs {
    const float *in, *w;   // input rows; taps [d_inner][d_conv]
    float *out;
    int64_t in_seq, in_tok, out_seq, out_tok;
    int32_t n_seqs, rows_in, rows_out, d_inner, d_conv;
};
hipError_t launch_conv(const ConvArgs &a, bool bwd, hipStream_t st);

// L2 normalisation of rows [n_seqs][T][H] of W floats (forward: out = x / n) or its backward
// (out = dy / n - x (x . dy) / n^3), n = sqrt(sum x^2 + eps); 1 <= W <= 1024 (see l2norm.hip).
struct NormArgs {
    const float *x, *dy;   // dy: backward only
    float *out;
    gdn_strides sx, sdy, so;
    int32_t n_seqs, T, H, W;
    float eps;
};
hipError_t launch_l2norm(const NormArgs &a, bool bwd, hipStream_t st);

// Selective state-space scan and its reverse recurrence (see ssm_scan.hip, ssm_chunk.hip).
// Contiguous tensors: s0/s_out/ds0 [n][H][P][N], x/y/gy/dx/ddrow [n][T][H][P], dt/ddt [n][T][H],
// A [H][N] (aps) or [H], B/C/dB/dC [n][T][G][N]; workspace: ck [rows][nck][N] (the state before
// every ckw-th 8-token window); for the per-token backward part [rows/seg_rows][T][2][N] and
// ddrow, the row-wise one also gsw [rows][ceil(T/8)][N] (the state gradient entering each
// window from the right); for the chunked backward dsq [n][H][ceil(T/32)][P][N] (the state
// gradient after each 32-token chunk) and cpart [hgs][2][n][T][G][N] (dB, dC per head slice).
struct SsmArgs {
    const float *s0, *x, *dt, *A, *B, *C, *gy, *gs;
    float *ck, *part, *ddrow, *dsq, *cpart, *gsw;
    float *y, *s_out, *ds0, *dx, *ddt, *dB, *dC;
    int32_t n_seqs, T, H, P, N, G, aps, softplus;
    int32_t ckw, nck;   // windows per saved state (1, or 4 for the chunked backward); states per row
    int32_t hgs;        // head slices per group in the chunked backward
    int32_t seg_rows;   // rows per column-sum segment of part (16, or 256 in the row-wise backward)
};
hipError_t launch_ssm(const SsmArgs &a, bool bwd, hipStream_t st);   // forward or walk
hipError_t launch_ssm_combine(const SsmArgs &a, hipStream_t st);
// Chunked backward (one decay per head, P = 64, N = 128, H P and G N at most 2^24): the chunk-end
// state gradients, the chunks' gradients on the matrix cores, then the head slices' dB and dC
// summed in order.
bool ssm_chunked(int P, int N, int aps, int64_t H, int64_t G);
// Row-wise backward for 16 states (rows of a group a multiple of 128, H P and G N at most 2^24):
// the state gradient entering every 8-token window, then the windows in parallel with two lanes
// per row, then the combine over 128-row segments.
bool ssm_rowwise(int P, int H, int G, int N);
hipError_t launch_ssm_rowwise_bwd(const SsmArgs &a, hipStream_t st);
// Its forward: the state before every window (and s_out), then y per window (y null: states
// only).  The saved states take nck = ceil(T / 8) + 1 slots per row (the last one spare).
hipError_t launch_ssm_rowwise_fwd(const SsmArgs &a, hipStream_t st);
hipError_t launch_ssm_chunk_bwd(const SsmArgs &a, hipStream_t st);
// Its forward: the state before every chunk (and s_out), then y per chunk (y null: states only).
hipError_t launch_ssm_chunk_fwd(const SsmArgs &a, hipStream_t st);
// head sizes: key width SK and value width SV, each in {16, 32, 64, 128}, not both 128
hipError_t launch_fwd(const FwdArgs &a, int SK, int SV, bool kda, int n_seqs_launch, hipStream_t st);
hipError_t launch_bwd(const BwdArgs &a, int SK, int SV, bool kda, int n_seqs_launch, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);

// Head size 128 on the matrix cores (gdn_mf.hip): one argument block for the block
// preparation, forward and backward kernels.  Blocks are the 16-token blocks of each sequence;
// rows [s][t][h] index the per-token workspace arrays.
struct Mf128Args {
    const void *q, *k, *v, *g, *beta, *gy;   // element type dtype (GDN_DTYPE_*)
    const float *state0, *dstate_out;
    float *y, *state_out;   // forward outputs (y null: the backward's checkpoint pass)
    float *snap;            // [unit][n_ck_max][S][S] state before tokens 0, C, 2C, ...
    float *wmat;            // [n_seqs][nblk][H_v][3][16][16] block matrices Bm, Te, Tb
    int32_t *wflag;         // [n_seqs][nblk][H_v] nonzero: block processed token by token
    float *cbuf;            // [n_seqs][T][H_v][G] running gate product c within the token's
                            // block (the gates a themselves in a token-by-token block)
    float *ebuf;            // [n_seqs][T][H_v][S] prediction errors e = v - u
    // The chain's per-token results for the column pass, for tokens pb_t0 .. pb_t0 + pb_T - 1
    // of every sequence (the whole sequence, or one piece of a pipelined pass):
    float *g1buf;           // [n_seqs][pb_T/16][H_v][nslab][16][16] Grams G1 = delta^T (scale gy),
    float *g2buf;           // s <= t, and G2 = delta^T du, s < t, over each slab's rows of a block
    float *dbp;             // [n_seqs][pb_T][H_v][nslab] dbeta per slab (nslab > 1)
    float *p3buf;           // [n_seqs][pb_T][H_v][S] P3 = X'^T delta per token (the chain's column
                            // sums of the state gradient against the token's delta)
    int32_t pb_T, pb_t0;
    float *anc;             // [unit][n_ck_max][S] dg at each checkpoint segment's first token
    float *dq, *dk, *dv, *dg, *dbeta, *dstate;   // dq, dk per key head, summed over its value heads
    gdn_strides sq, sk, sv, sg, sb, sgy, sy;
    int32_t s_base, n_seqs_launch, T, H_k, H_v, C, n_ck_max, kda, dtype;
    int32_t nslab;          // row slabs per unit of the forward and the chain: 1 or 2
    int32_t t_lo, t_hi;     // tokens of this launch: [t_lo, t_hi), t_lo a multiple of 16 (of C
                            // for the chain and the column pass); 0 and T for a whole pass
    float *carry;           // [unit][S][S] state (forward) or gradient (chain) between launches
    float scale;
    int32_t lens[kMaxSeqsPerLaunch];
};
hipError_t launch_prep128(const Mf128Args &a, hipStream_t st);
hipError_t launch_fwd_mf(const Mf128Args &a, hipStream_t st);
hipError_t launch_zero_anc(const Mf128Args &a, hipStream_t st);  // before the first chain launch
hipError_t launch_zero_p3(const Mf128Args &a, hipStream_t st);   // before a chain launch fills P3
hipError_t launch_zero_p3_all(const Mf128Args &a, hipStream_t st);   // also with one slab
hipError_t launch_chain(const Mf128Args &a, hipStream_t st);     // the chain over [t_lo, t_hi)
hipError_t launch_colsum(const Mf128Args &a, hipStream_t st);    // the column sums of its segments

}  // namespace gdn
