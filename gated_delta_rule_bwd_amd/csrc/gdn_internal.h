// gdn_internal.h -- argument blocks shared by the host side of the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Sequences handled by one launch; their lengths travel in the kernel argument block.
constexpr int kMaxSeqsPerLaunch = 256;

// Arguments of the forward scan (also used, with y == nullptr, as the checkpoint pass
// of the backward).
struct FwdArgs {
    const float *q, *k, *v, *g, *beta, *state0;
    float *y;          // nullptr: do not write y
    float *state_out;  // nullptr: do not write the final state
    float *snap;       // [unit][n_ck_max][S][S] snapshots (state before tokens 0, C, 2C, ...)
    // S = 128 path, written by the gate kernel, each [n_seqs][T][H_v][G]: in a window
    // processed column-scaled, cbuf holds the running product c of the gates a = exp(g)
    // within the token's 8-token window (inclusive) and dbuf the product d of the window's
    // later gates; in a window processed unscaled, cbuf holds a itself and dbuf 1.  wflag
    // [n_seqs][ceil(T / 8)][H_v] is nonzero for a window processed unscaled
    const float *cbuf, *dbuf;
    const int32_t *wflag;
    float *ebuf;       // S = 128 path: prediction errors e = v - u, [n_seqs][T][H_v][S]
    gdn_strides sq, sk, sv, sg, sb, sy;
    int32_t s_base;    // first sequence of this launch
    int32_t T, H_k, H_v, C, n_ck_max;
    float scale;
    // element type (GDN_DTYPE_*) of q, k, v, g, beta, which the S = 128 kernels read as such
    // (widened exactly at the load); the other kernels always receive fp32
    int32_t dtype;
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
    // S = 128 path
    const float *cbuf, *dbuf, *ebuf;  // gate kernel and forward outputs (see FwdArgs)
    const int32_t *wflag;
    float *vsbuf;              // [unit][4][nvs_max][32 x S] states at 64-token boundaries
    float *part;               // [n_seqs][T][H_v][4][3][S] column sums of each row quarter
    float *pbuf;               // [n_seqs][T][H_v][4] dbeta per quarter
    float *pgbuf;              // [n_seqs][T][H_v][4][2] scalar-gate dg per quarter and column half
    float *hfin;               // [n_seqs][H_v][4][G] column sums of dstate_out .* M_final per quarter
    int32_t nvs_max;
    gdn_strides sq, sk, sv, sg, sb, sgy;
    int32_t s_base;
    int32_t T, H_k, H_v, C, n_ck_max;
    float scale;
    int32_t dtype;      // element type of q, k, v, g, beta, gy (see FwdArgs)
    int32_t lens[kMaxSeqsPerLaunch];
};

// Per-window gate factors and flags of every token t < len of the launch's sequences, as
// described in FwdArgs (S = 128 path).
struct GateArgs {
    const float *g;
    float *cbuf, *dbuf;          // [n_seqs][T][H_v][G]
    int32_t *wflag;              // [n_seqs][ceil(T / 8)][H_v]
    gdn_strides sg;
    int32_t s_base, n_seqs_launch, T, H_v, G;
    int32_t dtype;               // element type of g (see FwdArgs)
    int32_t lens[kMaxSeqsPerLaunch];
};

// Sum of the row-quarter partials (and, for dq/dk, of the value heads of each key head) on
// the S = 128 path; writes dq, dk, dg, dbeta including the zero rows of padded tokens.
struct Combine128Args {
    const float *part, *pbuf, *pgbuf, *hfin;
    float *dq, *dk, *dg, *dbeta;
    int32_t s_base, n_seqs_launch, T, H_k, H_v, kda;
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

// Selective state-space scan and its reverse recurrence (see ssm_scan.hip).  Contiguous
// tensors: s0/s_out/ds0 [n][H][P][N], x/y/gy/dx/ddrow [n][T][H][P], dt/ddt [n][T][H],
// A [H][N] (aps) or [H], B/C/dB/dC [n][T][G][N]; workspace: ck [rows][ceil(T/8)][N],
// part [rows/16][T][2][N], ddrow.
struct SsmArgs {
    const float *s0, *x, *dt, *A, *B, *C, *gy, *gs;
    float *ck, *part, *ddrow;
    float *y, *s_out, *ds0, *dx, *ddt, *dB, *dC;
    int32_t n_seqs, T, H, P, N, G, aps, softplus;
};
hipError_t launch_ssm(const SsmArgs &a, bool bwd, hipStream_t st);   // forward or walk
hipError_t launch_ssm_combine(const SsmArgs &a, hipStream_t st);
// head sizes: key width SK and value width SV, each in {16, 32, 64, 128}, not both 128
hipError_t launch_fwd(const FwdArgs &a, int SK, int SV, bool kda, int n_seqs_launch, hipStream_t st);
hipError_t launch_bwd(const BwdArgs &a, int SK, int SV, bool kda, int n_seqs_launch, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);
hipError_t launch_gate128(const GateArgs &a, hipStream_t st);
hipError_t launch_fwd128(const FwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st);
hipError_t launch_bwd128(const BwdArgs &a, bool kda, int n_seqs_launch, hipStream_t st);
hipError_t launch_combine128(const Combine128Args &a, hipStream_t st);

}  // namespace gdn
