/*
 * gdn.h -- C ABI of the gated delta rule (forward scan and checkpointed backward) on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (per sequence s and value head h; key head hk = h mod H_k, the head map
 * "iv1 % neq1" of the first review of "metal: GATED_DELTA_NET_BACK"; the state is kept as
 * M = S^T, S_v rows j by S_k columns i, as in that page's approval review):
 *
 *   forward, per token t (decay before correction; meTile "Training kernels and gradients",
 *   section "Recurrent delta attention"):
 *       a = exp(g_t)  (per key channel, or one scalar)      Mp = M .* a  (column scaling)
 *       u = Mp k_t,   delta = beta_t (v_t - u),   M = Mp + delta k_t^T,   y_t = scale M q_t
 *   backward (the term-by-term math of the same PR's first review): seeded with
 *   dM = dstate_out at t = len, walking t downwards:
 *       dM += scale gy_t q_t^T;   dq_t += scale M_t^T gy_t;   dd = dM k_t;   dv_t = beta dd;
 *       du = -beta dd;   dbeta_t = dd . (v_t - u);   dk_t += dM^T delta + Mp^T du (dM before
 *       the next update);   dM += du k_t^T;   dg_t = sum_j dM .* Mp (per column, or in total
 *       for the scalar gate);   dM = dM .* a;     and dstate = dM after token 0.
 *   The backward recomputes states from snapshots taken every C tokens (C ~ sqrt(T), the
 *   PR description); the snapshot interval changes memory and time, not the result.
 *
 * Declared further down, under the same conventions: the steps around the recurrence in a
 * hybrid layer -- the short causal convolution that produces the mixed q/k/v rows and its
 * input gradient (gdn_ssm_conv_fwd / _bwd) and the per-row L2 normalisation of q and k and
 * its backward (gdn_l2norm_fwd / _bwd) -- and a second reverse recurrence, the selective
 * state-space scan of the Mamba-1 and Mamba-2 branches with its backward (gdn_ssm_*).
 *
 * All floating point data is fp32, apart from the inputs of gdn_fwd / gdn_bwd when
 * gdn_problem.dtype selects a half type.  Index arithmetic is 64-bit.
 *
 * Ownership and concurrency
 *   - The caller owns every buffer.  The library allocates no device memory (apart from the
 *     static array of gdn_bwd_noalloc) and keeps no data between calls.
 *   - For head size 128, gdn_fwd and gdn_bwd split the token axis into pieces and enqueue part
 *     of the work (the preparation of later pieces, the column sums of finished pieces) on a
 *     second stream that the library creates for the device on first use, at the default
 *     priority, with a pool of events; before returning, a call makes the caller's stream wait
 *     for that work, so the caller sees stream order as if everything ran on its stream.
 *     Calls from several host threads on one device take turns while enqueueing.
 *   - Calls are asynchronous on the given HIP stream (NULL = the legacy default stream);
 *     results are valid once the stream has passed the call.  Faults surface at the
 *     caller's synchronisation.
 *   - The workspace belongs to one call at a time; it may be reused once the stream has
 *     passed the call.  A workspace written by gdn_fwd holds that call's state snapshots
 *     (see GDN_BWD_REUSE_SNAPSHOTS).
 *   - Outputs (y, state_out, grad_packed, ...) must not overlap any input, the workspace or
 *     each other (gdn_l2norm_* alone may write exactly over an input view); the host checks
 *     the address ranges and returns GDN_ERR_ARG on overlap.
 *     Inputs and cotangents are never written.
 *   - Inputs must be finite for the results to be meaningful (no NaN checks).  Values at
 *     padded tokens (t >= len_s) are never read.
 *
 * Errors are synchronous return codes, checked before anything is enqueued: a non-zero
 * return means no work was enqueued.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GDN_OK 0
#define GDN_ERR_ARG (-1)         /* a NULL required pointer, a bad size, an overlap       */
#define GDN_ERR_UNSUPPORTED (-2) /* outside the verified envelope (see gdn_problem)      */
#define GDN_ERR_WORKSPACE (-3)   /* ws_bytes below gdn_workspace_size()                 */
#define GDN_ERR_DEVICE (-4)      /* the HIP runtime refused a launch                     */

/* Gate kinds (meTile "Recurrent delta attention": a scalar log-decay per token and head is
 * Gated DeltaNet, a per-key-channel log-decay is the Kimi Delta Attention core). */
#define GDN_GATE_SCALAR 0
#define GDN_GATE_KDA 1

/* Element type of the inputs q, k, v, g, beta and gy (gdn_problem.dtype).  The state, y and
 * every gradient are fp32 (the contract of "Training kernels and gradients", introduction:
 * half-precision inputs, fp32 gradient storage).  Half-precision inputs are widened exactly
 * to fp32 (at the load for head size 128; into workspace copies for the other head sizes), so
 * the results equal those of fp32 inputs holding the same values. */
#define GDN_DTYPE_F32 0
#define GDN_DTYPE_F16 1
#define GDN_DTYPE_BF16 2

/* gdn_bwd flags. */
#define GDN_BWD_REUSE_SNAPSHOTS 1u /* ws holds the snapshots written by gdn_fwd on the same
                                      problem and inputs: skip the checkpoint pass */

/* HIP stream handle (hipStream_t); declared here so that this header needs no HIP header. */
typedef struct ihipStream_t *gdn_stream_t;

/* Strides of a per-token tensor, in elements (floats).  The innermost (feature) stride is
 * always 1.  Element (s, t, head, i) lives at base + s*seq + t*tok + head*head_ + i.
 * Strides must be non-negative.  This admits row views into a packed buffer, as when q and
 * k are views of one mixed projection ("metal: GATED_DELTA_NET_BACK", first review). */
typedef struct gdn_strides {
    int64_t seq, tok, head;
} gdn_strides;

/* Problem description.
 *   n_seqs      number of sequences (>= 0); lengths are padded to T
 *   T           padded sequence length (>= 0)
 *   H_k, H_v    key and value head counts; H_v must be a multiple of H_k (grouped heads:
 *               value head h reads key head h mod H_k)
 *   S_k, S_v    key and value head sizes, each in {16, 32, 64, 128} (equal or not)
 *   gate        GDN_GATE_SCALAR (g is [.., H_v], one value per token and head) or
 *               GDN_GATE_KDA (g is [.., H_v, S_k])
 *   C           checkpoint interval in tokens; 0 selects ceil(sqrt(T)); values above T
 *               act as T (one segment).  For S = 128 the interval is rounded up to a
 *               multiple of 16 (the kernels carry the state column-scaled over 16-token
 *               blocks that checkpoints must not split); results are then bitwise the
 *               same for every interval
 *   scale       output scale (commonly 1/sqrt(S_k))
 *   seq_lens    HOST pointer to n_seqs lengths in [0, T], or NULL for all T
 *   q, k        strides of q, k   (head counts H_k, width S_k)
 *   v           strides of v      (H_v, S_v)
 *   g           strides of g      (H_v, width S_k or 1)
 *   beta        strides of beta   (H_v, width 1)
 *   gy          strides of the output cotangent (H_v, S_v); used by gdn_bwd only
 *   y           strides of the output y (H_v, S_v); used by gdn_fwd only
 *   dtype       GDN_DTYPE_* of q, k, v, g, beta, gy (strides count elements of that type);
 *               0 (fp32) in a zero-initialised struct
 * State tensors (state0, state_out, dstate_out, dstate) are contiguous
 * [n_seqs][H_v][S_v][S_k] in the M = S^T orientation (row = value index). */
typedef struct gdn_problem {
    int32_t n_seqs, T, H_k, H_v, S_k, S_v, gate, C;
    float scale;
    const int32_t *seq_lens;
    gdn_strides q, k, v, g, beta, gy, y;
    int32_t dtype;
} gdn_problem;

/* Bytes of device workspace that gdn_fwd and gdn_bwd need for this problem (0 on an
 * invalid problem).  The same workspace serves both calls.  It holds what the scratch of the
 * approval review's sizing note on "metal: GATED_DELTA_NET_BACK" holds -- the state snapshots
 * every C tokens -- plus, for head size 128, per-token arrays of the matrix-core kernels (the
 * running gate products, the prediction errors, the block matrices, and the chain's results
 * for the column sums: its Grams, dbeta per row slab and P3, for every token or, on long
 * sequences, for a ring of four pieces), dg at the first token of every segment and the state
 * carried between pieces; for the other head sizes the states recomputed inside one segment
 * and, when H_v > H_k, dq and dk per value head.  The caller allocates it once; nothing else
 * is allocated. */
size_t gdn_workspace_size(const gdn_problem *p);

/* Layout of the packed gradient buffer (PR description of "metal: GATED_DELTA_NET_BACK":
 * one output holding [dq|dk|dv|dg|dbeta|dstate]).  Writes the float offset of each region
 * into offsets[6] (may be NULL) and returns the total number of floats (0 on an invalid
 * problem).  Regions, contiguous, in this order:
 *   dq     [n_seqs][T][H_k][S_k]     dk  [n_seqs][T][H_k][S_k]
 *   dv     [n_seqs][T][H_v][S_v]     dg  [n_seqs][T][H_v][G]  (G = S_k or 1)
 *   dbeta  [n_seqs][T][H_v]          dstate [n_seqs][H_v][S_v][S_k]
 * Rows with t >= len_s are written as zeros. */
size_t gdn_grad_packed_floats(const gdn_problem *p, size_t offsets[6]);

/* Forward scan (meTile, "Training kernels and gradients", section "Recurrent delta
 * attention": per token the state decays by the gates, corrects by delta k^T with
 * delta = beta (v - u), and reads out y = scale M q): writes y (strided as p->y) and
 * state_out, and the state snapshots into the workspace.  All pointers are device pointers; q, k, v, g, beta (and gy) hold p->dtype
 * elements and are aligned to that element size, every other buffer is 4-byte aligned, ws
 * 16-byte aligned (GDN_ERR_UNSUPPORTED / GDN_ERR_ARG otherwise).  Returns GDN_OK or an error
 * code (nothing enqueued on error). */
int gdn_fwd(const gdn_problem *p, const void *q, const void *k, const void *v,
            const void *g, const void *beta, const float *state0, float *y,
            float *state_out, void *ws, size_t ws_bytes, gdn_stream_t stream);

/* Backward (the term-by-term gradients of the first review of "metal:
 * GATED_DELTA_NET_BACK", restated at the top of this header; states recomputed from the
 * snapshots every C tokens, the PR description's checkpointed recompute): given the forward's
 * inputs, the output cotangent gy (strided as p->gy) and the final-state cotangent
 * dstate_out (NULL means zero), writes the six input gradients
 * into grad_packed (layout: gdn_grad_packed_floats).  With GDN_BWD_REUSE_SNAPSHOTS the
 * snapshots already in ws from gdn_fwd are used; otherwise they are recomputed first.
 * dq and dk of one key head sum its value heads in increasing h, so results are bitwise
 * reproducible run to run.  Pointer alignment as for gdn_fwd; results do not depend on the
 * alignment of grad_packed. */
int gdn_bwd(const gdn_problem *p, const void *q, const void *k, const void *v,
            const void *g, const void *beta, const float *state0, const void *gy,
            const float *dstate_out, float *grad_packed, void *ws, size_t ws_bytes,
            unsigned flags, gdn_stream_t stream);

/* Allocation-free backward, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and checks as gdn_bwd without the snapshot reuse, but no workspace argument: the
 * workspace is a static device array of GDN_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends (its address is looked up once per device, on
 * that device's first call).  A problem whose gdn_workspace_size exceeds the array returns
 * GDN_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing.  Every call on
 * one GPU shares that GPU's array and the array keeps the last call's contents (none of which
 * a later call reads): calls that overlap in time on one GPU (other streams, other host
 * threads) race on it and give wrong results, so the caller must serialise them.  The
 * snapshots are always recomputed.  The stream's device selects the array. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gdn_bwd_noalloc(const gdn_problem *p, const void *q, const void *k, const void *v,
                    const void *g, const void *beta, const float *state0, const void *gy,
                    const float *dstate_out, float *grad_packed, gdn_stream_t stream);

/* Short causal depthwise convolution upstream of the recurrence (the one that produces the
 * mixed q/k/v rows) and its gradient with respect to the input; the weights are frozen and
 * take no gradient (page "S1-24: chunked attention -- the kernel-free long-context path",
 * the commit notes on SSM_CONV_BACK).  Channels are innermost:
 *   sx, d_sx [n_seqs][d_conv - 1 + T][d_inner]  the d_conv - 1 carried state rows, then T
 *   c        [d_inner][d_conv] (contiguous)
 *   y, dy    [n_seqs][T][d_inner]
 *   y[s][t][i]    = sum_j sx[s][t + j][i] c[i][j]              (j = 0 .. d_conv - 1)
 *   d_sx[s][u][i] = sum_j dy[s][u - j][i] c[i][j]  over 0 <= u - j < T
 * (the carried state rows get their gradient too).  Row strides are in floats; the channel
 * stride is 1.  Supported: 1 <= d_conv <= 8.  Pointers are device pointers, 4-byte aligned;
 * a tensor with no elements (n_seqs = 0, or no rows) may be NULL.  Outputs must not overlap
 * inputs.  Results are deterministic (one owner per output, taps
 * in increasing j).  Returns GDN_OK or an error code (nothing enqueued on error). */
typedef struct gdn_conv_problem {
    int32_t n_seqs, T, d_inner, d_conv;
    int64_t sx_seq, sx_tok;   /* strides of sx and d_sx */
    int64_t y_seq, y_tok;     /* strides of y and dy */
} gdn_conv_problem;

int gdn_ssm_conv_fwd(const gdn_conv_problem *p, const float *sx, const float *c, float *y,
                     gdn_stream_t stream);
int gdn_ssm_conv_bwd(const gdn_conv_problem *p, const float *dy, const float *c, float *d_sx,
                     gdn_stream_t stream);

/* L2 normalisation of the q and k rows between the short convolution and the recurrence, and
 * its backward (meTile, "Training kernels and gradients", section "Recurrent delta attention":
 * normalisation is a step of its own, outside the recurrence kernel).  Each row of W floats
 * (one token of one head) maps to
 *   n = sqrt(sum_i x_i^2 + eps),  y = x / n,
 * and the backward takes the cotangent dy of y to
 *   dx = dy / n - x (x . dy) / n^3.
 * Rows are [n_seqs][T][H]; each tensor has its own (seq, tok, head) strides in floats and unit
 * innermost stride, so q and k may be row views of the mixed rows and dx may be written into a
 * view of their gradient.  Supported: 1 <= W <= 1024, eps >= 0 and finite (eps = 0 maps an
 * all-zero row to non-finite values, as the formula does).  Pointers are device pointers,
 * 4-byte aligned; a tensor with no rows may be NULL.  The output may be the very same view as
 * an input (same pointer, same strides: in place) and must not otherwise overlap one, nor
 * overlap itself.  Deterministic.  Returns GDN_OK or an error code (nothing enqueued on
 * error). */
typedef struct gdn_l2norm_problem {
    int32_t n_seqs, T, H, W;
    float eps;
    gdn_strides x, dy, out;   /* dy: backward only */
} gdn_l2norm_problem;

int gdn_l2norm_fwd(const gdn_l2norm_problem *p, const float *x, float *y, gdn_stream_t stream);
int gdn_l2norm_bwd(const gdn_l2norm_problem *p, const float *x, const float *dy, float *dx,
                   gdn_stream_t stream);

/* Selective state-space scan (Mamba-1 and Mamba-2 branches) and its backward, the reverse
 * recurrence (page "S1-24: chunked attention": the SSM_SCAN_BACK commit notes and the n_group
 * fold).  Per sequence, head h, head element i and state n, with step d = softplus(dt) when
 * dt_softplus is 1 (d = dt when 0) and group g = h / (H / G):
 *   a = exp(d A[h][n])  (A[h] for every n when a_per_state is 0)
 *   s[i][n] = a s[i][n] + d x[i] B[g][n],   y[i] = sum_n s[i][n] C[g][n]
 * Contiguous fp32 tensors (device pointers):
 *   s0, s_out  [n_seqs][H][P][N]     x, y, gy  [n_seqs][T][H][P]     dt  [n_seqs][T][H]
 *   A          [H][N] or [H]         B, C      [n_seqs][T][G][N]
 * Supported: N in {16, 32, 64, 128}; H % G == 0 and P * H / G a multiple of 16 (16-row
 * blocks of the kernels never straddle a group); s0, s_out, A, B, C, gs_final, grad_packed
 * and ws 16-byte aligned, the rest 4-byte aligned.  Outputs must not overlap inputs or each
 * other.  Returns GDN_OK or an error code (nothing enqueued on error). */
typedef struct gdn_ssm_problem {
    int32_t n_seqs, T, H, P, N, G;
    int32_t a_per_state;   /* 1: A is [H][N] (Mamba-1); 0: A is [H] (Mamba-2) */
    int32_t dt_softplus;   /* 1: step = softplus(dt); 0: step = dt */
} gdn_ssm_problem;

/* Bytes of device workspace gdn_ssm_fwd and gdn_ssm_bwd need (0 on an invalid problem): the
 * state before every 8-token window, per-16-row column partials and per-row ddt terms (with
 * N = 16 and a multiple of 128 rows per group: per-128-row partials and the state gradient
 * entering every window); for one decay per head with P = 64 and N = 128, whose backward runs
 * in 32-token chunks on the matrix cores, the state before every chunk, the state gradient
 * after every chunk and dB/dC per head slice instead.  The same workspace serves both calls. */
size_t gdn_ssm_workspace_size(const gdn_ssm_problem *p);

/* Layout of the packed gradient (the page's [d_s | d_x | d_dt | d_B | d_C], contiguous, in
 * that order, shaped like s0, x, dt, B, C).  Writes the float offset of each region into
 * offsets[5] (may be NULL) and returns the total number of floats (0 on an invalid problem). */
size_t gdn_ssm_grad_packed_floats(const gdn_ssm_problem *p, size_t offsets[5]);

/* Forward: writes y and s_out, and the steps and window states into ws. */
int gdn_ssm_fwd(const gdn_ssm_problem *p, const float *s0, const float *x, const float *dt,
                const float *A, const float *B, const float *C, float *y, float *s_out,
                void *ws, size_t ws_bytes, gdn_stream_t stream);

/* Backward: the gradients of L = <gy, y> + <gs_final, s_out> (gs_final NULL means zero; the
 * reverse walk is seeded with it) with respect to s0, x, dt, B and C, into grad_packed.  A takes
 * no gradient.  With GDN_BWD_REUSE_SNAPSHOTS the window states that gdn_ssm_fwd left
 * in ws for the same inputs are used; otherwise they are recomputed first.  dB and dC of a
 * group sum its heads and rows in a fixed order: results are bitwise reproducible. */
int gdn_ssm_bwd(const gdn_ssm_problem *p, const float *s0, const float *x, const float *dt,
                const float *A, const float *B, const float *C, const float *gy,
                const float *gs_final, float *grad_packed, void *ws, size_t ws_bytes,
                unsigned flags, gdn_stream_t stream);

/* Human-readable name of a status code. */
const char *gdn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
