/*
 * gdn_oracle.c -- plain fp64 CPU reference of the gated delta rule, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke() entry and the CPU-baseline leg of the
 * benchmark may load this library.  The HIP product path shares no code with it.
 *
 * What it computes (all in double precision, plain loops, no blocking or fusion):
 *
 *   Notation per (sequence s, value head h), key head hk = h mod H_k.  The state is held as
 *   M = S^T with rows j = value index (S_v of them) and columns i = key index (S_k of them),
 *   the row-owner form of the CPU-reference author ("metal: GATED_DELTA_NET_BACK", approval
 *   review: each row of M = S^T is handled on its own by one worker).
 *
 *   Forward, per token t (decay before correction; meTile "Training kernels and gradients",
 *   section "Recurrent delta attention"; the row-owner form in the same review):
 *     a      = exp(g_t)            (vector over columns for the per-key-channel gate,
 *                                   one scalar broadcast for the scalar gate)
 *     Mp     = M .* a              (column i scaled by a_i)
 *     u      = Mp k_t
 *     e      = v_t - u,  delta = beta_t e
 *     M      = Mp + delta k_t^T
 *     y_t    = scale * M q_t
 *
 *   Backward (reverse walk, "metal: GATED_DELTA_NET_BACK", first review's term-by-term
 *   reading and the approval review's passes C/D/E), seeded with dM = dstate_out at t = len:
 *     sgy    = scale * gy_t
 *     dM    += sgy q_t^T
 *     dq_t  += M_t^T sgy                (M_t = state after token t; column sums)
 *     dd     = dM k_t
 *     dv_t   = beta dd,   du = -beta dd,   dbeta_t = dd . e
 *     dk_t  += dM^T delta + Mp^T du     (dM taken before the du update)
 *     dM    += du k_t^T
 *     dg_t   = sum_j dM[j][i] Mp[j][i]  per column i (per-key-channel gate), or summed over
 *              all (j, i) (scalar gate)
 *     dM     = dM .* a                  (gradient w.r.t. the previous state)
 *   and dstate = dM after token 0.  dq and dk of one key head accumulate the value heads
 *   h = hk, hk + H_k, hk + 2 H_k, ... in increasing order.
 *
 *   Checkpointed recompute (same pages, PR description and the approval review's scratch
 *   sizing): the forward pass keeps the state before tokens 0, C, 2C, ...; the backward
 *   replays each segment from its snapshot and walks it in reverse.  The replay executes the
 *   identical double-precision operations, so any C gives bit-identical results (C >= len is
 *   the store-all variant).  C <= 0 selects ceil(sqrt(T)).
 *
 * Layouts (all contiguous, double):
 *   q, k      [n_seqs][T][H_k][S_k]
 *   v, gy, y  [n_seqs][T][H_v][S_v]
 *   g         [n_seqs][T][H_v][G]   G = S_k (per-key-channel gate) or 1 (scalar gate)
 *   beta      [n_seqs][T][H_v]
 *   state0, state_out, dstate_out, dstate   [n_seqs][H_v][S_v][S_k]
 *   dq, dk    [n_seqs][T][H_k][S_k]; dv [n_seqs][T][H_v][S_v]; dg like g; dbeta like beta
 * Rows with t >= len_s of every per-token output are written as 0.
 *
 * Threads: work is split over (sequence, key head) pairs; each pair is owned by one thread,
 * which walks its value heads in increasing order, so results do not depend on thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread gdn_oracle.c -lm
 * A mutation build (-DGDN_ORACLE_MUTATION=n) plants one deliberate mistake; the test suite
 * uses these to prove that its pins can see such mistakes.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef GDN_ORACLE_MUTATION
#define GDN_ORACLE_MUTATION 0
#endif
#define MUT(n) (GDN_ORACLE_MUTATION == (n))

typedef struct {
    int n_seqs, T, H_k, H_v, S_k, S_v, kda, C;
    double scale;
    const int *seq_lens; /* NULL: every sequence has length T */
} gdn_oracle_problem;

/* Inputs and outputs of one call; any output pointer may be NULL (not computed). */
typedef struct {
    const double *q, *k, *v, *g, *beta, *state0, *gy, *dstate_out;
    double *y, *state_out;
    double *dq, *dk, *dv, *dg, *dbeta, *dstate;
} gdn_oracle_io;

int gdn_oracle_mutation(void) { return GDN_ORACLE_MUTATION; }

static int seq_len(const gdn_oracle_problem *p, int s) {
    return p->seq_lens ? p->seq_lens[s] : p->T;
}

static int key_head_of(const gdn_oracle_problem *p, int h) {
#if GDN_ORACLE_MUTATION == 4
    return h / (p->H_v / p->H_k); /* planted: interleaved head map instead of modulo */
#else
    return h % p->H_k;
#endif
}

int gdn_oracle_default_C(int T) {
    if (T <= 0) return 1;
    int c = (int)ceil(sqrt((double)T));
    while ((long)(c - 1) * (c - 1) >= T && c > 1) c--; /* exact integer ceil(sqrt(T)) */
    while ((long)c * c < T) c++;
    return c;
}

/* index helpers for the logical contiguous layouts */
static size_t ix_tok(const gdn_oracle_problem *p, int s, int t, int heads, int h, int width) {
    return (((size_t)s * p->T + t) * heads + h) * (size_t)width;
}
static size_t ix_state(const gdn_oracle_problem *p, int s, int h) {
    return ((size_t)s * p->H_v + h) * (size_t)p->S_v * p->S_k;
}

/* Per-token quantities of one forward step for unit (s, h) at token t. */
typedef struct {
    const double *q, *k, *v, *g; /* q, k: S_k; v: S_v; g: G entries */
    double beta;
} tok_in;

static tok_in token_inputs(const gdn_oracle_problem *p, const gdn_oracle_io *io, int s, int h,
                           int t) {
    tok_in ti;
    int hk = key_head_of(p, h);
    int G = p->kda ? p->S_k : 1;
    ti.q = io->q + ix_tok(p, s, t, p->H_k, hk, p->S_k);
    ti.k = io->k + ix_tok(p, s, t, p->H_k, hk, p->S_k);
    ti.v = io->v + ix_tok(p, s, t, p->H_v, h, p->S_v);
    ti.g = io->g + ix_tok(p, s, t, p->H_v, h, G);
    ti.beta = io->beta[ix_tok(p, s, t, p->H_v, h, 1)];
    return ti;
}

static double gate_at(const gdn_oracle_problem *p, const tok_in *ti, int i) {
    return exp(p->kda ? ti->g[i] : ti->g[0]);
}

#if GDN_ORACLE_MUTATION == 12
#define GATE_COL(i, j) ((j) % p->S_k) /* planted: per-channel gate applied along rows */
#else
#define GATE_COL(i, j) (i)
#endif

/* One forward step: Mnext = Mp + delta k^T with Mp = M .* a, u = Mp k, e = v - u.
 * Mp, u, e are returned for the backward's use (any may be NULL). M and Mnext may alias. */
static void forward_step(const gdn_oracle_problem *p, const tok_in *ti, const double *M,
                         double *Mnext, double *Mp_out, double *u_out, double *e_out) {
    int Sv = p->S_v, Sk = p->S_k;
    for (int j = 0; j < Sv; j++) {
        const double *Mr = M + (size_t)j * Sk;
        double u = 0.0;
        for (int i = 0; i < Sk; i++) u += Mr[i] * gate_at(p, ti, GATE_COL(i, j)) * ti->k[i];
#if GDN_ORACLE_MUTATION == 9
        double e = ti->v[j] + u; /* planted: wrong sign of the prediction */
#else
        double e = ti->v[j] - u;
#endif
        double delta = ti->beta * e;
        if (u_out) u_out[j] = u;
        if (e_out) e_out[j] = e;
        double *Mn = Mnext + (size_t)j * Sk;
        for (int i = 0; i < Sk; i++) {
            double mp = Mr[i] * gate_at(p, ti, GATE_COL(i, j));
#if GDN_ORACLE_MUTATION == 10
            mp = Mr[i]; /* planted: gate applied after the correction instead of before */
            if (Mp_out) Mp_out[(size_t)j * Sk + i] = mp;
            Mn[i] = (mp + delta * ti->k[i]) * gate_at(p, ti, i);
            continue;
#endif
            if (Mp_out) Mp_out[(size_t)j * Sk + i] = mp;
            Mn[i] = mp + delta * ti->k[i];
        }
    }
}

static void output_row(const gdn_oracle_problem *p, const tok_in *ti, const double *M, double *y) {
    for (int j = 0; j < p->S_v; j++) {
        double acc = 0.0;
        for (int i = 0; i < p->S_k; i++) acc += M[(size_t)j * p->S_k + i] * ti->q[i];
        y[j] = p->scale * acc;
    }
}

/* ---------------------------------------------------------------- forward */

static void forward_unit(const gdn_oracle_problem *p, const gdn_oracle_io *io, int s, int h,
                         double *M) {
    int L = seq_len(p, s);
    size_t SS = (size_t)p->S_v * p->S_k;
    memcpy(M, io->state0 + ix_state(p, s, h), SS * sizeof(double));
    for (int t = 0; t < p->T; t++) {
        double *yrow = io->y ? io->y + ix_tok(p, s, t, p->H_v, h, p->S_v) : NULL;
        if (t >= L) {
            if (yrow) memset(yrow, 0, sizeof(double) * p->S_v);
            continue;
        }
        tok_in ti = token_inputs(p, io, s, h, t);
        forward_step(p, &ti, M, M, NULL, NULL, NULL);
        if (yrow) output_row(p, &ti, M, yrow);
    }
    if (io->state_out) memcpy(io->state_out + ix_state(p, s, h), M, SS * sizeof(double));
}

/* ---------------------------------------------------------------- backward */

typedef struct {
    double *ck;          /* n_ck snapshots, S_v x S_k each                     */
    double *states;      /* C + 1 recomputed states of the current segment     */
    double *Mp, *u, *e;  /* per segment token: Mp (S_v x S_k), u, e (S_v)      */
    double *dM, *dd, *du, *delta, *sgy;
} bwd_scratch;

static void backward_unit(const gdn_oracle_problem *p, const gdn_oracle_io *io, int s, int h,
                          int C, bwd_scratch *w) {
    int Sv = p->S_v, Sk = p->S_k;
    int L = seq_len(p, s);
    int hk = key_head_of(p, h);
    int G = p->kda ? Sk : 1;
    size_t SS = (size_t)Sv * Sk;

    /* padded rows of the value-head outputs (dq/dk padded rows are zeroed by the caller) */
    for (int t = L; t < p->T; t++) {
        if (io->dv) memset(io->dv + ix_tok(p, s, t, p->H_v, h, Sv), 0, sizeof(double) * Sv);
        if (io->dg) memset(io->dg + ix_tok(p, s, t, p->H_v, h, G), 0, sizeof(double) * G);
        if (io->dbeta) io->dbeta[ix_tok(p, s, t, p->H_v, h, 1)] = 0.0;
    }

    /* checkpoint pass: snapshot before tokens 0, C, 2C, ... */
    int n_ck = L > 0 ? (L + C - 1) / C : 0;
    double *M = w->states; /* reuse slot 0 as the running state */
    memcpy(M, io->state0 + ix_state(p, s, h), SS * sizeof(double));
    for (int t = 0; t < L; t++) {
        if (t % C == 0) memcpy(w->ck + (size_t)(t / C) * SS, M, SS * sizeof(double));
        tok_in ti = token_inputs(p, io, s, h, t);
        forward_step(p, &ti, M, M, NULL, NULL, NULL);
    }

    double *dM = w->dM;
#if GDN_ORACLE_MUTATION == 2
    memset(dM, 0, SS * sizeof(double)); /* planted: final-state cotangent ignored */
#else
    if (io->dstate_out)
        memcpy(dM, io->dstate_out + ix_state(p, s, h), SS * sizeof(double));
    else
        memset(dM, 0, SS * sizeof(double));
#endif

    for (int sg = n_ck - 1; sg >= 0; sg--) {
        int t0 = sg * C, t1 = t0 + C < L ? t0 + C : L;
        /* replay the segment: states[0] = snapshot, states[n+1] = state after token t0+n */
        memcpy(w->states, w->ck + (size_t)sg * SS, SS * sizeof(double));
        for (int t = t0; t < t1; t++) {
            int n = t - t0;
            tok_in ti = token_inputs(p, io, s, h, t);
            forward_step(p, &ti, w->states + (size_t)n * SS, w->states + (size_t)(n + 1) * SS,
                         w->Mp + (size_t)n * SS, w->u + (size_t)n * Sv, w->e + (size_t)n * Sv);
        }
        for (int t = t1 - 1; t >= t0; t--) {
            int n = t - t0;
            tok_in ti = token_inputs(p, io, s, h, t);
            const double *Mt = w->states + (size_t)(n + 1) * SS; /* state after token t */
            const double *Mp = w->Mp + (size_t)n * SS;           /* decayed previous state */
            const double *e = w->e + (size_t)n * Sv;
            const double *gyr = io->gy + ix_tok(p, s, t, p->H_v, h, Sv);
            (void)gyr;
            (void)Mt;
            double *dq = io->dq + ix_tok(p, s, t, p->H_k, hk, Sk);
            double *dk = io->dk + ix_tok(p, s, t, p->H_k, hk, Sk);

            for (int j = 0; j < Sv; j++) {
#if GDN_ORACLE_MUTATION == 1
                w->sgy[j] = p->scale; /* planted: incoming output gradient ignored */
#else
                w->sgy[j] = p->scale * gyr[j];
#endif
                w->delta[j] = ti.beta * e[j];
            }
            /* dM += sgy q^T */
            for (int j = 0; j < Sv; j++)
                for (int i = 0; i < Sk; i++) dM[(size_t)j * Sk + i] += w->sgy[j] * ti.q[i];
            /* dq += M_t^T sgy */
            for (int i = 0; i < Sk; i++) {
                double acc = 0.0;
                for (int j = 0; j < Sv; j++) {
#if GDN_ORACLE_MUTATION == 6
                    double m = w->states[(size_t)n * SS + (size_t)j * Sk + i]; /* planted: M_{t-1} */
#else
                    double m = Mt[(size_t)j * Sk + i];
#endif
                    acc += m * w->sgy[j];
                }
                dq[i] += acc;
            }
            /* dd = dM k; dv; du; dbeta */
            double dbeta = 0.0;
            for (int j = 0; j < Sv; j++) {
                double acc = 0.0;
                for (int i = 0; i < Sk; i++) acc += dM[(size_t)j * Sk + i] * ti.k[i];
                w->dd[j] = acc;
                w->du[j] = -ti.beta * acc;
#if GDN_ORACLE_MUTATION == 8
                dbeta += acc * w->u[n * Sv + j]; /* planted: u in place of v - u */
#else
                dbeta += acc * e[j];
#endif
            }
            if (io->dv) {
                double *dvr = io->dv + ix_tok(p, s, t, p->H_v, h, Sv);
#if GDN_ORACLE_MUTATION == 11
                for (int j = 0; j < Sv; j++) dvr[j] = w->dd[j]; /* planted: beta dropped */
#else
                for (int j = 0; j < Sv; j++) dvr[j] = ti.beta * w->dd[j];
#endif
            }
            if (io->dbeta) io->dbeta[ix_tok(p, s, t, p->H_v, h, 1)] = dbeta;
#if GDN_ORACLE_MUTATION == 3
            /* planted: dk read after the du update */
            for (int j = 0; j < Sv; j++)
                for (int i = 0; i < Sk; i++) dM[(size_t)j * Sk + i] += w->du[j] * ti.k[i];
#endif
            /* dk += dM^T delta + Mp^T du */
            for (int i = 0; i < Sk; i++) {
                double acc = 0.0;
                for (int j = 0; j < Sv; j++)
                    acc += dM[(size_t)j * Sk + i] * w->delta[j] + Mp[(size_t)j * Sk + i] * w->du[j];
                dk[i] += acc;
            }
#if GDN_ORACLE_MUTATION == 7
            /* planted: dg taken from dM before the du update */
            if (io->dg) {
                double *dgr = io->dg + ix_tok(p, s, t, p->H_v, h, G);
                for (int i = 0; i < G; i++) dgr[i] = 0.0;
                for (int j = 0; j < Sv; j++)
                    for (int i = 0; i < Sk; i++)
                        dgr[p->kda ? i : 0] += dM[(size_t)j * Sk + i] * Mp[(size_t)j * Sk + i];
            }
#endif
#if GDN_ORACLE_MUTATION != 3
            /* dM += du k^T */
            for (int j = 0; j < Sv; j++)
                for (int i = 0; i < Sk; i++) dM[(size_t)j * Sk + i] += w->du[j] * ti.k[i];
#endif
            /* dg = sum_j dM .* Mp (per column, or over everything for the scalar gate) */
            if (io->dg && !MUT(7)) {
                double *dgr = io->dg + ix_tok(p, s, t, p->H_v, h, G);
                if (p->kda) {
                    for (int i = 0; i < Sk; i++) {
                        double acc = 0.0;
                        for (int j = 0; j < Sv; j++)
                            acc += dM[(size_t)j * Sk + i] * Mp[(size_t)j * Sk + i];
                        dgr[i] = acc;
                    }
                } else {
                    double acc = 0.0;
                    for (int j = 0; j < Sv; j++)
                        for (int i = 0; i < Sk; i++)
                            acc += dM[(size_t)j * Sk + i] * Mp[(size_t)j * Sk + i];
                    dgr[0] = acc;
                }
            }
            /* dM = dM .* a */
#if GDN_ORACLE_MUTATION != 5 /* planted (5): decay dropped from the state gradient */
            for (int j = 0; j < Sv; j++)
                for (int i = 0; i < Sk; i++) dM[(size_t)j * Sk + i] *= gate_at(p, &ti, i);
#endif
        }
    }
    if (io->dstate) memcpy(io->dstate + ix_state(p, s, h), dM, SS * sizeof(double));
}

/* ---------------------------------------------------------------- drivers */

typedef struct {
    const gdn_oracle_problem *p;
    const gdn_oracle_io *io;
    int backward, C;
    int next; /* next (s, hk) pair to take */
    pthread_mutex_t lock;
    int failed;
} job;

static void run_pair(job *jb, int pair, bwd_scratch *w, double *M) {
    const gdn_oracle_problem *p = jb->p;
    const gdn_oracle_io *io = jb->io;
    int s = pair / p->H_k, hk = pair % p->H_k;
    if (jb->backward) {
        /* zero this key head's dq/dk rows, then accumulate its value heads in increasing h */
        for (int t = 0; t < p->T; t++) {
            memset(io->dq + ix_tok(p, s, t, p->H_k, hk, p->S_k), 0, sizeof(double) * p->S_k);
            memset(io->dk + ix_tok(p, s, t, p->H_k, hk, p->S_k), 0, sizeof(double) * p->S_k);
        }
    }
    for (int h = 0; h < p->H_v; h++) {
        if (key_head_of(p, h) != hk) continue;
        if (jb->backward)
            backward_unit(p, io, s, h, jb->C, w);
        else
            forward_unit(p, io, s, h, M);
    }
}

static void *worker(void *arg) {
    job *jb = (job *)arg;
    const gdn_oracle_problem *p = jb->p;
    size_t SS = (size_t)p->S_v * p->S_k;
    int C = jb->C;
    int n_ck_max = p->T > 0 ? (p->T + C - 1) / C : 0;
    bwd_scratch w;
    memset(&w, 0, sizeof(w));
    double *M = malloc(SS * sizeof(double));
    int ok = M != NULL;
    if (jb->backward) {
        w.ck = malloc((n_ck_max + 1) * SS * sizeof(double));
        w.states = malloc(((size_t)C + 1) * SS * sizeof(double));
        w.Mp = malloc((size_t)C * SS * sizeof(double));
        w.u = malloc((size_t)C * p->S_v * sizeof(double));
        w.e = malloc((size_t)C * p->S_v * sizeof(double));
        w.dM = malloc(SS * sizeof(double));
        w.dd = malloc(p->S_v * sizeof(double));
        w.du = malloc(p->S_v * sizeof(double));
        w.delta = malloc(p->S_v * sizeof(double));
        w.sgy = malloc(p->S_v * sizeof(double));
        ok = ok && w.ck && w.states && w.Mp && w.u && w.e && w.dM && w.dd && w.du && w.delta &&
             w.sgy;
    }
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        int pair = jb->next++;
        if (!ok) jb->failed = 1;
        pthread_mutex_unlock(&jb->lock);
        if (!ok || pair >= p->n_seqs * p->H_k) break;
        run_pair(jb, pair, &w, M);
    }
    free(M);
    free(w.ck); free(w.states); free(w.Mp); free(w.u); free(w.e);
    free(w.dM); free(w.dd); free(w.du); free(w.delta); free(w.sgy);
    return NULL;
}

static int check_problem(const gdn_oracle_problem *p) {
    if (p->n_seqs < 0 || p->T < 0 || p->H_k <= 0 || p->H_v <= 0 || p->S_k <= 0 || p->S_v <= 0)
        return -1;
    if (p->H_v % p->H_k != 0) return -1;
    if (p->seq_lens)
        for (int s = 0; s < p->n_seqs; s++)
            if (p->seq_lens[s] < 0 || p->seq_lens[s] > p->T) return -1;
    return 0;
}

static int run(const gdn_oracle_problem *p, const gdn_oracle_io *io, int backward, int threads) {
    if (check_problem(p)) return -1;
    job jb;
    jb.p = p;
    jb.io = io;
    jb.backward = backward;
    jb.C = p->C > 0 ? p->C : gdn_oracle_default_C(p->T);
    jb.next = 0;
    jb.failed = 0;
    pthread_mutex_init(&jb.lock, NULL);
    int pairs = p->n_seqs * p->H_k;
    if (threads < 1) threads = 1;
    if (threads > pairs) threads = pairs > 0 ? pairs : 1;
    pthread_t *tid = malloc(sizeof(pthread_t) * threads);
    if (!tid) return -2;
    int started = 0;
    for (int i = 1; i < threads; i++)
        if (pthread_create(&tid[i], NULL, worker, &jb) == 0) started = i;
        else break;
    worker(&jb);
    for (int i = 1; i <= started; i++) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&jb.lock);
    return jb.failed ? -2 : 0;
}

/* Forward: writes y and state_out (either may be NULL). Returns 0, -1 bad problem, -2 no memory. */
int gdn_oracle_fwd(const gdn_oracle_problem *p, const gdn_oracle_io *io, int threads) {
    return run(p, io, 0, threads);
}

/* Backward: writes dq, dk, dv, dg, dbeta, dstate (dq and dk are required). */
int gdn_oracle_bwd(const gdn_oracle_problem *p, const gdn_oracle_io *io, int threads) {
    if (!io->dq || !io->dk || !io->gy) return -1;
    return run(p, io, 1, threads);
}
