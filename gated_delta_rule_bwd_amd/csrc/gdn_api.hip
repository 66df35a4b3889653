// gdn_api.hip -- host side of the C ABI declared in include/gdn.h: argument validation,
// workspace sizing and kernel launches.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kRingSlots = 4;   // piece slots of the head-128 chain's results on long sequences

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_sqrt(int64_t T) {
    if (T <= 1) return 1;
    int64_t c = (int64_t)std::ceil(std::sqrt((double)T));
    while (c > 1 && (c - 1) * (c - 1) >= T) --c;
    while (c * c < T) ++c;
    return (int)c;
}

struct Plan {
    int C = 1;         // effective checkpoint interval
    int n_ck_max = 1;  // snapshots per unit
    int G = 1;         // gate width
    int64_t units = 0;
    bool s128 = false;   // head size 128: matrix-core kernels
    bool parts = false;  // small heads: dq/dk go through per-value-head partials
    size_t off_snap = 0, off_seg = 0, off_e = 0, off_pq = 0, off_pk = 0;
    size_t off_wm = 0, off_wf = 0, off_c = 0, off_g1 = 0, off_g2 = 0, off_dbp = 0, off_p3 = 0,
           off_anc = 0, off_carry = 0;
    int nslab = 1;       // head size 128: row slabs per unit of the forward and the chain
    int piece = 1;       // head size 128: tokens per piece of the pipelined passes (a multiple of C)
    int np = 1;          // pieces
    int ring = 0;        // piece slots of the chain's results (0: one buffer for every token)
    int pb_T = 0;        // tokens per sequence of such a buffer
    size_t sz_g = 0, sz_dbp = 0, sz_p3 = 0;   // floats per slot
    // half-precision inputs: their fp32 copies, contiguous [n_seqs][T][heads][width] each
    size_t off_in = 0, in_q = 0, in_k = 0, in_v = 0, in_g = 0, in_b = 0, in_gy = 0;
    size_t total = 0;
};

bool strides_ok(const gdn_strides &s) { return s.seq >= 0 && s.tok >= 0 && s.head >= 0; }

int validate(const gdn_problem *p) {
    if (!p) return GDN_ERR_ARG;
    if (p->n_seqs < 0 || p->T < 0 || p->H_k <= 0 || p->H_v <= 0 || p->S_k <= 0 ||
        p->S_v <= 0 || p->C < 0)
        return GDN_ERR_ARG;
    if (p->gate != GDN_GATE_SCALAR && p->gate != GDN_GATE_KDA) return GDN_ERR_ARG;
    if (p->dtype != GDN_DTYPE_F32 && p->dtype != GDN_DTYPE_F16 && p->dtype != GDN_DTYPE_BF16)
        return GDN_ERR_ARG;
    if (!std::isfinite(p->scale)) return GDN_ERR_ARG;
    if (p->seq_lens)
        for (int s = 0; s < p->n_seqs; ++s)
            if (p->seq_lens[s] < 0 || p->seq_lens[s] > p->T) return GDN_ERR_ARG;
    if (p->H_v % p->H_k != 0) return GDN_ERR_UNSUPPORTED;
    auto size_ok = [](int x) { return x == 16 || x == 32 || x == 64 || x == 128; };
    if (!size_ok(p->S_k) || !size_ok(p->S_v)) return GDN_ERR_UNSUPPORTED;
    const gdn_strides *all[] = {&p->q, &p->k, &p->v, &p->g, &p->beta, &p->gy, &p->y};
    for (auto *s : all)
        if (!strides_ok(*s)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

Plan make_plan(const gdn_problem *p) {
    Plan pl;
    const int64_t S = p->S_v, SK = p->S_k, SV = p->S_v;   // S only where SK == SV == 128
    pl.C = p->C > 0 ? std::min(p->C, std::max(p->T, 1)) : ceil_sqrt(p->T);
    pl.s128 = SK == 128 && SV == 128;
    // head size 128: checkpoints fall on the 16-token blocks of the matrix-core kernels, so
    // the interval is rounded up to a multiple of 16 and every interval gives the same bits
    if (pl.s128) pl.C = (pl.C + 15) / 16 * 16;
    pl.n_ck_max = std::max(1, (p->T + pl.C - 1) / pl.C);
    pl.G = p->gate == GDN_GATE_KDA ? p->S_k : 1;
    pl.units = (int64_t)p->n_seqs * p->H_v;
    size_t off = 0;
    // half-precision inputs of the small-head kernels are widened into fp32 copies first
    // (offsets in floats from off_in); the head-128 kernels read them as they are
    if (p->dtype != GDN_DTYPE_F32 && !pl.s128) {
        const size_t nt = (size_t)p->n_seqs * p->T;
        pl.off_in = off;
        pl.in_q = 0;
        pl.in_k = pl.in_q + nt * p->H_k * SK;
        pl.in_v = pl.in_k + nt * p->H_k * SK;
        pl.in_g = pl.in_v + nt * p->H_v * SV;
        pl.in_b = pl.in_g + nt * p->H_v * pl.G;
        pl.in_gy = pl.in_b + nt * p->H_v;
        off = align_up(off + (pl.in_gy + nt * p->H_v * SV) * sizeof(float));
    }
    pl.off_snap = off;
    off = align_up(off + (size_t)pl.units * pl.n_ck_max * SV * SK * sizeof(float));
    if (pl.s128) {
        const size_t tok_rows = (size_t)p->n_seqs * p->T * p->H_v;
        const size_t nblk = (size_t)(p->T + 15) / 16;
        pl.off_wm = off;   // block matrices Bm, Te, Tb
        off = align_up(off + (size_t)p->n_seqs * nblk * p->H_v * 3 * 256 * sizeof(float));
        pl.off_wf = off;   // block flags
        off = align_up(off + (size_t)p->n_seqs * nblk * p->H_v * sizeof(int32_t));
        pl.off_c = off;    // running gate products within blocks
        off = align_up(off + tok_rows * pl.G * sizeof(float));
        pl.off_e = off;
        off = align_up(off + tok_rows * S * sizeof(float));
        // too few units to fill the chip with one workgroup each: the forward and the chain split
        // every unit's rows into two slabs, whose sums over rows are kept apart
        pl.nslab = pl.units <= 128 ? 2 : 1;
        // pieces of about 1024 tokens, at most 16, each a whole number of checkpoint segments
        const int64_t np = std::min<int64_t>(16, std::max<int64_t>(1, p->T / 1024));
        const int64_t per = (p->T + np - 1) / np;
        pl.piece = (int)std::max<int64_t>(pl.C, (per + pl.C - 1) / pl.C * pl.C);
        pl.np = (p->T + pl.piece - 1) / pl.piece;
        // the chain's results for the column pass (G1, G2, dbeta per slab, P3): for the whole
        // sequence, or, beyond kRingSlots pieces, in a ring of that many piece slots
        pl.ring = pl.np > kRingSlots ? kRingSlots : 0;
        pl.pb_T = pl.ring ? pl.piece : (int)nblk * 16;
        const size_t pb_rows = (size_t)p->n_seqs * pl.pb_T * p->H_v, slots = pl.ring ? pl.ring : 1;
        pl.sz_g = pb_rows / 16 * pl.nslab * 256;
        pl.sz_dbp = pl.nslab > 1 ? pb_rows * pl.nslab : 0;
        pl.sz_p3 = pb_rows * S;
        pl.off_g1 = off;   // Grams G1 and G2 of the blocks, per slab
        off = align_up(off + slots * pl.sz_g * sizeof(float));
        pl.off_g2 = off;
        off = align_up(off + slots * pl.sz_g * sizeof(float));
        pl.off_dbp = off;  // dbeta per slab
        off = align_up(off + slots * pl.sz_dbp * sizeof(float));
        pl.off_p3 = off;   // the chain's column sums X'^T delta per token
        off = align_up(off + slots * pl.sz_p3 * sizeof(float));
        pl.off_anc = off;  // dg at the first token of every checkpoint segment
        off = align_up(off + (size_t)pl.units * pl.n_ck_max * S * sizeof(float));
        pl.off_carry = off;   // the state or gradient between the pieces of a pipelined pass
        off = align_up(off + (size_t)pl.units * S * S * sizeof(float));
        // dq and dk go straight to the outputs: the column pass sums the value heads of a key
        // head in one workgroup
        pl.parts = false;
        pl.total = off;
        return pl;
    }
    pl.parts = p->H_v != p->H_k;
    pl.off_seg = off;
    off = align_up(off + (size_t)pl.units * pl.C * SV * SK * sizeof(float));
    pl.off_e = off;
    off = align_up(off + (size_t)pl.units * pl.C * SV * sizeof(float));
    if (pl.parts) {
        const size_t part = (size_t)p->n_seqs * p->T * p->H_v * SK * sizeof(float);
        pl.off_pq = off;
        off = align_up(off + part);
        pl.off_pk = off;
        off = align_up(off + part);
    }
    pl.total = off;
    return pl;
}

// Byte range [lo, hi) covered by a strided per-token tensor (empty when any extent is 0).
struct Range {
    uintptr_t lo = 0, hi = 0;
};

Range span_tok(const void *base, const gdn_strides &s, int64_t n, int64_t T, int64_t H,
               int64_t W, int64_t esize = sizeof(float)) {
    Range r;
    if (!base || n <= 0 || T <= 0 || H <= 0 || W <= 0) return r;
    const int64_t last = (n - 1) * s.seq + (T - 1) * s.tok + (H - 1) * s.head + W;
    r.lo = (uintptr_t)base;
    r.hi = r.lo + (uintptr_t)(last * esize);
    return r;
}

Range span_flat(const void *base, int64_t count_floats) {
    Range r;
    if (!base || count_floats <= 0) return r;
    r.lo = (uintptr_t)base;
    r.hi = r.lo + (uintptr_t)count_floats * sizeof(float);
    return r;
}

Range span_bytes(const void *base, size_t bytes) {
    Range r;
    if (!base || bytes == 0) return r;
    r.lo = (uintptr_t)base;
    r.hi = r.lo + bytes;
    return r;
}

bool overlap(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// A written strided view must not map two elements onto one address: sort the dimensions
// by stride and require each stride to exceed the span of the dimensions inside it.
bool non_self_overlapping(const gdn_strides &s, int64_t n, int64_t T, int64_t H, int64_t W) {
    struct Dim {
        int64_t stride, extent;
    } d[3] = {{s.seq, n}, {s.tok, T}, {s.head, H}};
    if (n <= 0 || T <= 0 || H <= 0 || W <= 0) return true;   // no element at all
    std::sort(d, d + 3, [](const Dim &x, const Dim &y) { return x.stride < y.stride; });
    int64_t span = W;  // innermost: W contiguous floats
    for (auto &x : d) {
        if (x.extent <= 1) continue;
        if (x.stride < span) return false;
        span = x.stride * (x.extent - 1) + span;
    }
    return true;
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
int64_t in_esize(const gdn_problem *p) { return p->dtype == GDN_DTYPE_F32 ? 4 : 2; }
bool aligned_in(const gdn_problem *p, const void *x) {
    return ((uintptr_t)x & (uintptr_t)(in_esize(p) - 1)) == 0;
}
gdn_strides contiguous(int64_t T, int64_t H, int64_t W) { return gdn_strides{T * H * W, H * W, W}; }

void fill_lens(const gdn_problem *p, int s0, int count, int32_t *dst) {
    for (int i = 0; i < count; ++i) dst[i] = p->seq_lens ? p->seq_lens[s0 + i] : p->T;
}

int device_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_DEVICE; }

// Argument block of the head-128 matrix-core kernels for sequences s0 .. s0 + cnt - 1.
gdn::Mf128Args mf_args(const gdn_problem *p, const Plan &pl, void *ws, int s0, int cnt) {
    gdn::Mf128Args a;
    std::memset(&a, 0, sizeof(a));
    char *w = (char *)ws;
    a.snap = (float *)(w + pl.off_snap);
    a.wmat = (float *)(w + pl.off_wm);
    a.wflag = (int32_t *)(w + pl.off_wf);
    a.cbuf = (float *)(w + pl.off_c);
    a.ebuf = (float *)(w + pl.off_e);
    a.g1buf = (float *)(w + pl.off_g1);
    a.g2buf = (float *)(w + pl.off_g2);
    a.dbp = (float *)(w + pl.off_dbp);
    a.nslab = pl.nslab;
    a.p3buf = (float *)(w + pl.off_p3);
    a.pb_T = pl.pb_T;
    a.pb_t0 = 0;
    a.anc = (float *)(w + pl.off_anc);
    a.carry = (float *)(w + pl.off_carry);
    a.t_lo = 0;
    a.t_hi = p->T;
    a.sq = p->q; a.sk = p->k; a.sv = p->v; a.sg = p->g; a.sb = p->beta; a.sgy = p->gy; a.sy = p->y;
    a.s_base = s0; a.n_seqs_launch = cnt;
    a.T = p->T; a.H_k = p->H_k; a.H_v = p->H_v; a.C = pl.C; a.n_ck_max = pl.n_ck_max;
    a.kda = p->gate == GDN_GATE_KDA ? 1 : 0; a.dtype = p->dtype;
    a.scale = p->scale;
    fill_lens(p, s0, cnt, a.lens);
    return a;
}

// Second stream and events of the pipelined head-128 passes, one set per device, created on
// first use (default priority) and kept until the process ends.  A call holds its device's lock
// while it enqueues, so calls from several host threads take turns.
constexpr int kMaxSideDevices = 64, kSideEvents = 64;
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t ev[kSideEvents] = {};
    int next = 0;
    hipEvent_t take() {
        hipEvent_t e = ev[next];
        next = (next + 1) % kSideEvents;
        return e;
    }
};
std::mutex g_side_mu[kMaxSideDevices];
Side g_side[kMaxSideDevices];

int side_for(hipStream_t st, std::unique_lock<std::mutex> &lk, Side **out) {
    int dev = -1, cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_DEVICE;
    if (hipStreamGetDevice(st, &dev) != hipSuccess) dev = cur;
    if (dev < 0 || dev >= kMaxSideDevices) return GDN_ERR_DEVICE;
    lk = std::unique_lock<std::mutex>(g_side_mu[dev]);
    Side &sd = g_side[dev];
    if (!sd.s) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GDN_ERR_DEVICE;
        bool ok = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; ok && i < kSideEvents; ++i)
            ok = hipEventCreateWithFlags(&sd.ev[i], hipEventDisableTiming) == hipSuccess;
        if (dev != cur && hipSetDevice(cur) != hipSuccess) ok = false;
        if (!ok) return GDN_ERR_DEVICE;
    }
    *out = &sd;
    return GDN_OK;
}
// work enqueued on `to` from now on waits for everything enqueued on `from` so far
int order_after(Side &sd, hipStream_t from, hipStream_t to) {
    hipEvent_t e = sd.take();
    if (hipEventRecord(e, from) != hipSuccess || hipStreamWaitEvent(to, e, 0) != hipSuccess) return GDN_ERR_DEVICE;
    return GDN_OK;
}
gdn::Mf128Args piece_of(gdn::Mf128Args a, int t_lo, int t_hi) {
    a.t_lo = t_lo;
    a.t_hi = t_hi;
    return a;
}

// Block preparation and forward scan of the head-128 kernels (y null: snapshots and errors
// only).  Pipelined: the token axis in pieces, the preparation of the next piece on the second
// stream while the forward walks the current one on st.
int mf_forward(const gdn_problem *p, const Plan &pl, void *ws, const void *q, const void *k,
               const void *v, const void *g, const void *beta, const float *state0, float *y,
               float *state_out, hipStream_t st, bool pipelined) {
    const int T = p->T, PT = pl.piece, np = (T + PT - 1) / PT;
    for (int s0 = 0; s0 < p->n_seqs; s0 += gdn::kMaxSeqsPerLaunch) {
        const int cnt = std::min(gdn::kMaxSeqsPerLaunch, p->n_seqs - s0);
        gdn::Mf128Args a = mf_args(p, pl, ws, s0, cnt);
        a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state0 = state0;
        a.y = y; a.state_out = state_out;
        if (!pipelined || np <= 1) {
            int rc = device_status(gdn::launch_prep128(a, st));
            if (rc == GDN_OK) rc = device_status(gdn::launch_fwd_mf(a, st));
            if (rc != GDN_OK) return rc;
            continue;
        }
        std::unique_lock<std::mutex> lk;
        Side *sd = nullptr;
        int rc = side_for(st, lk, &sd);
        if (rc == GDN_OK) rc = order_after(*sd, st, sd->s);
        if (rc == GDN_OK) rc = device_status(gdn::launch_prep128(piece_of(a, 0, PT), st));
        for (int j = 0; rc == GDN_OK && j < np; ++j) {
            if (j + 1 < np)
                rc = device_status(gdn::launch_prep128(piece_of(a, (j + 1) * PT, std::min(T, (j + 2) * PT)), sd->s));
            if (rc == GDN_OK && j > 0) rc = order_after(*sd, sd->s, st);   // piece j prepared
            if (rc == GDN_OK) rc = device_status(gdn::launch_fwd_mf(piece_of(a, j * PT, std::min(T, (j + 1) * PT)), st));
        }
        if (rc != GDN_OK) return rc;
    }
    return GDN_OK;
}

// The chain and the column sums of the head-128 backward.  Pipelined: the chain walks the pieces
// from the last on st, and the column sums of each piece run on the second stream as soon as the
// chain has passed it.  With a ring of piece slots the chain's results for piece i (counted in
// processing order) go to slot i % ring, and the chain of piece i waits for the column sums of
// piece i - ring, which read that slot.
int mf_backward(const gdn_problem *p, const Plan &pl, void *ws, gdn::Mf128Args a, hipStream_t st,
                bool pipelined) {
    const int T = p->T, PT = pl.piece, np = pl.np;
    for (int s0 = 0; s0 < p->n_seqs; s0 += gdn::kMaxSeqsPerLaunch) {
        const int cnt = std::min(gdn::kMaxSeqsPerLaunch, p->n_seqs - s0);
        gdn::Mf128Args b = mf_args(p, pl, ws, s0, cnt);
        b.q = a.q; b.k = a.k; b.v = a.v; b.g = a.g; b.beta = a.beta; b.gy = a.gy;
        b.state0 = a.state0; b.dstate_out = a.dstate_out;
        b.dq = a.dq; b.dk = a.dk; b.dv = a.dv; b.dg = a.dg; b.dbeta = a.dbeta; b.dstate = a.dstate;
        int rc = device_status(gdn::launch_zero_anc(b, st));
        for (int k = 0; rc == GDN_OK && k < (pl.ring ? pl.ring : 1); ++k) {   // P3 of every slot
            gdn::Mf128Args bk = b;
            bk.p3buf += k * pl.sz_p3;
            rc = device_status(gdn::launch_zero_p3(bk, st));
        }
        if (rc != GDN_OK) return rc;
        if (np <= 1 || (!pipelined && !pl.ring)) {   // one launch of each over every token
            rc = device_status(gdn::launch_chain(b, st));
            if (rc == GDN_OK) rc = device_status(gdn::launch_colsum(b, st));
            if (rc != GDN_OK) return rc;
            continue;
        }
        std::unique_lock<std::mutex> lk;
        Side *sd = nullptr;
        if (pipelined) rc = side_for(st, lk, &sd);
        hipEvent_t done[gdn::kMaxPieces] = {};   // column sums of piece i finished (ring reuse)
        for (int i = 0; rc == GDN_OK && i < np; ++i) {
            const int j = np - 1 - i;
            gdn::Mf128Args bj = piece_of(b, j * PT, std::min(T, (j + 1) * PT));
            if (pl.ring) {
                const int slot = i % pl.ring;
                bj.g1buf += slot * pl.sz_g;
                bj.g2buf += slot * pl.sz_g;
                bj.dbp += slot * pl.sz_dbp;
                bj.p3buf += slot * pl.sz_p3;
                bj.pb_t0 = j * PT;
                if (pipelined && i >= pl.ring && hipStreamWaitEvent(st, done[i - pl.ring], 0) != hipSuccess)
                    rc = GDN_ERR_DEVICE;
            }
            if (rc == GDN_OK) rc = device_status(gdn::launch_chain(bj, st));
            if (!pipelined) {
                if (rc == GDN_OK) rc = device_status(gdn::launch_colsum(bj, st));
                // the slot's P3 back to zeros for the piece that reuses it (two slabs add into it)
                if (rc == GDN_OK && pl.ring && i + pl.ring < np) rc = device_status(gdn::launch_zero_p3(bj, st));
                continue;
            }
            if (rc == GDN_OK) rc = order_after(*sd, st, sd->s);
            // The slot of the previous piece, whose column sums have ended, back to zeros for the
            // piece that reuses it (two slabs add their P3 into it).  Enqueued between the wait
            // for this chain and the column sums (also where no piece reuses the slot), it lets
            // the next chain launch (queued right behind this one on st) take the CUs this chain
            // frees before the column sums do.
            if (rc == GDN_OK && pl.ring && i >= 1) {
                gdn::Mf128Args prev = bj;
                prev.p3buf = b.p3buf + ((i - 1) % pl.ring) * pl.sz_p3;
                rc = device_status(gdn::launch_zero_p3_all(prev, sd->s));
                done[i - 1] = sd->take();
                if (rc == GDN_OK && hipEventRecord(done[i - 1], sd->s) != hipSuccess) rc = GDN_ERR_DEVICE;
            }
            if (rc == GDN_OK) rc = device_status(gdn::launch_colsum(bj, sd->s));
        }
        if (rc == GDN_OK && pipelined) rc = order_after(*sd, sd->s, st);   // st waits for the last column sums
        if (rc != GDN_OK) return rc;
    }
    return GDN_OK;
}

// Widen the given half-precision inputs into the workspace (a null source is skipped but
// still redirected: its copy is already there) and describe the copies in pc: contiguous
// fp32 tensors, dtype fp32.
int widen_inputs(const gdn_problem *p, const Plan &pl, void *ws, const void *q, const void *k,
                 const void *v, const void *g, const void *beta, const void *gy, hipStream_t st,
                 gdn_problem &pc, const float *&qf, const float *&kf, const float *&vf,
                 const float *&gf, const float *&bf, const float **gyf) {
    float *base = (float *)((char *)ws + pl.off_in);
    const int64_t n = p->n_seqs, T = p->T, SK = p->S_k, SV = p->S_v;
    struct Job {
        const void *src;
        const gdn_strides *st;
        size_t off;
        int64_t H, W;
        gdn_strides *dst_st;
        const float **dst;
    } jobs[] = {{q, &p->q, pl.in_q, p->H_k, SK, &pc.q, &qf},
                {k, &p->k, pl.in_k, p->H_k, SK, &pc.k, &kf},
                {v, &p->v, pl.in_v, p->H_v, SV, &pc.v, &vf},
                {g, &p->g, pl.in_g, p->H_v, pl.G, &pc.g, &gf},
                {beta, &p->beta, pl.in_b, p->H_v, 1, &pc.beta, &bf},
                {gy, &p->gy, pl.in_gy, p->H_v, SV, &pc.gy, gyf}};
    for (auto &j : jobs) {
        if (!j.dst) continue;   // gy of the forward
        if (j.src) {
            gdn::WidenArgs w;
            w.src = (const uint16_t *)j.src;
            w.st = *j.st;
            w.dst = base + j.off;
            w.n = n; w.T = T; w.H = j.H; w.W = j.W;
            w.bf16 = p->dtype == GDN_DTYPE_BF16;
            const int rc = device_status(gdn::launch_widen(w, st));
            if (rc != GDN_OK) return rc;
        }
        *j.dst_st = contiguous(T, j.H, j.W);
        *j.dst = base + j.off;
    }
    pc.dtype = GDN_DTYPE_F32;
    return GDN_OK;
}

// Workspace of gdn_bwd_noalloc: one copy per GPU, held until the process ends.  Host code uses
// it only through the device address looked up below, never through the array's name.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the scratch array on the device of stream st (looked up once per device,
// with that device current).
int scratch_address(hipStream_t st, void **out) {
    int dev = -1, cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_DEVICE;
    if (hipStreamGetDevice(st, &dev) != hipSuccess) dev = cur;
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GDN_ERR_DEVICE;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return GDN_ERR_DEVICE;
        if (e != hipSuccess || !ptr) return GDN_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported problem";
        case GDN_ERR_WORKSPACE: return "workspace too small";
        case GDN_ERR_DEVICE: return "device launch failed";
    }
    return "unknown status";
}

size_t gdn_workspace_size(const gdn_problem *p) {
    if (validate(p) != GDN_OK) return 0;
    return make_plan(p).total;
}

size_t gdn_grad_packed_floats(const gdn_problem *p, size_t offsets[6]) {
    if (validate(p) != GDN_OK) return 0;
    const size_t n = p->n_seqs, T = p->T, Hk = p->H_k, Hv = p->H_v, Sk = p->S_k, Sv = p->S_v;
    const size_t G = p->gate == GDN_GATE_KDA ? Sk : 1;
    const size_t sizes[6] = {n * T * Hk * Sk, n * T * Hk * Sk, n * T * Hv * Sv,
                             n * T * Hv * G,  n * T * Hv,      n * Hv * Sv * Sk};
    size_t off = 0;
    for (int i = 0; i < 6; ++i) {
        if (offsets) offsets[i] = off;
        off += sizes[i];
    }
    return off;
}

int gdn_fwd(const gdn_problem *p, const void *q_in, const void *k_in, const void *v_in,
            const void *g_in, const void *beta_in, const float *state0, float *y,
            float *state_out, void *ws, size_t ws_bytes, gdn_stream_t stream) {
    int rc = validate(p);
    if (rc != GDN_OK) return rc;
    const Plan pl = make_plan(p);
    const int64_t n = p->n_seqs, T = p->T, Hk = p->H_k, Hv = p->H_v, SK = p->S_k, SV = p->S_v;
    if (!q_in || !k_in || !v_in || !g_in || !beta_in || !state0 || !y || !state_out) return GDN_ERR_ARG;
    const void *ins[] = {q_in, k_in, v_in, g_in, beta_in};
    for (auto *x : ins)
        if (!aligned_in(p, x)) return GDN_ERR_UNSUPPORTED;
    const void *ptrs[] = {state0, y, state_out};
    for (auto *x : ptrs)
        if (!aligned4(x)) return GDN_ERR_UNSUPPORTED;
    if (ws_bytes < pl.total) return GDN_ERR_WORKSPACE;
    if (!ws || ((uintptr_t)ws % 16) != 0) return GDN_ERR_ARG;
    if (!non_self_overlapping(p->y, n, T, Hv, SV)) return GDN_ERR_ARG;

    const int64_t es = in_esize(p);
    const Range in[] = {span_tok(q_in, p->q, n, T, Hk, SK, es), span_tok(k_in, p->k, n, T, Hk, SK, es),
                        span_tok(v_in, p->v, n, T, Hv, SV, es), span_tok(g_in, p->g, n, T, Hv, pl.G, es),
                        span_tok(beta_in, p->beta, n, T, Hv, 1, es), span_flat(state0, n * Hv * SV * SK)};
    const Range out[] = {span_tok(y, p->y, n, T, Hv, SV), span_flat(state_out, n * Hv * SV * SK),
                         span_bytes(ws, pl.total)};
    for (auto &o : out)
        for (auto &i : in)
            if (overlap(o, i)) return GDN_ERR_ARG;
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_ARG;

    if (pl.s128)   // head size 128: the matrix-core kernels read every input type directly
        return mf_forward(p, pl, ws, q_in, k_in, v_in, g_in, beta_in, state0, y, state_out,
                          (hipStream_t)stream, true);

    // half-precision inputs: widened into the workspace, then the fp32 path on the copies
    gdn_problem pc = *p;
    const float *q = (const float *)q_in, *k = (const float *)k_in, *v = (const float *)v_in;
    const float *g = (const float *)g_in, *beta = (const float *)beta_in;
    if (p->dtype != GDN_DTYPE_F32) {
        rc = widen_inputs(p, pl, ws, q_in, k_in, v_in, g_in, beta_in, nullptr, (hipStream_t)stream, pc,
                          q, k, v, g, beta, nullptr);
        if (rc != GDN_OK) return rc;
    }
    p = &pc;

    gdn::FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state0 = state0;
    a.y = y; a.state_out = state_out;
    a.snap = (float *)((char *)ws + pl.off_snap);
    a.sq = p->q; a.sk = p->k; a.sv = p->v; a.sg = p->g; a.sb = p->beta; a.sy = p->y;
    a.T = p->T; a.H_k = p->H_k; a.H_v = p->H_v; a.C = pl.C; a.n_ck_max = pl.n_ck_max;
    a.scale = p->scale;
    a.dtype = p->dtype;
    for (int s0 = 0; s0 < p->n_seqs; s0 += gdn::kMaxSeqsPerLaunch) {
        const int cnt = std::min(gdn::kMaxSeqsPerLaunch, p->n_seqs - s0);
        a.s_base = s0;
        fill_lens(p, s0, cnt, a.lens);
        const bool kda = p->gate == GDN_GATE_KDA;
        rc = device_status(gdn::launch_fwd(a, (int)SK, (int)SV, kda, cnt, (hipStream_t)stream));
        if (rc != GDN_OK) return rc;
    }
    return GDN_OK;
}

}  // extern "C"

namespace {

// gdn_bwd; pipelined: the head-128 passes may use the device's second stream
int bwd_impl(const gdn_problem *p, const void *q_in, const void *k_in, const void *v_in,
             const void *g_in, const void *beta_in, const float *state0, const void *gy_in,
             const float *dstate_out, float *grad_packed, void *ws, size_t ws_bytes,
             unsigned flags, gdn_stream_t stream, bool pipelined) {
    int rc = validate(p);
    if (rc != GDN_OK) return rc;
    if (flags & ~GDN_BWD_REUSE_SNAPSHOTS) return GDN_ERR_ARG;
    const Plan pl = make_plan(p);
    const int64_t n = p->n_seqs, T = p->T, Hk = p->H_k, Hv = p->H_v, SK = p->S_k, SV = p->S_v;
    if (!q_in || !k_in || !v_in || !g_in || !beta_in || !state0 || !gy_in || !grad_packed)
        return GDN_ERR_ARG;
    const void *ins[] = {q_in, k_in, v_in, g_in, beta_in, gy_in};
    for (auto *x : ins)
        if (!aligned_in(p, x)) return GDN_ERR_UNSUPPORTED;
    const void *ptrs[] = {state0, dstate_out, grad_packed};
    for (auto *x : ptrs)
        if (x && !aligned4(x)) return GDN_ERR_UNSUPPORTED;
    if (ws_bytes < pl.total) return GDN_ERR_WORKSPACE;
    if (!ws || ((uintptr_t)ws % 16) != 0) return GDN_ERR_ARG;

    size_t off[6];
    const size_t total = gdn_grad_packed_floats(p, off);
    const int64_t es = in_esize(p);
    const Range in[] = {span_tok(q_in, p->q, n, T, Hk, SK, es),      span_tok(k_in, p->k, n, T, Hk, SK, es),
                        span_tok(v_in, p->v, n, T, Hv, SV, es),      span_tok(g_in, p->g, n, T, Hv, pl.G, es),
                        span_tok(beta_in, p->beta, n, T, Hv, 1, es), span_flat(state0, n * Hv * SV * SK),
                        span_tok(gy_in, p->gy, n, T, Hv, SV, es),    span_flat(dstate_out, n * Hv * SV * SK)};
    const Range outg = span_flat(grad_packed, (int64_t)total);
    const Range wsr = span_bytes(ws, pl.total);
    for (auto &i : in)
        if (overlap(outg, i) || overlap(wsr, i)) return GDN_ERR_ARG;
    if (overlap(outg, wsr)) return GDN_ERR_ARG;

    float *dq = grad_packed + off[0], *dk = grad_packed + off[1], *dv = grad_packed + off[2];
    float *dg = grad_packed + off[3], *dbeta = grad_packed + off[4], *dstate = grad_packed + off[5];

    if (pl.s128) {   // head size 128: matrix-core kernels, every input type read directly
        if (!(flags & GDN_BWD_REUSE_SNAPSHOTS)) {
            rc = mf_forward(p, pl, ws, q_in, k_in, v_in, g_in, beta_in, state0, nullptr, nullptr,
                            (hipStream_t)stream, pipelined);
            if (rc != GDN_OK) return rc;
        }
        gdn::Mf128Args a;
        std::memset(&a, 0, sizeof(a));
        a.q = q_in; a.k = k_in; a.v = v_in; a.g = g_in; a.beta = beta_in; a.gy = gy_in;
        a.state0 = state0; a.dstate_out = dstate_out;
        a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dstate = dstate;
        return mf_backward(p, pl, ws, a, (hipStream_t)stream, pipelined);
    }

    // half-precision inputs of the small-head kernels: gy widened into the workspace, and q, k,
    // v, g, beta too unless the forward on the same inputs left their copies there
    // (GDN_BWD_REUSE_SNAPSHOTS)
    gdn_problem pc = *p;
    const float *q = (const float *)q_in, *k = (const float *)k_in, *v = (const float *)v_in;
    const float *g = (const float *)g_in, *beta = (const float *)beta_in, *gy = (const float *)gy_in;
    if (p->dtype != GDN_DTYPE_F32) {
        const bool reuse = flags & GDN_BWD_REUSE_SNAPSHOTS;
        rc = widen_inputs(p, pl, ws, reuse ? nullptr : q_in, reuse ? nullptr : k_in,
                          reuse ? nullptr : v_in, reuse ? nullptr : g_in, reuse ? nullptr : beta_in,
                          gy_in, (hipStream_t)stream, pc, q, k, v, g, beta, &gy);
        if (rc != GDN_OK) return rc;
    }
    p = &pc;

    float *snap = (float *)((char *)ws + pl.off_snap);
    const bool kda = p->gate == GDN_GATE_KDA;

    for (int s0 = 0; s0 < p->n_seqs; s0 += gdn::kMaxSeqsPerLaunch) {
        const int cnt = std::min(gdn::kMaxSeqsPerLaunch, p->n_seqs - s0);
        if (!(flags & GDN_BWD_REUSE_SNAPSHOTS)) {
            gdn::FwdArgs f;
            std::memset(&f, 0, sizeof(f));
            f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.state0 = state0;
            f.snap = snap;
            f.sq = p->q; f.sk = p->k; f.sv = p->v; f.sg = p->g; f.sb = p->beta; f.sy = p->y;
            f.s_base = s0;
            f.T = p->T; f.H_k = p->H_k; f.H_v = p->H_v; f.C = pl.C; f.n_ck_max = pl.n_ck_max;
            f.scale = p->scale;
            f.dtype = p->dtype;
            fill_lens(p, s0, cnt, f.lens);
            rc = device_status(gdn::launch_fwd(f, (int)SK, (int)SV, kda, cnt, (hipStream_t)stream));
            if (rc != GDN_OK) return rc;
        }
        gdn::BwdArgs b;
        std::memset(&b, 0, sizeof(b));
        b.q = q; b.k = k; b.v = v; b.g = g; b.beta = beta; b.gy = gy; b.dstate_out = dstate_out;
        b.snap = snap;
        b.segbuf = (float *)((char *)ws + pl.off_seg);
        b.ebuf_seg = (float *)((char *)ws + pl.off_e);
        if (pl.parts) {
            b.dq = (float *)((char *)ws + pl.off_pq);
            b.dk = (float *)((char *)ws + pl.off_pk);
            b.dqk_head = p->H_v;
        } else {
            b.dq = dq;
            b.dk = dk;
            b.dqk_head = p->H_k;
        }
        b.dv = dv; b.dg = dg; b.dbeta = dbeta; b.dstate = dstate;
        b.sq = p->q; b.sk = p->k; b.sv = p->v; b.sg = p->g; b.sb = p->beta; b.sgy = p->gy;
        b.s_base = s0;
        b.T = p->T; b.H_k = p->H_k; b.H_v = p->H_v; b.C = pl.C; b.n_ck_max = pl.n_ck_max;
        b.scale = p->scale;
        b.dtype = p->dtype;
        fill_lens(p, s0, cnt, b.lens);
        rc = device_status(gdn::launch_bwd(b, (int)SK, (int)SV, kda, cnt, (hipStream_t)stream));
        if (rc != GDN_OK) return rc;
    }
    if (pl.parts) {
        gdn::CombineArgs c;
        c.dq_part = (const float *)((char *)ws + pl.off_pq);
        c.dk_part = (const float *)((char *)ws + pl.off_pk);
        c.dq = dq; c.dk = dk;
        c.n_seqs = p->n_seqs; c.T = p->T; c.H_k = p->H_k; c.H_v = p->H_v; c.S = (int)SK;
        rc = device_status(gdn::launch_combine(c, (hipStream_t)stream));
        if (rc != GDN_OK) return rc;
    }
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_bwd(const gdn_problem *p, const void *q_in, const void *k_in, const void *v_in,
            const void *g_in, const void *beta_in, const float *state0, const void *gy_in,
            const float *dstate_out, float *grad_packed, void *ws, size_t ws_bytes,
            unsigned flags, gdn_stream_t stream) {
    return bwd_impl(p, q_in, k_in, v_in, g_in, beta_in, state0, gy_in, dstate_out, grad_packed,
                    ws, ws_bytes, flags, stream, true);
}

static int conv_check(const gdn_conv_problem *p, const void *in, const void *c, const void *out,
                      bool bwd) {
    if (!p) return GDN_ERR_ARG;
    if (p->n_seqs < 0 || p->T < 0 || p->d_inner <= 0 || p->d_conv <= 0) return GDN_ERR_ARG;
    if (p->d_conv > 8) return GDN_ERR_UNSUPPORTED;
    if (p->sx_seq < 0 || p->sx_tok < 0 || p->y_seq < 0 || p->y_tok < 0) return GDN_ERR_UNSUPPORTED;
    const int64_t n = p->n_seqs, D = p->d_inner, rows_sx = p->T + p->d_conv - 1;
    // a tensor with no elements may be NULL: sx / d_sx has n rows_sx rows, y / dy n T rows
    const bool need_in = n * (bwd ? p->T : rows_sx) > 0, need_out = n * (bwd ? rows_sx : p->T) > 0;
    if ((need_in && !in) || !c || (need_out && !out)) return GDN_ERR_ARG;
    if (!aligned4(in) || !aligned4(c) || !aligned4(out)) return GDN_ERR_UNSUPPORTED;
    const gdn_strides ssx{p->sx_seq, p->sx_tok, 0}, sy{p->y_seq, p->y_tok, 0};
    const Range rsx = span_tok(bwd ? out : in, ssx, n, rows_sx, 1, D);
    const Range ry = span_tok(bwd ? in : out, sy, n, p->T, 1, D);
    const Range rc = span_flat(c, D * p->d_conv);
    const Range &ro = bwd ? rsx : ry, &ri = bwd ? ry : rsx;
    if (overlap(ro, ri) || overlap(ro, rc)) return GDN_ERR_ARG;
    if (!non_self_overlapping(bwd ? ssx : sy, n, bwd ? rows_sx : p->T, 1, D)) return GDN_ERR_ARG;
    return GDN_OK;
}

int gdn_ssm_conv_fwd(const gdn_conv_problem *p, const float *sx, const float *c, float *y,
                     gdn_stream_t stream) {
    const int rc = conv_check(p, sx, c, y, false);
    if (rc != GDN_OK) return rc;
    gdn::ConvArgs a;
    a.in = sx; a.w = c; a.out = y;
    a.in_seq = p->sx_seq; a.in_tok = p->sx_tok; a.out_seq = p->y_seq; a.out_tok = p->y_tok;
    a.n_seqs = p->n_seqs; a.rows_in = p->T + p->d_conv - 1; a.rows_out = p->T;
    a.d_inner = p->d_inner; a.d_conv = p->d_conv;
    return device_status(gdn::launch_conv(a, false, (hipStream_t)stream));
}

int gdn_ssm_conv_bwd(const gdn_conv_problem *p, const float *dy, const float *c, float *d_sx,
                     gdn_stream_t stream) {
    const int rc = conv_check(p, dy, c, d_sx, true);
    if (rc != GDN_OK) return rc;
    gdn::ConvArgs a;
    a.in = dy; a.w = c; a.out = d_sx;
    a.in_seq = p->y_seq; a.in_tok = p->y_tok; a.out_seq = p->sx_seq; a.out_tok = p->sx_tok;
    a.n_seqs = p->n_seqs; a.rows_in = p->T; a.rows_out = p->T + p->d_conv - 1;
    a.d_inner = p->d_inner; a.d_conv = p->d_conv;
    return device_status(gdn::launch_conv(a, true, (hipStream_t)stream));
}

static bool same_view(const void *a, const gdn_strides &sa, const void *b, const gdn_strides &sb) {
    return a == b && sa.seq == sb.seq && sa.tok == sb.tok && sa.head == sb.head;
}

static int l2norm_check(const gdn_l2norm_problem *p, const float *x, const float *dy,
                        const float *out, bool bwd) {
    if (!p) return GDN_ERR_ARG;
    if (p->n_seqs < 0 || p->T < 0 || p->H < 0 || p->W <= 0) return GDN_ERR_ARG;
    if (p->W > 1024) return GDN_ERR_UNSUPPORTED;
    if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return GDN_ERR_ARG;
    const gdn_strides *ss[3] = {&p->x, &p->dy, &p->out};
    for (int i = 0; i < 3; ++i) {
        if (i == 1 && !bwd) continue;
        if (ss[i]->seq < 0 || ss[i]->tok < 0 || ss[i]->head < 0) return GDN_ERR_UNSUPPORTED;
    }
    const int64_t n = p->n_seqs, T = p->T, H = p->H, W = p->W;
    const bool any = n * T * H > 0;
    if (any && (!x || !out || (bwd && !dy))) return GDN_ERR_ARG;
    if (!aligned4(x) || !aligned4(out) || (bwd && !aligned4(dy))) return GDN_ERR_UNSUPPORTED;
    if (!non_self_overlapping(p->out, n, T, H, W)) return GDN_ERR_ARG;
    const Range ro = span_tok(out, p->out, n, T, H, W);
    if (!same_view(out, p->out, x, p->x) && overlap(ro, span_tok(x, p->x, n, T, H, W))) return GDN_ERR_ARG;
    if (bwd && !same_view(out, p->out, dy, p->dy) && overlap(ro, span_tok(dy, p->dy, n, T, H, W)))
        return GDN_ERR_ARG;
    return GDN_OK;
}

static int l2norm_run(const gdn_l2norm_problem *p, const float *x, const float *dy, float *out,
                      bool bwd, gdn_stream_t stream) {
    const int rc = l2norm_check(p, x, dy, out, bwd);
    if (rc != GDN_OK) return rc;
    gdn::NormArgs a;
    a.x = x; a.dy = bwd ? dy : nullptr; a.out = out;
    a.sx = p->x; a.sdy = bwd ? p->dy : gdn_strides{0, 0, 0}; a.so = p->out;
    a.n_seqs = p->n_seqs; a.T = p->T; a.H = p->H; a.W = p->W; a.eps = p->eps;
    return device_status(gdn::launch_l2norm(a, bwd, (hipStream_t)stream));
}

int gdn_l2norm_fwd(const gdn_l2norm_problem *p, const float *x, float *y, gdn_stream_t stream) {
    return l2norm_run(p, x, nullptr, y, false, stream);
}

int gdn_l2norm_bwd(const gdn_l2norm_problem *p, const float *x, const float *dy, float *dx,
                   gdn_stream_t stream) {
    return l2norm_run(p, x, dy, dx, true, stream);
}

// ---- selective scan ----------------------------------------------------------------------

struct SsmPlan {
    size_t off_ck, off_part, off_dd, off_dsq, off_cpart, off_gsw, total;
    int64_t rows, nwin;
    int32_t ckw, nck, hgs, seg_rows;
    bool chunked;   // backward in 32-token chunks on the matrix cores (see ssm_chunk.hip)
    bool rowwise;   // 16 states: backward in two passes, one lane per row (see ssm_scan.hip)
};

static int ssm_validate(const gdn_ssm_problem *p) {
    if (!p) return GDN_ERR_ARG;
    if (p->n_seqs < 0 || p->T < 0 || p->H < 1 || p->P < 1 || p->N < 1 || p->G < 1) return GDN_ERR_ARG;
    if (p->H % p->G != 0) return GDN_ERR_ARG;
    if ((p->a_per_state != 0 && p->a_per_state != 1) || (p->dt_softplus != 0 && p->dt_softplus != 1))
        return GDN_ERR_ARG;
    if (p->N != 16 && p->N != 32 && p->N != 64 && p->N != 128) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)p->P * (p->H / p->G) % 16 != 0) return GDN_ERR_UNSUPPORTED;
    // one workgroup per 16 rows: the grid must fit a launch dimension
    if ((int64_t)p->n_seqs * p->H * p->P / 16 > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    // the chunked backward: at most one workgroup per (sequence, head, 32-token chunk); the
    // row-wise one: one per (128 rows, 8-token window)
    if (gdn::ssm_chunked(p->P, p->N, p->a_per_state, p->H, p->G) &&
        (int64_t)p->n_seqs * p->H * (((int64_t)p->T + 31) / 32) > INT32_MAX)
        return GDN_ERR_UNSUPPORTED;
    if (gdn::ssm_rowwise(p->P, p->H, p->G, p->N) &&
        (int64_t)p->n_seqs * p->H * p->P / 128 * (((int64_t)p->T + 7) / 8) > INT32_MAX)
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

static SsmPlan ssm_plan(const gdn_ssm_problem *p) {
    SsmPlan pl;
    const size_t n = p->n_seqs, T = p->T, H = p->H, P = p->P, N = p->N, G = p->G;
    pl.rows = (int64_t)(n * H * P);
    pl.nwin = (p->T + 7) / 8;
    pl.chunked = gdn::ssm_chunked(p->P, p->N, p->a_per_state, p->H, p->G);
    pl.rowwise = !pl.chunked && gdn::ssm_rowwise(p->P, p->H, p->G, p->N);
    size_t off = 0;
    pl.off_part = pl.off_dd = pl.off_dsq = pl.off_cpart = pl.off_gsw = 0;
    pl.hgs = 1;
    pl.seg_rows = pl.rowwise ? 128 : 16;   // rows per column-sum partial
    if (pl.chunked) {
        // the state before every 32-token chunk; the state gradient after each chunk; dB, dC
        // per head slice, enough slices for about 2048 workgroups
        const int64_t nc = (p->T + 31) / 32, Hg = p->H / p->G;
        const int64_t wgs = std::max<int64_t>(1, (int64_t)n * nc * p->G);
        pl.hgs = (int32_t)std::max<int64_t>(1, std::min<int64_t>({(2048 + wgs - 1) / wgs, Hg, 16}));
        pl.ckw = 4;
        pl.nck = (int32_t)nc;
        pl.off_ck = off;    off += align_up((size_t)pl.rows * nc * N * 4);
        pl.off_dsq = off;   off += align_up(n * H * nc * P * N * 4);
        pl.off_cpart = off; off += align_up((size_t)pl.hgs * 2 * n * T * G * N * 4);
    } else {
        pl.ckw = 1;
        pl.nck = (int32_t)pl.nwin + (pl.rowwise ? 1 : 0);   // row-wise: one spare slot per row
        pl.off_ck = off;   off += align_up((size_t)pl.rows * pl.nck * N * 4);
        pl.off_part = off; off += align_up((size_t)pl.rows / pl.seg_rows * T * 2 * N * 4);
        pl.off_dd = off;   off += align_up(n * T * H * P * 4);
        if (pl.rowwise) {  // the state gradient entering every window
            pl.off_gsw = off; off += align_up((size_t)pl.rows * pl.nwin * N * 4);
        }
    }
    pl.total = off;
    return pl;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t gdn_ssm_workspace_size(const gdn_ssm_problem *p) {
    if (ssm_validate(p) != GDN_OK) return 0;
    return ssm_plan(p).total;
}

size_t gdn_ssm_grad_packed_floats(const gdn_ssm_problem *p, size_t offsets[5]) {
    if (ssm_validate(p) != GDN_OK) return 0;
    const size_t n = p->n_seqs, T = p->T, H = p->H, P = p->P, N = p->N, G = p->G;
    const size_t sizes[5] = {n * H * P * N, n * T * H * P, n * T * H, n * T * G * N, n * T * G * N};
    size_t off = 0;
    for (int i = 0; i < 5; ++i) {
        if (offsets) offsets[i] = off;
        off += sizes[i];
    }
    return off;
}

// Pointer and overlap checks shared by both directions: ins[] are read, outs[] written.
static int ssm_check_ptrs(const gdn_ssm_problem *p, const float *s0, const float *x, const float *dt,
                          const float *A, const float *B, const float *C, const Range *extra_in,
                          int n_extra_in, const Range *outs, int n_outs) {
    const int64_t n = p->n_seqs, T = p->T, H = p->H, P = p->P, N = p->N, G = p->G;
    const bool any_state = n > 0, any_tok = n * T > 0;
    if ((any_state && !s0) || !A || (any_tok && (!x || !dt || !B || !C))) return GDN_ERR_ARG;
    if (!aligned16(s0) || !aligned16(A) || !aligned16(B) || !aligned16(C)) return GDN_ERR_UNSUPPORTED;
    if (!aligned4(x) || !aligned4(dt)) return GDN_ERR_UNSUPPORTED;
    const Range in[] = {span_flat(s0, n * H * P * N), span_flat(x, n * T * H * P), span_flat(dt, n * T * H),
                        span_flat(A, p->a_per_state ? H * N : H), span_flat(B, n * T * G * N),
                        span_flat(C, n * T * G * N)};
    for (int o = 0; o < n_outs; ++o) {
        for (auto &i : in)
            if (overlap(outs[o], i)) return GDN_ERR_ARG;
        for (int e = 0; e < n_extra_in; ++e)
            if (overlap(outs[o], extra_in[e])) return GDN_ERR_ARG;
        for (int q = o + 1; q < n_outs; ++q)
            if (overlap(outs[o], outs[q])) return GDN_ERR_ARG;
    }
    return GDN_OK;
}

static gdn::SsmArgs ssm_args(const gdn_ssm_problem *p, const SsmPlan &pl, void *ws, const float *s0,
                             const float *x, const float *dt, const float *A, const float *B,
                             const float *C) {
    gdn::SsmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.s0 = s0; a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C;
    char *w = (char *)ws;
    a.ck = (float *)(w + pl.off_ck);
    a.part = (float *)(w + pl.off_part);
    a.ddrow = (float *)(w + pl.off_dd);
    a.dsq = (float *)(w + pl.off_dsq);
    a.cpart = (float *)(w + pl.off_cpart);
    a.gsw = (float *)(w + pl.off_gsw);
    a.ckw = pl.ckw; a.nck = pl.nck; a.hgs = pl.hgs; a.seg_rows = pl.seg_rows;
    a.n_seqs = p->n_seqs; a.T = p->T; a.H = p->H; a.P = p->P; a.N = p->N; a.G = p->G;
    a.aps = p->a_per_state; a.softplus = p->dt_softplus;
    return a;
}

int gdn_ssm_fwd(const gdn_ssm_problem *p, const float *s0, const float *x, const float *dt,
                const float *A, const float *B, const float *C, float *y, float *s_out,
                void *ws, size_t ws_bytes, gdn_stream_t stream) {
    int rc = ssm_validate(p);
    if (rc != GDN_OK) return rc;
    const SsmPlan pl = ssm_plan(p);
    const int64_t n = p->n_seqs, T = p->T, H = p->H, P = p->P, N = p->N;
    if ((n * T > 0 && !y) || (n > 0 && !s_out) || (pl.total > 0 && !ws)) return GDN_ERR_ARG;
    if (!aligned4(y) || !aligned16(s_out) || !aligned16(ws)) return GDN_ERR_UNSUPPORTED;
    if (ws_bytes < pl.total) return GDN_ERR_WORKSPACE;
    const Range outs[] = {span_flat(y, n * T * H * P), span_flat(s_out, n * H * P * N), span_bytes(ws, pl.total)};
    rc = ssm_check_ptrs(p, s0, x, dt, A, B, C, nullptr, 0, outs, 3);
    if (rc != GDN_OK) return rc;
    gdn::SsmArgs a = ssm_args(p, pl, ws, s0, x, dt, A, B, C);
    a.y = y; a.s_out = s_out;
    if (pl.chunked) return device_status(gdn::launch_ssm_chunk_fwd(a, (hipStream_t)stream));
    if (pl.rowwise) return device_status(gdn::launch_ssm_rowwise_fwd(a, (hipStream_t)stream));
    return device_status(gdn::launch_ssm(a, false, (hipStream_t)stream));
}

int gdn_ssm_bwd(const gdn_ssm_problem *p, const float *s0, const float *x, const float *dt,
                const float *A, const float *B, const float *C, const float *gy,
                const float *gs_final, float *grad_packed, void *ws, size_t ws_bytes,
                unsigned flags, gdn_stream_t stream) {
    int rc = ssm_validate(p);
    if (rc != GDN_OK) return rc;
    if (flags & ~GDN_BWD_REUSE_SNAPSHOTS) return GDN_ERR_ARG;
    const SsmPlan pl = ssm_plan(p);
    const int64_t n = p->n_seqs, T = p->T, H = p->H, P = p->P, N = p->N;
    size_t off[5];
    const size_t total = gdn_ssm_grad_packed_floats(p, off);
    if ((n * T > 0 && !gy) || (total > 0 && !grad_packed) || (pl.total > 0 && !ws)) return GDN_ERR_ARG;
    if (!aligned4(gy) || !aligned16(gs_final) || !aligned16(grad_packed) || !aligned16(ws))
        return GDN_ERR_UNSUPPORTED;
    if (ws_bytes < pl.total) return GDN_ERR_WORKSPACE;
    const Range extra[] = {span_flat(gy, n * T * H * P), span_flat(gs_final, n * H * P * N)};
    const Range outs[] = {span_flat(grad_packed, (int64_t)total), span_bytes(ws, pl.total)};
    rc = ssm_check_ptrs(p, s0, x, dt, A, B, C, extra, 2, outs, 2);
    if (rc != GDN_OK) return rc;
    gdn::SsmArgs a = ssm_args(p, pl, ws, s0, x, dt, A, B, C);
    a.gy = gy; a.gs = gs_final;
    a.ds0 = grad_packed + off[0]; a.dx = grad_packed + off[1]; a.ddt = grad_packed + off[2];
    a.dB = grad_packed + off[3]; a.dC = grad_packed + off[4];
    hipError_t e = hipSuccess;
    if (!(flags & GDN_BWD_REUSE_SNAPSHOTS))     // window states first (no y, s_out)
        e = pl.chunked ? gdn::launch_ssm_chunk_fwd(a, (hipStream_t)stream)
            : pl.rowwise ? gdn::launch_ssm_rowwise_fwd(a, (hipStream_t)stream)
                         : gdn::launch_ssm(a, false, (hipStream_t)stream);
    if (pl.chunked) {
        if (e == hipSuccess) e = gdn::launch_ssm_chunk_bwd(a, (hipStream_t)stream);
    } else if (pl.rowwise) {
        if (e == hipSuccess) e = gdn::launch_ssm_rowwise_bwd(a, (hipStream_t)stream);
    } else {
        if (e == hipSuccess) e = gdn::launch_ssm(a, true, (hipStream_t)stream);
        if (e == hipSuccess) e = gdn::launch_ssm_combine(a, (hipStream_t)stream);
    }
    return device_status(e);
}

int gdn_bwd_noalloc(const gdn_problem *p, const void *q, const void *k, const void *v,
                    const void *g, const void *beta, const float *state0, const void *gy,
                    const float *dstate_out, float *grad_packed, gdn_stream_t stream) {
    const int rc = validate(p);
    if (rc != GDN_OK) return rc;
    const size_t need = make_plan(p).total;
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void *ws = nullptr;
    const int rs = scratch_address((hipStream_t)stream, &ws);
    if (rs != GDN_OK) return rs;
    // one stream: no second stream or events are created on this path
    return bwd_impl(p, q, k, v, g, beta, state0, gy, dstate_out, grad_packed, ws,
                    GDN_NOALLOC_SCRATCH_BYTES, 0u, stream, false);
}

}  // extern "C"
