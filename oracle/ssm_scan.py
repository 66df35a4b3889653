"""Plain fp64 CPU oracle of the selective state-space scan (Mamba-1 and Mamba-2 branches) and
of its backward, the reverse recurrence.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may
import this module; the HIP path never imports it and shares no code with it.

Source: page "S1-24: chunked attention -- the kernel-free long-context path", the commit notes
on SSM_SCAN_BACK (the reverse recurrence, its packed five-gradient output, the seed at
t = n_t from the state region of the incoming gradient, store-all recomputation) and on the
n_group fold (head h reads group h / (H / G); dB and dC of a group sum its heads).  The scan
itself is the published selective state-space recurrence.  Per sequence, head h, head element
i and state n, with step d_t = softplus(dt[t, h]) (or dt itself when softplus is off):

    a_t[n]     = exp(d_t * A[h, n])          (Mamba-1: one A per state; Mamba-2: A[h] for all n)
    s_t[i, n]  = a_t[n] s_{t-1}[i, n] + d_t x[t, h, i] B[t, g, n]
    y[t, h, i] = sum_n s_t[i, n] C[t, g, n]

returning y and the final state.  The backward keeps every state (store-all) and walks
t = T - 1 .. 0 with gs = dL/ds seeded by the cotangent of the final state:

    gs        += gy[t, h, i] C[t, g, n]
    dC[t, g]  += sum_i gy[t, h, i] s_t[i, :]           (heads of the group, increasing h)
    dx[t, h]   = d_t sum_n gs[:, n] B[t, g, n]
    dB[t, g]  += sum_i gs[i, :] d_t x[t, h, i]
    dd         = sum_{i,n} gs (A a_t s_{t-1} + x B)     (the decay path and the input path)
    ddt[t, h]  = dd * sigmoid(dt[t, h])                  (dd itself without softplus)
    gs         = a_t gs
and d_s0 = gs after token 0.  A takes no gradient.

Layouts (the page's ggml tensors, innermost last): s [n][H][P][N], x [n][T][H][P],
dt [n][T][H], A [H][N] or [H], B and C [n][T][G][N], y [n][T][H][P].

``_MUTATION`` plants one known mistake (tests only): 1 ignores the final-state cotangent,
2 drops the decay path of dd, 3 reads the state one token late in dd, 4 maps heads to groups
by h mod G, 5 forgets the softplus derivative.
"""
from __future__ import annotations

import numpy as np

_MUTATION = 0


def softplus(z):
    """log(1 + exp(z)), evaluated without overflow."""
    return np.logaddexp(0.0, z)


def _setup(x, dt, A, B, softplus_dt, mutation_groups=False):
    n, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert H % G == 0
    grp = (np.arange(H) % G) if mutation_groups else (np.arange(H) // (H // G))
    d = softplus(dt) if softplus_dt else np.array(dt, dtype=np.float64)      # [n, T, H]
    A = np.asarray(A, dtype=np.float64)
    Ah = A[:, None, :] if A.ndim == 2 else A[:, None, None]                   # [H, 1, N|1]
    return grp, d, Ah


def ssm_fwd(s0, x, dt, A, B, C, softplus_dt=True, keep_states=False):
    """(y, s_final[, states]) of the scan; states[t] is the state after t tokens."""
    s0, x, dt, B, C = (np.asarray(v, dtype=np.float64) for v in (s0, x, dt, B, C))
    grp, d, Ah = _setup(x, dt, A, B, softplus_dt)
    n, T, H, P = x.shape
    s = s0.copy()
    states = [s]
    y = np.zeros((n, T, H, P))
    for t in range(T):
        a = np.exp(d[:, t, :, None, None] * Ah[None])                        # [n, H, 1, N|1]
        Bt, Ct = B[:, t][:, grp], C[:, t][:, grp]                            # [n, H, N]
        s = a * s + (d[:, t, :, None] * x[:, t])[..., None] * Bt[:, :, None, :]
        y[:, t] = np.einsum("nhpk,nhk->nhp", s, Ct)
        states.append(s)
    return (y, s, states) if keep_states else (y, s)


def ssm_bwd(s0, x, dt, A, B, C, gy, gs_final=None, softplus_dt=True):
    """(d_s0, dx, ddt, dB, dC) of L = <gy, y> + <gs_final, s_final>."""
    m = _MUTATION
    s0, x, dt, B, C, gy = (np.asarray(v, dtype=np.float64) for v in (s0, x, dt, B, C, gy))
    _, _, states = ssm_fwd(s0, x, dt, A, B, C, softplus_dt, keep_states=True)
    grp, d, Ah = _setup(x, dt, A, B, softplus_dt, mutation_groups=(m == 4))
    n, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    g = np.zeros_like(s0) if (gs_final is None or m == 1) else np.array(gs_final, dtype=np.float64)
    dx = np.zeros_like(x)
    ddt = np.zeros_like(dt)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    sig = 1.0 / (1.0 + np.exp(-dt))
    for t in range(T - 1, -1, -1):
        a = np.exp(d[:, t, :, None, None] * Ah[None])
        Bt, Ct = B[:, t][:, grp], C[:, t][:, grp]
        s_t, s_prev = states[t + 1], states[t]
        g = g + gy[:, t][..., None] * Ct[:, :, None, :]
        dC_h = np.einsum("nhp,nhpk->nhk", gy[:, t], s_t)
        gB = np.einsum("nhpk,nhk->nhp", g, Bt)
        dx[:, t] = d[:, t, :, None] * gB
        dB_h = np.einsum("nhpk,nhp->nhk", g, d[:, t, :, None] * x[:, t])
        s_dec = s_t if m == 3 else s_prev
        dd = np.einsum("nhpk,nhpk->nh", g, np.broadcast_to(Ah[None] * a * s_dec, g.shape))
        if m == 2:
            dd = 0.0 * dd
        dd = dd + np.einsum("nhp,nhp->nh", gB, x[:, t])
        ddt[:, t] = dd * (sig[:, t] if (softplus_dt and m != 5) else 1.0)
        for h in range(H):                       # fold heads into their group, increasing h
            dB[:, t, grp[h]] += dB_h[:, h]
            dC[:, t, grp[h]] += dC_h[:, h]
        g = a * g
    return g, dx, ddt, dB, dC
