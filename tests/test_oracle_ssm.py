"""Pins of the selective-scan oracle (``oracle/ssm_scan.py``) against facts other than itself:
central differences of a weighted objective that includes the final state (both branches,
grouped heads, with and without softplus), the forward written in its materialised form (each
output a sum over earlier tokens with explicit decay products from cumulative sums), closed
forms, linearity, the group fold against explicit repetition of B and C, and, with one decay per
head, the backward in the chunked closed form (the gradients of a chunk as dense products of
its Grams, given the state before it and the gradient after it).  Five planted mistakes must
each fail a pin."""
import numpy as np
import pytest

from oracle import ssm_scan as S


def case(seed, n=2, T=5, H=4, P=3, N=4, G=2, per_state=False, positive_dt=False):
    """Inputs of one scan; with positive_dt the raw steps are |N(0, 1)| (a step used without
    softplus must be positive, or the state grows instead of decaying)."""
    rng = np.random.default_rng(seed)
    s0 = rng.standard_normal((n, H, P, N))
    x = rng.standard_normal((n, T, H, P))
    dt = rng.standard_normal((n, T, H))
    if positive_dt:
        dt = np.abs(dt)
    A = -np.exp(rng.standard_normal((H, N) if per_state else (H,)))   # negative: decaying
    B = rng.standard_normal((n, T, G, N))
    C = rng.standard_normal((n, T, G, N))
    return s0, x, dt, A, B, C


CASES = [
    dict(P=1, N=3, H=4, G=2, per_state=True),     # Mamba-1 branch, two heads per group
    dict(P=3, N=4, H=4, G=2, per_state=False),    # Mamba-2 branch, two heads per group
    dict(P=2, N=2, H=3, G=1, per_state=False),    # one group
]


def pin_fd(bwd_fn, kw, softplus_dt=True, seed=11, h=1e-6):
    """Central differences of L = <wy, y> + <ws, s_final> w.r.t. s0, x, dt, B, C."""
    s0, x, dt, A, B, C = case(seed, positive_dt=not softplus_dt, **kw)
    rng = np.random.default_rng(seed + 1)
    y, sT = S.ssm_fwd(s0, x, dt, A, B, C, softplus_dt)
    wy, ws = rng.standard_normal(y.shape), rng.standard_normal(sT.shape)

    def L(s0_, x_, dt_, B_, C_):
        y_, sT_ = S.ssm_fwd(s0_, x_, dt_, A, B_, C_, softplus_dt)
        return np.sum(wy * y_) + np.sum(ws * sT_)

    grads = bwd_fn(s0, x, dt, A, B, C, wy, ws, softplus_dt)
    args = [s0, x, dt, B, C]
    for k, (arr, gr) in enumerate(zip(args, grads)):
        for idx in np.ndindex(*arr.shape):
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[k][idx] += h
            m[k][idx] -= h
            fd = (L(*p) - L(*m)) / (2 * h)
            if abs(fd - gr[idx]) > 1e-6 * (1 + abs(fd)):
                return False
    return True


def _bwd(*a):
    return S.ssm_bwd(*a[:6], a[6], a[7], softplus_dt=a[8])


@pytest.mark.parametrize("kw", CASES)
def test_finite_differences(kw):
    assert pin_fd(_bwd, kw, softplus_dt=True)


def test_finite_differences_without_softplus():
    assert pin_fd(_bwd, CASES[1], softplus_dt=False)


def materialised(s0, x, dt, A, B, C):
    """y[t] = sum_n C_t[n] (exp(A_n D_t) s0[:, n] + sum_{tau <= t} exp(A_n (D_t - D_tau))
    d_tau x_tau B_tau[n]) with D the cumulative sum of the steps."""
    n, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    d = S.softplus(dt)
    D = np.cumsum(d, axis=1)                                  # [n, T, H]
    An = A if A.ndim == 2 else np.repeat(A[:, None], N, axis=1)
    y = np.zeros((n, T, H, P))
    for s in range(n):
        for h in range(H):
            g = h // (H // G)
            for t in range(T):
                acc = np.zeros(P)
                for k in range(N):
                    v = np.exp(An[h, k] * D[s, t, h]) * s0[s, h, :, k]
                    for tau in range(t + 1):
                        v = v + np.exp(An[h, k] * (D[s, t, h] - D[s, tau, h])) * d[s, tau, h] \
                            * x[s, tau, h] * B[s, tau, g, k]
                    acc += C[s, t, g, k] * v
                y[s, t, h] = acc
    return y


@pytest.mark.parametrize("kw", CASES)
def test_forward_equals_materialised_form(kw):
    s0, x, dt, A, B, C = case(21, **kw)
    y, _ = S.ssm_fwd(s0, x, dt, A, B, C)
    np.testing.assert_allclose(y, materialised(s0, x, dt, A, B, C), rtol=1e-11, atol=1e-12)


def test_closed_forms():
    s0, x, dt, A, B, C = case(31, P=2, N=3, H=2, G=1, per_state=True)
    d = S.softplus(dt)
    # no input: pure decay, s_T = exp(A sum_t d_t) s0
    _, sT = S.ssm_fwd(s0, x, dt, A, np.zeros_like(B), C)
    decay = np.exp(A[None, :, None, :] * d.sum(axis=1)[:, :, None, None])
    np.testing.assert_allclose(sT, decay * s0, rtol=1e-13)
    # no decay: s_T = s0 + sum_t d_t x_t B_t^T
    _, sT = S.ssm_fwd(s0, x, dt, np.zeros_like(A), B, C)
    ref = s0 + np.einsum("nth,nthp,ntk->nhpk", d, x, B[:, :, 0])
    np.testing.assert_allclose(sT, ref, rtol=1e-12, atol=1e-12)


def test_linear_in_state_and_input():
    s0, x, dt, A, B, C = case(41, **CASES[1])
    s1, x1, *_ = case(42, **CASES[1])
    al, be = 0.7, -1.3
    y, sT = S.ssm_fwd(al * s0 + be * s1, al * x + be * x1, dt, A, B, C)
    ya, sa = S.ssm_fwd(s0, x, dt, A, B, C)
    yb, sb = S.ssm_fwd(s1, x1, dt, A, B, C)
    np.testing.assert_allclose(y, al * ya + be * yb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sT, al * sa + be * sb, rtol=1e-12, atol=1e-12)


def pin_fold(bwd_fn, seed=51):
    """Grouped B, C equal the same run with B, C repeated per head (G = H), whose dB, dC summed
    over the heads of each group are the grouped gradients."""
    kw = dict(P=2, N=3, H=4, G=2, per_state=False)
    s0, x, dt, A, B, C = case(seed, **kw)
    H, G = 4, 2
    grp = np.arange(H) // (H // G)
    rng = np.random.default_rng(seed + 1)
    gy = rng.standard_normal(x.shape)
    gs = rng.standard_normal(s0.shape)
    ok = True
    y, sT = S.ssm_fwd(s0, x, dt, A, B, C)
    yr, sTr = S.ssm_fwd(s0, x, dt, A, B[:, :, grp], C[:, :, grp])
    ok &= np.allclose(y, yr, rtol=1e-14, atol=0) and np.allclose(sT, sTr, rtol=1e-14, atol=0)
    g1 = bwd_fn(s0, x, dt, A, B, C, gy, gs, True)
    g2 = bwd_fn(s0, x, dt, A, B[:, :, grp], C[:, :, grp], gy, gs, True)
    for a, b in zip(g1[:3], g2[:3]):
        ok &= np.allclose(a, b, rtol=1e-13, atol=1e-14)
    for k in (3, 4):
        folded = np.stack([g2[k][:, :, grp == gg].sum(axis=2) for gg in range(G)], axis=2)
        ok &= np.allclose(g1[k], folded, rtol=1e-13, atol=1e-14)
    return bool(ok)


def test_group_fold():
    assert pin_fold(_bwd)


@pytest.mark.parametrize("mutation", [1, 2, 3, 4, 5])
def test_planted_mistakes_are_caught(mutation):
    S._MUTATION = mutation
    try:
        caught = not (pin_fold(_bwd) and all(pin_fd(_bwd, kw) for kw in CASES))
    finally:
        S._MUTATION = 0
    assert caught, mutation


def chunked_bwd(s0, x, dt, A, B, C, gy, gs, softplus_dt=True, Q=4):
    """The backward with one decay per head in chunks of Q tokens, from the closed form of the
    state inside a chunk, s_t = e^{L_t} s_in + sum_{u <= t} e^{L_t - L_u} d_u x_u B_u^T (L the
    running sum of d A): per chunk the gradient of the state after it (dS, walked backwards over
    the chunks), then every gradient as a product of the chunk's Grams CB = C B^T and
    GX = gy x^T masked by D[t][u] = e^{L_t - L_u} (u <= t)."""
    n, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    d = np.logaddexp(0.0, dt) if softplus_dt else np.array(dt, dtype=np.float64)
    grp = np.arange(H) // (H // G)
    nc = (T + Q - 1) // Q
    _, _, states = S.ssm_fwd(s0, x, dt, A, B, C, softplus_dt, keep_states=True)
    dx, ddt = np.zeros((n, T, H, P)), np.zeros((n, T, H))
    dB, dC = np.zeros((n, T, G, N)), np.zeros((n, T, G, N))
    ds0 = np.zeros((n, H, P, N))
    sig = 1.0 / (1.0 + np.exp(-dt)) if softplus_dt else np.ones_like(dt)

    def chunk(s, h, c):
        t0 = c * Q
        cnt = min(Q, T - t0)
        g = grp[h]
        pad = lambda v, w: np.concatenate([v, np.zeros((Q - cnt, w))]) if cnt < Q else v
        dd = np.concatenate([d[s, t0:t0 + cnt, h], np.zeros(Q - cnt)])
        L = np.cumsum(dd * A[h])
        return (t0, cnt, dd, L, pad(x[s, t0:t0 + cnt, h], P), pad(gy[s, t0:t0 + cnt, h], P),
                pad(B[s, t0:t0 + cnt, g], N), pad(C[s, t0:t0 + cnt, g], N))

    for s in range(n):
        for h in range(H):
            dS = np.zeros((nc, P, N))
            cur = np.zeros((P, N)) if gs is None else np.array(gs[s, h], dtype=np.float64)
            for c in range(nc - 1, -1, -1):
                _, _, _, L, _, gyc, _, Cc = chunk(s, h, c)
                dS[c] = cur
                cur = np.exp(L[-1]) * cur + (gyc * np.exp(L)[:, None]).T @ Cc
            ds0[s, h] = cur
            for c in range(nc):
                t0, cnt, dd, L, xc, gyc, Bc, Cc = chunk(s, h, c)
                s_in, dSQ = states[t0][s, h], dS[c]
                D = np.tril(np.exp(L[:, None] - L[None, :]))
                CB, GX = Cc @ Bc.T, gyc @ xc.T
                w, eL = np.exp(L[-1] - L), np.exp(L)
                Wd = D * GX * dd[None, :]
                GBi, GBe = (D * CB).T @ gyc, (w[:, None] * Bc) @ dSQ.T
                dCi = (eL[:, None] * gyc) @ s_in
                Z = Wd * CB
                row = np.array([Z[t, :t].sum() for t in range(Q)])
                col = np.array([Z[t + 1:, t].sum() for t in range(Q)])
                excl = lambda v: np.concatenate([[0.0], np.cumsum(v)[:-1]])
                R = dd * np.einsum("up,up->u", xc, GBe)
                Y = np.einsum("tn,tn->t", Cc, dCi)
                dl = (np.cumsum(Y[::-1])[::-1] + np.exp(L[-1]) * np.sum(dSQ * s_in)
                      + excl(col - row) + excl(R))
                GB = GBi + GBe
                dx[s, t0:t0 + cnt, h] = (dd[:, None] * GB)[:cnt]
                ddt[s, t0:t0 + cnt, h] = ((A[h] * dl + np.einsum("up,up->u", xc, GB))[:cnt]
                                           * sig[s, t0:t0 + cnt, h])
                dB[s, t0:t0 + cnt, grp[h]] += (Wd.T @ Cc + ((dd * w)[:, None] * xc) @ dSQ)[:cnt]
                dC[s, t0:t0 + cnt, grp[h]] += (Wd @ Bc + dCi)[:cnt]
    return ds0, dx, ddt, dB, dC


@pytest.mark.parametrize("T,softplus_dt,with_gs", [(11, True, True), (8, False, True), (3, True, False)])
def test_backward_equals_chunked_closed_form(T, softplus_dt, with_gs):
    """With one decay per head: ragged and whole chunks, raw steps, no final-state cotangent."""
    s0, x, dt, A, B, C = case(31 + T, T=T, H=4, P=3, N=5, G=2, positive_dt=not softplus_dt)
    rng = np.random.default_rng(T)
    gy = rng.standard_normal(x.shape)
    gs = rng.standard_normal(s0.shape) if with_gs else None
    ref = S.ssm_bwd(s0, x, dt, A, B, C, gy, gs, softplus_dt)
    got = chunked_bwd(s0, x, dt, A, B, C, gy, gs, softplus_dt)
    for r, g in zip(ref, got):
        assert np.allclose(g, r, rtol=1e-10, atol=1e-12)
