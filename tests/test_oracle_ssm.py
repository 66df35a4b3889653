"""Pins of the selective-scan oracle (``oracle/ssm_scan.py``) against facts other than itself:
central differences of a weighted objective that includes the final state (both branches,
grouped heads, with and without softplus), the forward written in its materialised form (each
output a sum over earlier tokens with explicit decay products from cumulative sums), closed
forms, linearity, and the group fold against explicit repetition of B and C.  Five planted
mistakes must each fail a pin."""
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
