"""Pins of the fp64 oracle: checks against facts that the pages and the mathematics fix,
not against the oracle itself.  Each ``pin_*`` returns (ok, detail) so the same battery
serves the ordinary tests (all must pass) and the planted-mutation tests (each planted
mistake must fail at least one).

Sources of each fact:
  * finite differences: the backward is the gradient of the forward (the pages check
    GATED_DELTA_NET_BACK by finite differences of the forward with a weighted objective
    over the output and the final state);
  * Euler identities: the forward is linear in (state0, v) jointly and y is linear in q;
  * closed forms: one token from a zero state; beta = 0 (pure decay); g = 0, beta = 1 and
    unit keys (the delta rule stores v exactly under key k);
  * scalar gate = per-key-channel gate with equal columns, dg summed (workload statement);
  * grouped heads = explicit repetition of q/k, dq/dk summed over the repeated heads
    (value head h reads key head h mod H_k);
  * rows of the state evolve independently, so the problem splits into single-row problems;
  * checkpoint interval does not change any bit.
"""
from __future__ import annotations

import math

import numpy as np

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dstate")
INPUTS = ("q", "k", "v", "g", "beta", "state0")


def rand_problem(seed, n_seqs=2, T=7, H_k=2, H_v=4, S_k=4, S_v=4, kda=True, C=3, lens=None,
                 g_lo=-0.6, unit_keys=True):
    rng = np.random.default_rng(seed)
    shape = dict(n_seqs=n_seqs, T=T, H_k=H_k, H_v=H_v, S_k=S_k, S_v=S_v, kda=kda, C=C,
                 scale=1.0 / math.sqrt(S_k), seq_lens=list(lens) if lens else None)
    G = S_k if kda else 1
    q = rng.standard_normal((n_seqs, T, H_k, S_k))
    k = rng.standard_normal((n_seqs, T, H_k, S_k))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(
        q=q, k=k,
        v=rng.standard_normal((n_seqs, T, H_v, S_v)),
        g=rng.uniform(g_lo, 0.0, (n_seqs, T, H_v, G)),
        beta=rng.uniform(0.05, 0.95, (n_seqs, T, H_v)),
        state0=0.3 * rng.standard_normal((n_seqs, H_v, S_v, S_k)),
        gy=rng.standard_normal((n_seqs, T, H_v, S_v)),
        dstate_out=rng.standard_normal((n_seqs, H_v, S_v, S_k)),
    )
    if lens:
        for s, L in enumerate(lens):
            for name in ("q", "k", "v", "g", "beta", "gy"):
                x[name][s, L:] = 0.0
    return shape, x


def objective(orc, shape, x):
    y, so = orc.fwd(shape, *(x[n] for n in INPUTS))
    return float(np.sum(x["gy"] * y) + np.sum(x["dstate_out"] * so))


def _rel(a, b):
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def pin_finite_differences(orc, shape, x, h=1e-6, tol=1e-7):
    """Central differences of L = <gy, y> + <dstate_out, state_out> against all six grads."""
    an = orc.bwd(shape, *(x[n] for n in INPUTS), x["gy"], x["dstate_out"])
    worst = 0.0
    for name, gname in zip(INPUTS, GRADS):
        base = x[name]
        fd = np.zeros_like(base)
        flat = base.reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + h
            lp = objective(orc, shape, x)
            flat[idx] = old - h
            lm = objective(orc, shape, x)
            flat[idx] = old
            fd.reshape(-1)[idx] = (lp - lm) / (2 * h)
        a = an[gname].reshape(fd.shape)
        err = _rel(a, fd)
        worst = max(worst, err)
        if not (err <= tol):
            return False, f"{gname}: normwise FD error {err:.3e} > {tol:g}"
    return True, f"worst normwise FD error {worst:.2e}"


def pin_euler(orc, shape, x, tol=1e-11):
    """<dq, q> = <gy, y>;  <dstate, state0> + <dv, v> = L  (homogeneity)."""
    y, so = orc.fwd(shape, *(x[n] for n in INPUTS))
    an = orc.bwd(shape, *(x[n] for n in INPUTS), x["gy"], x["dstate_out"])
    Ly = float(np.sum(x["gy"] * y))
    L = Ly + float(np.sum(x["dstate_out"] * so))
    e1 = abs(float(np.sum(an["dq"] * x["q"])) - Ly) / max(abs(Ly), 1e-300)
    e2 = abs(float(np.sum(an["dstate"] * x["state0"]) + np.sum(an["dv"] * x["v"])) - L) / max(abs(L), 1e-300)
    ok = e1 <= tol and e2 <= tol
    return ok, f"q-homogeneity {e1:.2e}, (state0,v)-homogeneity {e2:.2e}"


def pin_closed_forms(orc, seed=11, tol=1e-12):
    rng = np.random.default_rng(seed)
    msgs = []
    ok = True
    # (a) one token from a zero state, per-key-channel gate
    S, Hk, Hv = 5, 1, 1
    shape = dict(n_seqs=1, T=1, H_k=Hk, H_v=Hv, S_k=S, S_v=S, kda=True, C=1, scale=0.37,
                 seq_lens=None)
    q = rng.standard_normal((1, 1, 1, S)); k = rng.standard_normal((1, 1, 1, S))
    v = rng.standard_normal((1, 1, 1, S)); g = rng.uniform(-1, 0, (1, 1, 1, S))
    beta = np.array([[[0.7]]]); s0 = np.zeros((1, 1, S, S)); gy = rng.standard_normal((1, 1, 1, S))
    y, so = orc.fwd(shape, q, k, v, g, beta, s0)
    d = orc.bwd(shape, q, k, v, g, beta, s0, gy, None)
    sc, b = 0.37, 0.7
    qv, kv, vv, gv, gyv = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], g[0, 0, 0], gy[0, 0, 0]
    a = np.exp(gv)
    exp = dict(
        y=sc * b * vv * (kv @ qv),
        state_out=b * np.outer(vv, kv),
        dq=sc * b * (vv @ gyv) * kv,
        dk=sc * b * (gyv @ vv) * qv,
        dv=sc * b * (qv @ kv) * gyv,
        dbeta=sc * (qv @ kv) * (gyv @ vv),
        dg=np.zeros(S),
        dstate=(sc * np.outer(gyv, qv) - b * sc * (qv @ kv) * np.outer(gyv, kv)) * a[None, :],
    )
    got = dict(y=y[0, 0, 0], state_out=so[0, 0], dq=d["dq"][0, 0, 0], dk=d["dk"][0, 0, 0],
               dv=d["dv"][0, 0, 0], dbeta=d["dbeta"][0, 0, 0], dg=d["dg"][0, 0, 0],
               dstate=d["dstate"][0, 0])
    for n in exp:
        e = np.max(np.abs(got[n] - exp[n])) / max(np.max(np.abs(exp[n])), 1.0)
        if not e <= tol:
            ok = False
            msgs.append(f"one-token {n} err {e:.2e}")

    # (b) beta = 0: pure per-column decay, M_t = state0 .* exp(cumsum g)
    T, S = 6, 4
    shape = dict(n_seqs=1, T=T, H_k=1, H_v=1, S_k=S, S_v=S, kda=True, C=2, scale=0.5,
                 seq_lens=None)
    q = rng.standard_normal((1, T, 1, S)); k = rng.standard_normal((1, T, 1, S))
    v = rng.standard_normal((1, T, 1, S)); g = rng.uniform(-0.8, 0, (1, T, 1, S))
    beta = np.zeros((1, T, 1)); s0 = rng.standard_normal((1, 1, S, S))
    gy = rng.standard_normal((1, T, 1, S)); dso = rng.standard_normal((1, 1, S, S))
    y, so = orc.fwd(shape, q, k, v, g, beta, s0)
    d = orc.bwd(shape, q, k, v, g, beta, s0, gy, dso)
    Gc = np.cumsum(g[0, :, 0, :], axis=0)          # [T, S]
    M0 = s0[0, 0]
    Ms = [M0 * np.exp(Gc[t])[None, :] for t in range(T)]
    y_exp = np.stack([0.5 * Ms[t] @ q[0, t, 0] for t in range(T)])
    dq_exp = np.stack([0.5 * Ms[t].T @ gy[0, t, 0] for t in range(T)])
    dst_exp = dso[0, 0] * np.exp(Gc[-1])[None, :] + sum(
        0.5 * np.outer(gy[0, t, 0], q[0, t, 0]) * np.exp(Gc[t])[None, :] for t in range(T))
    # dL/dg[tau, i] = sum_{t >= tau} sum_j 0.5 gy_t,j M_t[j,i] q_t,i + sum_j dso[j,i] M_T[j,i]
    per_t = np.stack([np.sum(0.5 * gy[0, t, 0][:, None] * Ms[t] * q[0, t, 0][None, :], axis=0)
                      for t in range(T)])
    fin = np.sum(dso[0, 0] * Ms[-1], axis=0)
    dg_exp = np.cumsum(per_t[::-1], axis=0)[::-1] + fin[None, :]
    checks = dict(y=(y[0, :, 0], y_exp), state_out=(so[0, 0], Ms[-1]),
                  dq=(d["dq"][0, :, 0], dq_exp), dstate=(d["dstate"][0, 0], dst_exp),
                  dg=(d["dg"][0, :, 0], dg_exp),
                  dv=(d["dv"], np.zeros_like(d["dv"])), dk=(d["dk"], np.zeros_like(d["dk"])))
    for n, (a_, b_) in checks.items():
        e = np.max(np.abs(a_ - b_)) / max(np.max(np.abs(b_)), 1.0)
        if not e <= tol:
            ok = False
            msgs.append(f"beta=0 {n} err {e:.2e}")

    # (c) g = 0, beta = 1, unit keys: the state stores v under k, so q = k reads v back
    T, S = 5, 6
    shape = dict(n_seqs=1, T=T, H_k=1, H_v=1, S_k=S, S_v=S, kda=False, C=0, scale=0.8,
                 seq_lens=None)
    k = rng.standard_normal((1, T, 1, S)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, S)); g = np.zeros((1, T, 1, 1)); beta = np.ones((1, T, 1))
    s0 = rng.standard_normal((1, 1, S, S))
    y, so = orc.fwd(shape, k, k, v, g, beta, s0)
    e = np.max(np.abs(y[0, :, 0] - 0.8 * v[0, :, 0]))
    if not e <= 1e-12:
        ok = False
        msgs.append(f"memorisation err {e:.2e}")
    return ok, "; ".join(msgs) or "closed forms hold"


def pin_scalar_equals_kda(orc, seed=21, tol=1e-13):
    shape, x = rand_problem(seed, kda=False, lens=[7, 4])
    shape_k = dict(shape, kda=True)
    xk = dict(x, g=np.repeat(x["g"], shape["S_k"], axis=-1))
    y, so = orc.fwd(shape, *(x[n] for n in INPUTS))
    yk, sok = orc.fwd(shape_k, *(xk[n] for n in INPUTS))
    d = orc.bwd(shape, *(x[n] for n in INPUTS), x["gy"], x["dstate_out"])
    dk_ = orc.bwd(shape_k, *(xk[n] for n in INPUTS), xk["gy"], xk["dstate_out"])
    errs = {"y": _rel(yk, y), "state_out": _rel(sok, so)}
    for n in ("dq", "dk", "dv", "dbeta", "dstate"):
        errs[n] = _rel(dk_[n], d[n])
    errs["dg"] = _rel(dk_["dg"].sum(axis=-1, keepdims=True), d["dg"])
    bad = {n: e for n, e in errs.items() if not e <= tol}
    return not bad, f"max {max(errs.values()):.2e}" + (f" bad {bad}" if bad else "")


def pin_gqa_equals_repeat(orc, seed=31, tol=1e-13):
    shape, x = rand_problem(seed, H_k=2, H_v=6, lens=[7, 6])
    Hk, Hv = shape["H_k"], shape["H_v"]
    rep = [h % Hk for h in range(Hv)]
    shape_r = dict(shape, H_k=Hv)
    xr = dict(x, q=x["q"][:, :, rep], k=x["k"][:, :, rep])
    y, so = orc.fwd(shape, *(x[n] for n in INPUTS))
    yr, sor = orc.fwd(shape_r, *(xr[n] for n in INPUTS))
    d = orc.bwd(shape, *(x[n] for n in INPUTS), x["gy"], x["dstate_out"])
    dr = orc.bwd(shape_r, *(xr[n] for n in INPUTS), xr["gy"], xr["dstate_out"])
    errs = {"y": _rel(yr, y), "state_out": _rel(sor, so)}
    for n in ("dv", "dg", "dbeta", "dstate"):
        errs[n] = _rel(dr[n], d[n])
    for n in ("dq", "dk"):
        summed = np.zeros_like(d[n])
        for h in range(Hv):
            summed[:, :, h % Hk] += dr[n][:, :, h]
        errs[n] = _rel(summed, d[n])
    bad = {n: e for n, e in errs.items() if not e <= tol}
    return not bad, f"max {max(errs.values()):.2e}" + (f" bad {bad}" if bad else "")


def pin_row_additivity(orc, seed=41, tol=1e-12):
    """Rows of M are independent: split S_v rows into S_v single-row problems."""
    shape, x = rand_problem(seed, H_k=1, H_v=2, S_k=5, S_v=3, lens=[7, 5])
    full_y, full_so = orc.fwd(shape, *(x[n] for n in INPUTS))
    full = orc.bwd(shape, *(x[n] for n in INPUTS), x["gy"], x["dstate_out"])
    acc = {n: np.zeros_like(full[n]) for n in ("dq", "dk", "dg", "dbeta")}
    errs = {}
    for j in range(shape["S_v"]):
        sj = dict(shape, S_v=1)
        xj = dict(x, v=x["v"][..., j:j + 1], gy=x["gy"][..., j:j + 1],
                  state0=x["state0"][:, :, j:j + 1, :], dstate_out=x["dstate_out"][:, :, j:j + 1, :])
        yj, soj = orc.fwd(sj, *(xj[n] for n in INPUTS))
        dj = orc.bwd(sj, *(xj[n] for n in INPUTS), xj["gy"], xj["dstate_out"])
        errs[f"y{j}"] = _rel(yj[..., 0], full_y[..., j])
        errs[f"so{j}"] = _rel(soj[:, :, 0], full_so[:, :, j])
        errs[f"dv{j}"] = _rel(dj["dv"][..., 0], full["dv"][..., j])
        errs[f"dstate{j}"] = _rel(dj["dstate"][:, :, 0], full["dstate"][:, :, j])
        for n in acc:
            acc[n] += dj[n]
    for n in acc:
        errs[n] = _rel(acc[n], full[n])
    bad = {n: e for n, e in errs.items() if not e <= tol}
    return not bad, f"max {max(errs.values()):.2e}" + (f" bad {bad}" if bad else "")


def pin_checkpoint_invariance(orc, seed=51):
    shape, x = rand_problem(seed, T=11, lens=[11, 8], C=1)
    ref = None
    for C in (1, 2, 3, 4, 5, 11, 0):
        d = orc.bwd(dict(shape, C=C), *(x[n] for n in INPUTS), x["gy"], x["dstate_out"])
        if ref is None:
            ref = d
            continue
        for n in GRADS:
            if not np.array_equal(d[n], ref[n]):
                return False, f"C={C} changes {n}"
    return True, "bit-identical over C"


def standard_fd_cases():
    """Tiny problems for the finite-difference pin: per-key-channel gate with grouped heads
    and ragged lengths; scalar gate; a non-square state."""
    return [
        rand_problem(101, n_seqs=2, T=7, H_k=2, H_v=4, S_k=4, S_v=4, kda=True, C=3, lens=[7, 5]),
        rand_problem(102, n_seqs=2, T=9, H_k=1, H_v=2, S_k=6, S_v=6, kda=False, C=2, lens=[9, 4]),
        rand_problem(103, n_seqs=1, T=5, H_k=1, H_v=3, S_k=5, S_v=3, kda=True, C=2),
    ]


def battery(orc, fd=True):
    """All pins; returns {name: (ok, detail)}."""
    out = {}
    if fd:
        for i, (shape, x) in enumerate(standard_fd_cases()):
            out[f"fd{i}"] = pin_finite_differences(orc, shape, x)
    for i, (shape, x) in enumerate([
            rand_problem(201, T=9, S_k=8, S_v=8, lens=[9, 6]),
            rand_problem(202, kda=False, T=9, H_k=1, H_v=3, S_k=6, S_v=6)]):
        out[f"euler{i}"] = pin_euler(orc, shape, x)
    out["closed_forms"] = pin_closed_forms(orc)
    out["scalar_eq_kda"] = pin_scalar_equals_kda(orc)
    out["gqa_eq_repeat"] = pin_gqa_equals_repeat(orc)
    out["row_additivity"] = pin_row_additivity(orc)
    out["checkpoint_invariance"] = pin_checkpoint_invariance(orc)
    return out
