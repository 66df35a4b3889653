"""Comparator of GPU results against the oracle.

Per output region and per (sequence, head) slice: max|x - r| / max|r| <= tol (2e-4 for the
fp32 path).  A slice whose oracle values are all zero (padding, empty sequences) must be
exactly zero.  An empty comparison fails.  An elementwise |x - r| / (|r| + 1e-3 max|r|) is
reported as a diagnostic only.
"""
from __future__ import annotations

import numpy as np

TOL = 2e-4
# slicing of each region: (head axis, index of the sequence axis is always 0)
HEAD_AXIS = {"y": 2, "dv": 2, "dq": 2, "dk": 2, "dg": 2, "dbeta": 2,
             "state_out": 1, "dstate": 1}


def slice_errors(name, x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (name, x.shape, r.shape)
    ax = HEAD_AXIS[name]
    worst, worst_at, n = 0.0, None, 0
    diag = 0.0
    for s in range(r.shape[0]):
        for h in range(r.shape[ax]):
            xs = np.take(x[s], h, axis=ax - 1)
            rs = np.take(r[s], h, axis=ax - 1)
            n += 1
            m = float(np.max(np.abs(rs))) if rs.size else 0.0
            if rs.size == 0:
                continue
            if not np.all(np.isfinite(xs)):
                return float("inf"), (s, h, "non-finite"), n, float("inf")
            if m == 0.0:
                if np.any(xs != 0):
                    return float("inf"), (s, h, "nonzero where oracle is zero"), n, float("inf")
                continue
            e = float(np.max(np.abs(xs - rs))) / m
            d = float(np.max(np.abs(xs - rs) / (np.abs(rs) + 1e-3 * m)))
            diag = max(diag, d)
            if e > worst:
                worst, worst_at = e, (s, h)
    return worst, worst_at, n, diag


def check(results: dict, ref: dict, names=None, tol=TOL):
    """Asserts every named region is within tol; returns {name: worst error}."""
    names = names or list(ref)
    report = {}
    assert names, "empty comparison"
    for name in names:
        worst, at, n, diag = slice_errors(name, results[name], ref[name])
        assert n > 0, f"{name}: empty comparison"
        report[name] = worst
        assert worst <= tol, f"{name}: max relative error {worst:.3e} at {at} > {tol:g} (diag {diag:.2e})"
    return report


def slice_rel(x, r, axes=(0,), group=None):
    """Worst relative error over slices: every index combination of `axes` (and, with `group`,
    groups of that many entries along the last axis) is one slice, compared as
    max|x - r| / max|r|; a slice whose reference is all zero must be exactly zero in x."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if r.size == 0:
        return 0.0
    if group:
        assert r.shape[-1] % group == 0, (r.shape, group)
        x = x.reshape(*x.shape[:-1], -1, group)
        r = r.reshape(*r.shape[:-1], -1, group)
        axes = tuple(axes) + (r.ndim - 2,)
    rest = tuple(a for a in range(r.ndim) if a not in axes)
    xs = np.moveaxis(x, axes, range(len(axes))).reshape(*[r.shape[a] for a in axes], -1)
    rs = np.moveaxis(r, axes, range(len(axes))).reshape(*[r.shape[a] for a in axes], -1)
    del rest
    if not np.all(np.isfinite(xs)):
        return float("inf")
    m = np.max(np.abs(rs), axis=-1)
    d = np.max(np.abs(xs - rs), axis=-1)
    if np.any((m == 0) & (d != 0)):
        return float("inf")
    return float(np.max(np.where(m > 0, d / np.where(m > 0, m, 1.0), 0.0)))
