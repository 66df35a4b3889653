"""Pins of the L2-normalisation oracle (``oracle/l2norm.py``) against facts other than itself:
torch's own ``normalize`` and its autograd (CPU, fp64, eps = 0), closed forms, invariants of a
normalisation (unit length, scale invariance, a gradient orthogonal to x) and central
differences with eps > 0.  Three planted mistakes (eps outside the root, the n^3 term dropped,
its sign flipped) must each fail a pin."""
import numpy as np
import pytest

from oracle import l2norm as L


def _rows(seed, shape=(3, 5, 2, 16)):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape), rng.standard_normal(shape)


def test_forward_matches_torch_normalize():
    torch = pytest.importorskip("torch")
    x, _ = _rows(1)
    ref = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy()
    np.testing.assert_allclose(L.l2norm_fwd(x, 0.0), ref, rtol=1e-14, atol=1e-15)


def pin_autograd(bwd):
    """eps = 0: the backward equals torch autograd of ``normalize`` (fp64, CPU)."""
    import torch
    x, dy = _rows(2)
    xt = torch.from_numpy(x).requires_grad_(True)
    torch.nn.functional.normalize(xt, dim=-1).backward(torch.from_numpy(dy))
    return np.allclose(bwd(x, dy, 0.0), xt.grad.numpy(), rtol=1e-12, atol=1e-13)


def pin_closed_forms(fwd):
    """x = c e_j maps to c e_j / sqrt(c^2 + eps); a zero row with eps > 0 maps to zero."""
    ok = True
    for c, eps in ((3.0, 0.0), (0.5, 1e-2), (-2.0, 0.25)):
        x = np.zeros((1, 8)); x[0, 5] = c
        ref = np.zeros((1, 8)); ref[0, 5] = c / np.sqrt(c * c + eps)
        ok &= np.allclose(fwd(x, eps), ref, rtol=1e-15, atol=0)
    ok &= not np.any(fwd(np.zeros((2, 8)), 1e-6))
    return ok


def test_invariants():
    x, dy = _rows(3)
    y = L.l2norm_fwd(x, 0.0)
    np.testing.assert_allclose(np.sum(y * y, axis=-1), 1.0, rtol=1e-14)          # unit length
    np.testing.assert_allclose(L.l2norm_fwd(7.5 * x, 0.0), y, rtol=1e-14)        # scale invariance
    dx = L.l2norm_bwd(x, dy, 0.0)
    np.testing.assert_allclose(np.sum(x * dx, axis=-1), 0.0, atol=1e-13)         # dx orthogonal to x
    eps = 0.3                                                                   # |y|^2 = s / (s + eps)
    s = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(L.l2norm_fwd(x, eps) ** 2, axis=-1), s / (s + eps), rtol=1e-14)


def pin_fd(fwd, bwd, eps=0.2, h=1e-6):
    """Central differences of L = sum w .* y on every entry of a few rows, eps > 0."""
    x, w = _rows(4, shape=(2, 3, 6))
    g = bwd(x, w, eps)
    for idx in np.ndindex(*x.shape):
        p, m = x.copy(), x.copy()
        p[idx] += h
        m[idx] -= h
        fd = (np.sum(fwd(p, eps) * w) - np.sum(fwd(m, eps) * w)) / (2 * h)
        if abs(fd - g[idx]) > 1e-8 * (1 + abs(fd)):
            return False
    return True


def test_pins_hold():
    pytest.importorskip("torch")
    assert pin_closed_forms(L.l2norm_fwd)
    assert pin_autograd(L.l2norm_bwd)
    assert pin_fd(L.l2norm_fwd, L.l2norm_bwd)


def test_planted_mistakes_are_caught():
    pytest.importorskip("torch")

    def eps_outside_root(x, eps):            # x / (sqrt(sum x^2) + eps)
        return x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)

    def eps_outside_root_bwd(x, dy, eps):    # its own exact derivative: only the definition differs
        r = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        xdy = np.sum(x * dy, axis=-1, keepdims=True)
        return dy / (r + eps) - x * xdy / (r * (r + eps) ** 2)

    def no_cubic(x, dy, eps):                # the projection term dropped
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
        return dy / n

    def flipped(x, dy, eps):                 # the projection term with the wrong sign
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
        return dy / n + x * np.sum(x * dy, axis=-1, keepdims=True) / n ** 3

    assert not pin_closed_forms(eps_outside_root)
    assert pin_fd(eps_outside_root, eps_outside_root_bwd)   # consistent with itself, yet caught above
    for bad in (no_cubic, flipped):
        assert not (pin_autograd(bad) and pin_fd(L.l2norm_fwd, bad)), bad.__name__
