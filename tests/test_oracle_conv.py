"""Pins of the convolution oracle (``oracle/ssm_conv.py``) against facts other than itself:
numpy's own convolution, closed forms, the adjoint identity of a linear map, and finite
differences of a weighted objective.  Two planted mistakes (a backward that ignores the
incoming gradient, one that drops the carried-state rows) must each fail a pin."""
import numpy as np
import pytest

from oracle import ssm_conv as C


def _case(seed, n=2, T=9, D=5, K=4):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, T + K - 1, D)), rng.standard_normal((D, K)), rng.standard_normal((n, T, D))


@pytest.mark.parametrize("K", [1, 2, 4, 7])
def test_forward_is_numpy_valid_convolution(K):
    sx, c, _ = _case(1, K=K)
    y = C.conv_fwd(sx, c)
    for s in range(sx.shape[0]):
        for i in range(sx.shape[2]):
            # numpy.convolve flips its second argument: flipping the taps back gives
            # sum_j x[t + j] c[j] over the windows that fit ("valid")
            ref = np.convolve(sx[s, :, i], c[i, ::-1], mode="valid")
            np.testing.assert_allclose(y[s, :, i], ref, rtol=1e-13, atol=1e-13)


def test_closed_forms():
    sx, _, _ = _case(2)
    D, K, T = sx.shape[2], 4, sx.shape[1] - 3
    last = np.zeros((D, K)); last[:, K - 1] = 1.0      # newest tap only: the token itself
    first = np.zeros((D, K)); first[:, 0] = 1.0        # oldest tap only: K - 1 rows back
    np.testing.assert_array_equal(C.conv_fwd(sx, last), sx[:, K - 1:])
    np.testing.assert_array_equal(C.conv_fwd(sx, first), sx[:, :T])
    ones = np.ones((D, K))                             # moving sum = difference of prefix sums
    cs = np.concatenate([np.zeros_like(sx[:, :1]), np.cumsum(sx, axis=1)], axis=1)
    np.testing.assert_allclose(C.conv_fwd(sx, ones), cs[:, K:] - cs[:, :T], atol=1e-12)


def pin_adjoint(bwd, seed=3):
    """<conv(sx), w> = <sx, conv_bwd(w)>: the backward is the transpose of the linear map."""
    sx, c, w = _case(seed)
    lhs = np.sum(C.conv_fwd(sx, c) * w)
    rhs = np.sum(sx * bwd(w, c))
    return abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1)


def pin_fd(bwd, seed=4, h=1e-6):
    """Central differences of L = sum w .* conv(sx) on every input entry, the carried rows
    included (weighted, so a backward that ignores w cannot pass)."""
    sx, c, w = _case(seed, n=1, T=5, D=3, K=3)
    g = bwd(w, c)
    for idx in np.ndindex(*sx.shape):
        p, m = sx.copy(), sx.copy()
        p[idx] += h
        m[idx] -= h
        fd = (np.sum(C.conv_fwd(p, c) * w) - np.sum(C.conv_fwd(m, c) * w)) / (2 * h)
        if abs(fd - g[idx]) > 1e-7 * (1 + abs(fd)):
            return False
    return True


def test_backward_pins():
    assert pin_adjoint(C.conv_bwd)
    assert pin_fd(C.conv_bwd)


def test_planted_mistakes_are_caught():
    def ignore_dy(dy, c):          # scatters the taps alone (the pages' unweighted-test trap)
        return C.conv_bwd(np.ones_like(dy), c)

    def drop_state_rows(dy, c):    # no gradient for the d_conv - 1 carried rows
        g = C.conv_bwd(dy, c)
        g[:, :c.shape[1] - 1] = 0
        return g

    for bad in (ignore_dy, drop_state_rows):
        assert not (pin_adjoint(bad) and pin_fd(bad)), bad.__name__
