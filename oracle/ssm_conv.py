"""Plain fp64 CPU oracle of the short causal depthwise convolution upstream of the gated
delta rule (it produces the mixed q/k/v rows) and of its backward with respect to the input.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may
import this module; the HIP path never imports it and shares no code with it.

Source: page "S1-24: chunked attention -- the kernel-free long-context path", the commit
notes on SSM_CONV_BACK.  The forward is a depthwise causal convolution over a sliding window
of d_conv tokens whose input carries the previous d_conv - 1 tokens (the convolution state)
in front of the new ones; the weights are frozen, so only the input takes a gradient, and
that gradient is the scatter of each output's gradient back over the d_conv inputs that
produced it, the carried-state rows included.

Layouts (one reading of the page's ggml tensors, chosen so that a token's channels are
contiguous, as in the mixed q/k/v rows the recurrence reads):
  sx   [n_seqs][d_conv - 1 + T][d_inner]   carried state rows first, then the T tokens
  c    [d_inner][d_conv]                   per-channel taps
  y    [n_seqs][T][d_inner]                y[s][t][i] = sum_j sx[s][t + j][i] * c[i][j]
  d_sx [n_seqs][d_conv - 1 + T][d_inner]   d_sx[s][t + j][i] += dy[s][t][i] * c[i][j]
"""
from __future__ import annotations

import numpy as np


def conv_fwd(sx, c):
    """y[s][t][i] = sum over taps j = 0 .. d_conv - 1 (in that order) of sx[s][t + j][i] c[i][j]."""
    sx = np.asarray(sx, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    n, TT, D = sx.shape
    K = c.shape[1]
    assert c.shape == (D, K) and TT >= K - 1
    T = TT - (K - 1)
    y = np.zeros((n, T, D))
    for j in range(K):
        y += sx[:, j:j + T, :] * c[:, j]
    return y


def conv_bwd(dy, c):
    """The page's scatter: for every output (s, t, i) and tap j, d_sx[s][t + j][i] receives
    dy[s][t][i] c[i][j]; taps in increasing j."""
    dy = np.asarray(dy, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    n, T, D = dy.shape
    K = c.shape[1]
    assert c.shape == (D, K)
    dsx = np.zeros((n, T + K - 1, D))
    for j in range(K):
        dsx[:, j:j + T, :] += dy * c[:, j]
    return dsx
