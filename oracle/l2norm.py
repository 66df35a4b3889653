"""Plain fp64 CPU oracle of the per-(token, head) L2 normalisation of q and k that sits between
the short convolution and the gated delta rule, and of its backward.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may
import this module; the HIP path never imports it and shares no code with it.

Source: meTile's "Training kernels and gradients", section "Recurrent delta attention" (the
normalisation of the recurrence's inputs is a separate step, outside the recurrence kernel),
and page "metal: GATED_DELTA_NET_BACK", first review (q and k are row views of the mixed rows
on the fused path).  The pages name the step without a formula; the reading taken is the plain
one: each row x of width W (one token of one head) maps to

    n = sqrt(sum_i x_i^2 + eps),   y = x / n,

and the backward is the Jacobian-transpose product of that map,

    dx = dy / n - x (x . dy) / n^3.
"""
from __future__ import annotations

import numpy as np


def l2norm_fwd(x, eps):
    """y = x / sqrt(sum over the last axis of x^2 + eps), row by row."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    return x / n


def l2norm_bwd(x, dy, eps):
    """dx = dy / n - x (x . dy) / n^3 with n = sqrt(sum x^2 + eps), row by row."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    xdy = np.sum(x * dy, axis=-1, keepdims=True)
    return dy / n - x * xdy / n ** 3
