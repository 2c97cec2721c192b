"""Hidden-state-reuse fusion oracle (float64; test infrastructure only).

The draft model receives no raw visual tokens; it concatenates the current
text embedding e_t with the target's reused text hidden state h_{t-1} and
projects the pair with one fully connected layer (Sparrow zh explainer,
technical summary 3.1 "HSR"; Sparrow pt explainer 3.A).

Readings: concatenation order [e ; h] as the pages word it; no bias; the
weight is output-major ``W [D, 2D]`` so that ``Y[r, o] = sum_k X[r, k] W[o, k]``
with ``X[r] = concat(E[r], H[r])``.
"""
from __future__ import annotations

import numpy as np


def hsr_fuse(e, h, w):
    """Y = concat(E, H) @ W^T in float64.  E, H ``[M, D]``, W ``[D, 2D]``."""
    e = np.asarray(e, np.float64)
    h = np.asarray(h, np.float64)
    w = np.asarray(w, np.float64)
    if e.shape != h.shape or w.shape != (e.shape[1], 2 * e.shape[1]):
        raise ValueError("shape mismatch")
    x = np.concatenate([e, h], axis=1)             # [M, 2D]
    return x @ w.T


def hsr_fuse_loops(e, h, w):
    """The same definition written as explicit sums (small inputs only)."""
    e = np.asarray(e, np.float64)
    h = np.asarray(h, np.float64)
    w = np.asarray(w, np.float64)
    M, D = e.shape
    y = np.zeros((M, D), np.float64)
    for r in range(M):
        x = list(e[r]) + list(h[r])
        for o in range(D):
            s = 0.0
            for kk in range(2 * D):
                s += x[kk] * w[o, kk]
            y[r, o] = s
    return y
