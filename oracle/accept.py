"""Greedy acceptance oracle (test infrastructure only).

Given the dense model's logits for the gamma+1 verification rows and the
gamma draft tokens, find the longest prefix of draft tokens that equal the
dense model's own greedy predictions, then take one extra "bonus" token from
the dense model (Sparse-to-Dense pt explainer, "Metodologia", decoding
procedure; the accepted block is appended to the context).

Readings: greedy only (the pages describe no sampling rule); the argmax takes
the lowest index among equal maxima; comparisons follow IEEE rules (so -0 and
+0 are equal); NaN is outside the contract and rejected.
"""
from __future__ import annotations

import numpy as np


def argmax_lowest(row) -> int:
    """Lowest index v with row[v] equal to the row maximum."""
    row = np.asarray(row, np.float64)
    if not np.all(np.isfinite(row)):
        raise ValueError("logits must be finite")
    best = 0
    for j in range(1, row.shape[0]):
        if row[j] > row[best]:
            best = j
    return best


def accept(logits, draft, gamma=None, fast: bool = True):
    """Returns (target_tok [B, n_max], accept_len [B], next_tok [B]) int32.

    logits ``[B, n_max, V]``; draft ``[B, n_max-1]``; gamma ``[B]`` (default
    n_max-1).  For i <= gamma_b: t[b, i] = lowest-index argmax of row i;
    n_b = max{n <= gamma_b : draft[b, j] == t[b, j] for all j < n};
    next_b = t[b, n_b].  Entries t[b, i] for i > gamma_b are -1.

    ``fast`` uses numpy.argmax (first occurrence of the maximum, the same rule)
    instead of the explicit scan.
    """
    logits = np.asarray(logits)
    B, n_max, V = logits.shape
    draft = np.asarray(draft)
    gam = np.full(B, n_max - 1, np.int64) if gamma is None else np.asarray(gamma, np.int64)
    t = np.full((B, n_max), -1, np.int32)
    n_acc = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        g = int(gam[b])
        if not 0 <= g <= n_max - 1:
            raise ValueError("gamma out of range")
        for i in range(g + 1):
            row = np.asarray(logits[b, i], np.float64)
            if fast:
                if not np.all(np.isfinite(row)):
                    raise ValueError("logits must be finite")
                t[b, i] = int(np.argmax(row))
            else:
                t[b, i] = argmax_lowest(row)
        n = 0
        while n < g and int(draft[b, n]) == int(t[b, n]):
            n += 1
        n_acc[b] = n
        nxt[b] = t[b, n]
    return t, n_acc, nxt
