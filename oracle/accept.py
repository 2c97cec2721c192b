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


def commit(kv_len, draft, accept_len, next_tok, gamma=None, tokens=None, tok_len=None,
           text_idx=None, text_len=None):
    """Bookkeeping after acceptance, as plain integer updates (copies in,
    copies out).

    Sparse-to-Dense pt explainer, "Metodologia", decoding procedure: the
    accepted tokens and the bonus token join the context for the next round.
    Reading: during verification sequence b's cache held kv_len[b] positions,
    the last gamma_b + 1 of them the verified rows (the last committed token
    at C = kv_len[b] - gamma_b - 1, then the drafts).  With n = accept_len[b]
    the rows C..C+n stay valid and the rest is rolled back:
        kv_len'[b]  = C + n + 1
        last_tok[b] = next_tok[b]          (its K/V is written next round)
        tokens[b]  += draft[b, :n] + [next_tok[b]]      (n + 1 tokens)
        text_idx[b] += positions C .. C+n               (n + 1 positions)
    Appends stop at the row capacity; the lengths saturate there.
    Returns (kv_len', last_tok, tokens', tok_len', text_idx', text_len').
    """
    kv_len = np.array(kv_len, np.int32)
    B = kv_len.shape[0]
    draft = np.asarray(draft)
    n_max = draft.shape[1] + 1
    gam = np.full(B, n_max - 1, np.int64) if gamma is None else np.asarray(gamma, np.int64)
    last = np.array(next_tok, np.int32).copy()
    tokens = None if tokens is None else np.array(tokens, np.int32)
    tok_len = None if tok_len is None else np.array(tok_len, np.int32)
    text_idx = None if text_idx is None else np.array(text_idx, np.int32)
    text_len = None if text_len is None else np.array(text_len, np.int32)
    for b in range(B):
        n = int(accept_len[b])
        C = int(kv_len[b]) - int(gam[b]) - 1
        new_toks = [int(x) for x in draft[b, :n]] + [int(next_tok[b])]
        if tokens is not None:
            for x in new_toks:
                if tok_len[b] < tokens.shape[1]:
                    tokens[b, tok_len[b]] = x
                    tok_len[b] += 1
        if text_idx is not None:
            for p in range(C, C + n + 1):
                if text_len[b] < text_idx.shape[1]:
                    text_idx[b, text_len[b]] = p
                    text_len[b] += 1
        kv_len[b] = C + n + 1
    return kv_len, last, tokens, tok_len, text_idx, text_len
