"""Attention oracles (float64, plain softmax; test infrastructure only).

Conventions shared by every function here (readings where the pages are
silent):

* q is ``[B, n_max, Hq, d]``; query head h uses KV head ``h // (Hq // Hkv)``
  (consecutive query heads share a KV head).
* Sequence b holds ``kv_len[b]`` KV positions, which already include the
  query rows' own K/V; query row i (< q_len[b]) sits at absolute position
  ``P = kv_len[b] - q_len[b] + i`` and sees key position j iff ``j <= P``
  (bottom-right causal mask).  Rows i >= q_len[b] are padding: O = 0,
  LSE = -inf.
* Softmax scale ``scale`` is passed by the caller (1/sqrt(d) normally).
* LSE is the natural-log log-sum-exp of the scaled scores.
* K/V are either contiguous ``[B, Hkv, L_max, d]`` or a paged pool
  ``[P, Hkv, page_size, d]`` addressed through ``page_table[b, pos // page_size]``.
"""
from __future__ import annotations

import numpy as np


def paged_rows(pool: np.ndarray, page_table: np.ndarray, b: int, length: int,
               page_size: int) -> np.ndarray:
    """Logical ``[Hkv, length, d]`` rows of sequence b, read from a paged pool.

    Position p lives in physical page ``page_table[b, p // page_size]`` at
    slot ``p % page_size``.  (Storage layout only; not part of the method.)
    """
    pos = np.arange(length)
    phys = page_table[b, pos // page_size]
    slot = pos % page_size
    rows = pool[phys, :, slot, :]                  # [length, Hkv, d]
    return np.ascontiguousarray(rows.transpose(1, 0, 2))


def _kv_rows(k, b, length, page_table, page_size):
    if page_size:
        return paged_rows(k, page_table, b, length, page_size)
    return k[b, :, :length, :]


def _attend(q_rows: np.ndarray, keys: np.ndarray, vals: np.ndarray,
            visible: np.ndarray, scale: float):
    """Plain masked softmax attention for a block of query rows.

    q_rows [R, d], keys/vals [N, d], visible [R, N] bool.  Returns O [R, d]
    and LSE [R] with, per row r and A_r = {j : visible[r, j]}:
        s_j = scale * <q_r, k_j>,  m = max_A s_j,  Z = sum_A exp(s_j - m),
        O_r = sum_A exp(s_j - m) / Z * v_j,  LSE_r = m + ln Z.
    A row with an empty A gets O = 0 and LSE = -inf.
    """
    q_rows = np.asarray(q_rows, np.float64)
    keys = np.asarray(keys, np.float64)
    vals = np.asarray(vals, np.float64)
    R = q_rows.shape[0]
    out = np.zeros((R, vals.shape[1]), np.float64)
    lse = np.full(R, -np.inf, np.float64)
    if keys.shape[0] == 0:
        return out, lse
    s = scale * (q_rows @ keys.T)                  # [R, N]
    s = np.where(visible, s, -np.inf)
    for r in range(R):
        if not visible[r].any():
            continue
        m = s[r].max()
        e = np.exp(s[r] - m)                        # exp(-inf) = 0 off the mask
        z = e.sum()
        out[r] = (e / z) @ vals
        lse[r] = m + np.log(z)
    return out, lse


def _check(q, num_kv_heads):
    B, n_max, Hq, d = q.shape
    if Hq % num_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, n_max, Hq, d, Hq // num_kv_heads


def verify_attention(q, k, v, kv_len, q_len, num_kv_heads: int, scale: float,
                     page_table=None, page_size: int = 0, units=None):
    """Dense verification attention over the full KV cache.

    Returns (O [B, n_max, Hq, d], LSE [B, n_max, Hq]) in float64.  ``units``
    optionally restricts the computation to a list of (b, kv_head) pairs; the
    other outputs stay at O = 0, LSE = -inf.
    """
    B, n_max, Hq, d, G = _check(q, num_kv_heads)
    out = np.zeros((B, n_max, Hq, d), np.float64)
    lse = np.full((B, n_max, Hq), -np.inf, np.float64)
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(num_kv_heads)]
    for b, g in todo:
        L, n = int(kv_len[b]), int(q_len[b])
        kr = _kv_rows(k, b, L, page_table, page_size)[g]
        vr = _kv_rows(v, b, L, page_table, page_size)[g]
        heads = range(g * G, (g + 1) * G)
        qr = np.stack([q[b, i, h] for i in range(n) for h in heads]) if n else np.zeros((0, d))
        pos_q = np.repeat(L - n + np.arange(n), G)
        visible = np.arange(L)[None, :] <= pos_q[:, None]
        o, l = _attend(qr, kr, vr, visible, scale)
        r = 0
        for i in range(n):
            for h in heads:
                out[b, i, h] = o[r]
                lse[b, i, h] = l[r]
                r += 1
    return out, lse


def vata_attention(q, k, v, kv_len, q_len, text_idx, text_len, num_kv_heads: int,
                   scale: float, page_table=None, page_size: int = 0, units=None):
    """Text-anchored attention: only the KV rows named by the text-position
    list are read.

    For row i of sequence b the attended set is
    ``A = {t < text_len[b] : text_idx[b, t] <= kv_len[b] - q_len[b] + i}``
    with keys/values ``K[b, g, text_idx[b, t]]``.  The list is used as given
    (a repeated position counts twice).  Empty A gives O = 0, LSE = -inf.
    """
    B, n_max, Hq, d, G = _check(q, num_kv_heads)
    out = np.zeros((B, n_max, Hq, d), np.float64)
    lse = np.full((B, n_max, Hq), -np.inf, np.float64)
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(num_kv_heads)]
    for b, g in todo:
        L, n, T = int(kv_len[b]), int(q_len[b]), int(text_len[b])
        idx = np.asarray(text_idx[b, :T], np.int64)
        if T and (idx.min() < 0 or idx.max() >= L):
            raise ValueError("text position outside [0, kv_len)")
        kr = _kv_rows(k, b, L, page_table, page_size)[g][idx]
        vr = _kv_rows(v, b, L, page_table, page_size)[g][idx]
        heads = range(g * G, (g + 1) * G)
        qr = np.stack([q[b, i, h] for i in range(n) for h in heads]) if n else np.zeros((0, d))
        pos_q = np.repeat(L - n + np.arange(n), G)
        visible = idx[None, :] <= pos_q[:, None]
        o, l = _attend(qr, kr, vr, visible, scale)
        r = 0
        for i in range(n):
            for h in heads:
                out[b, i, h] = o[r]
                lse[b, i, h] = l[r]
                r += 1
    return out, lse


def topk_scores(q, k, kv_len, num_kv_heads: int, page_table=None, page_size: int = 0):
    """Relevance score of every key for the single draft query.

    Per (b, g): qbar = sum of the group's query vectors, score_j = <qbar, k_j>
    for j < kv_len[b].  This is the group-mean pre-softmax attention score up
    to the positive factor scale/G, which does not change the ranking (reading
    of the Sparse-to-Dense "Seleção de Cache KV" mean-score criterion applied
    per decoding step).

    Evaluated in float64 in a fixed order so that any implementation can
    reproduce it bit for bit: qbar accumulates heads in increasing order;
    each score accumulates products over c = 0..d-1 in increasing order, every
    product and every sum rounded to float64 (no fused multiply-add).
    Returns a list (per b) of ``[Hkv, kv_len[b]]`` float64 arrays.
    """
    B, n_max, Hq, d, G = _check(q, num_kv_heads)
    res = []
    for b in range(B):
        L = int(kv_len[b])
        kr = np.asarray(_kv_rows(k, b, L, page_table, page_size), np.float64)  # [Hkv, L, d]
        sc = np.zeros((num_kv_heads, L), np.float64)
        for g in range(num_kv_heads):
            qbar = np.zeros(d, np.float64)
            for h in range(g * G, (g + 1) * G):
                qbar = qbar + np.asarray(q[b, 0, h], np.float64)
            acc = np.zeros(L, np.float64)
            for c in range(d):
                acc = acc + qbar[c] * kr[g, :, c]
            sc[g] = acc
        res.append(sc)
    return res


def topk_select(q, k, kv_len, num_kv_heads: int, top_k: int, page_table=None,
                page_size: int = 0):
    """Indices of the top_k highest-scoring keys per (b, KV head).

    Keys are ranked by (score descending, index ascending); the first
    min(top_k, kv_len[b]) are kept and emitted in ascending index order;
    slots past kv_len[b] hold -1.  Returns int32 ``[B, Hkv, top_k]``.
    """
    B = q.shape[0]
    scores = topk_scores(q, k, kv_len, num_kv_heads, page_table, page_size)
    sel = np.full((B, num_kv_heads, top_k), -1, np.int32)
    for b in range(B):
        L = int(kv_len[b])
        for g in range(num_kv_heads):
            s = scores[b][g]
            order = sorted(range(L), key=lambda j: (-s[j], j))
            keep = sorted(order[:min(top_k, L)])
            sel[b, g, :len(keep)] = keep
    return sel


def topk_attention(q, k, v, kv_len, num_kv_heads: int, top_k: int, scale: float,
                   page_table=None, page_size: int = 0):
    """Top-K sparse draft attention for one query row per sequence.

    q is ``[B, 1, Hq, d]``; the query sits at position kv_len[b]-1, so every
    kept key is visible.  Each head of group g attends only to the keys in
    ``topk_select``'s list for (b, g).  Returns (sel_idx, O [B,1,Hq,d], LSE).
    """
    B, n_max, Hq, d, G = _check(q, num_kv_heads)
    if n_max != 1:
        raise ValueError("top-K draft attention takes one query row")
    sel = topk_select(q, k, kv_len, num_kv_heads, top_k, page_table, page_size)
    out = np.zeros((B, 1, Hq, d), np.float64)
    lse = np.full((B, 1, Hq), -np.inf, np.float64)
    for b in range(B):
        L = int(kv_len[b])
        for g in range(num_kv_heads):
            idx = sel[b, g]
            idx = idx[idx >= 0]
            kr = _kv_rows(k, b, L, page_table, page_size)[g][idx]
            vr = _kv_rows(v, b, L, page_table, page_size)[g][idx]
            qr = np.stack([q[b, 0, h] for h in range(g * G, (g + 1) * G)])
            visible = np.ones((G, len(idx)), bool)
            o, l = _attend(qr, kr, vr, visible, scale)
            out[b, 0, g * G:(g + 1) * G] = o
            lse[b, 0, g * G:(g + 1) * G] = l
    return sel, out, lse
