"""Sparse-to-Dense prefill KV selection and the sparse draft attention that
uses it (float64; test infrastructure only).

Sparse-to-Dense pt explainer, "Metodologia", "Seleção de Cache KV": the
sparse (draft) mode keeps, per layer and attention head, the top-K visual KV
entries, chosen once during prefill by the mean attention that the text
tokens pay to each visual token; the text KV is kept.  Readings taken where
the page is silent:

* Granularity is one selection per (sequence b, KV head g): the KV cache is
  shared by the G query heads of a group, so the mean runs over those heads
  and over the text tokens.
* A text token's attention is its ordinary causal prefill softmax over every
  earlier position (visual and text alike) and itself; keys after it get 0.
* "Visual" positions are the positions below kv_len[b] that are not in the
  text list.  Ties rank by lower index; the kept list is ascending.
* Decoding then attends to the kept list plus every position written after
  the prefill (``tail_start[b] <= j < kv_len[b]``), under the usual causal
  mask.  The same call with per-head anchor lists and a sliding window of
  the last W positions gives the text-anchored window variants.
"""
from __future__ import annotations

import numpy as np

from .attention import _attend, _check, _kv_rows


def std_prefill_scores(q_text, k, kv_len, text_idx, text_len, num_kv_heads: int, scale: float,
                       page_table=None, page_size: int = 0):
    """Mean text-to-key attention per (b, KV head) ("Seleção de Cache KV").

    q_text is ``[B, t_max, Hq, d]``: row t holds the prefill queries of the
    text token at position ``p_t = text_idx[b, t]`` (t < text_len[b]).  With
    ``A[h, t, j] = softmax_j'(scale * <q_text[b, t, h], k_j'>)`` over
    ``j' <= p_t`` (0 for j > p_t),
        ``score[g, j] = 1/(G*T) * sum_{h in group g} sum_{t<T} A[h, t, j]``
    for every j < kv_len[b].  T = 0 gives all zeros.  Returns a list (per b)
    of ``[Hkv, kv_len[b]]`` float64 arrays.
    """
    B, t_max, Hq, d, G = _check(q_text, num_kv_heads)
    res = []
    for b in range(B):
        L, T = int(kv_len[b]), int(text_len[b])
        pos = np.asarray(text_idx[b, :T], np.int64)
        if T and (pos.min() < 0 or pos.max() >= L):
            raise ValueError("text position outside [0, kv_len)")
        kr = np.asarray(_kv_rows(k, b, L, page_table, page_size), np.float64)   # [Hkv, L, d]
        sc = np.zeros((num_kv_heads, L), np.float64)
        for g in range(num_kv_heads):
            if T == 0:
                continue
            for t in range(T):
                p = int(pos[t])
                keys = kr[g, :p + 1]                                   # [p+1, d]
                qh = np.asarray(q_text[b, t, g * G:(g + 1) * G], np.float64)   # [G, d]
                s = scale * (keys @ qh.T)                              # [p+1, G], one column per head
                e = np.exp(s - s.max(axis=0))
                sc[g, :p + 1] += (e / e.sum(axis=0)).sum(axis=1)
            sc[g] /= G * T
        res.append(sc)
    return res


def std_prefill_select(q_text, k, kv_len, text_idx, text_len, num_kv_heads: int, top_k: int,
                       scale: float, page_table=None, page_size: int = 0):
    """Top-K visual positions per (b, KV head) by the mean text attention.

    The visual positions are ``{j < kv_len[b]} minus the text list``; they are
    ranked by (score descending, index ascending) and the first
    ``min(top_k, #visual)`` are returned in ascending order, -1 after them.
    Returns (sel int32 ``[B, Hkv, top_k]``, the scores of
    ``std_prefill_scores``).
    """
    B = q_text.shape[0]
    scores = std_prefill_scores(q_text, k, kv_len, text_idx, text_len, num_kv_heads, scale,
                                page_table, page_size)
    sel = np.full((B, num_kv_heads, top_k), -1, np.int32)
    for b in range(B):
        L, T = int(kv_len[b]), int(text_len[b])
        text = set(int(x) for x in text_idx[b, :T])
        visual = [j for j in range(L) if j not in text]
        for g in range(num_kv_heads):
            s = scores[b][g]
            order = sorted(visual, key=lambda j: (-s[j], j))
            keep = sorted(order[:min(top_k, len(visual))])
            sel[b, g, :len(keep)] = keep
    return sel, scores


def std_keep_list(sel, text_idx, text_len):
    """The positions the sparse draft keeps: the selected visual positions
    and every text position, as one ascending list per (b, KV head).

    Returns (keep int32 ``[B, Hkv, top_k + t_max]`` padded with -1,
    keep_len int32 ``[B, Hkv]``).
    """
    B, Hkv, K = sel.shape
    t_max = text_idx.shape[1]
    keep = np.full((B, Hkv, K + t_max), -1, np.int32)
    keep_len = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        text = [int(x) for x in text_idx[b, :int(text_len[b])]]
        for g in range(Hkv):
            vis = [int(x) for x in sel[b, g] if x >= 0]
            merged = sorted(vis + text)
            keep[b, g, :len(merged)] = merged
            keep_len[b, g] = len(merged)
    return keep, keep_len


def sparse_attention(q, k, v, kv_len, q_len, list_idx, list_len, tail_start, num_kv_heads: int,
                     scale: float, page_table=None, page_size: int = 0, window: int = 0):
    """Draft attention over a persistent per-head position list plus a dense
    tail of recent positions.

    The tail of sequence b starts at ``t0 = tail_start[b]``, or, without
    tail_start, covers the last ``window`` positions (``t0 = kv_len[b] -
    min(window, kv_len[b])``; window 0: no tail).  For (b, g) the attended set
    is the union of the list entries below t0,
    ``list_idx[b, g, :list_len[b, g]]`` (used as given), and the tail
    ``t0 <= j < kv_len[b]``: entries inside the tail count once, as tail
    positions.  Query row i < q_len[b] sits at position
    ``P = kv_len[b] - q_len[b] + i`` and sees the members at positions <= P.
    Returns (O ``[B, n_max, Hq, d]``, LSE ``[B, n_max, Hq]``) in float64.
    """
    B, n_max, Hq, d, G = _check(q, num_kv_heads)
    out = np.zeros((B, n_max, Hq, d), np.float64)
    lse = np.full((B, n_max, Hq), -np.inf, np.float64)
    for b in range(B):
        L, n = int(kv_len[b]), int(q_len[b])
        if tail_start is not None:
            t0 = int(tail_start[b])
        else:
            t0 = L - min(int(window), L)
        kr_all = _kv_rows(k, b, L, page_table, page_size)
        vr_all = _kv_rows(v, b, L, page_table, page_size)
        for g in range(num_kv_heads):
            lst = np.asarray(list_idx[b, g, :int(list_len[b, g])], np.int64)
            members = np.concatenate([lst[lst < t0], np.arange(t0, L, dtype=np.int64)])
            if members.size and (members.min() < 0 or members.max() >= L):
                raise ValueError("attended position outside [0, kv_len)")
            kr, vr = kr_all[g][members], vr_all[g][members]
            heads = range(g * G, (g + 1) * G)
            qr = np.stack([q[b, i, h] for i in range(n) for h in heads]) if n else np.zeros((0, d))
            pos_q = np.repeat(L - n + np.arange(n), G)
            visible = members[None, :] <= pos_q[:, None]
            o, l = _attend(qr, kr, vr, visible, scale)
            r = 0
            for i in range(n):
                for h in heads:
                    out[b, i, h] = o[r]
                    lse[b, i, h] = l[r]
                    r += 1
    return out, lse
