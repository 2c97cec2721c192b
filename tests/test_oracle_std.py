"""Pins of the Sparse-to-Dense prefill-selection oracle and of the sparse
draft attention over per-head lists: closed forms (zero queries give uniform
causal attention; a dominant key takes all the weight), a library softmax for
the one-token one-head case, the row-sum invariant, exact selections with
ties, and reductions of the sparse attention to the text-anchored and dense
attentions."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W


def _kv(rng, B, Hkv, L, d, scale=0.5):
    return (rng.standard_normal((B, Hkv, L, d)) * scale,
            rng.standard_normal((B, Hkv, L, d)) * scale)


def test_zero_queries_give_uniform_causal_attention():
    """q = 0 makes every visible logit equal, so text token t spreads weight
    1/(p_t+1) over positions 0..p_t: score_j = 1/T * sum_t [j <= p_t]/(p_t+1)."""
    rng = np.random.default_rng(0)
    B, Hq, Hkv, d, L = 2, 4, 2, 8, 30
    k, _ = _kv(rng, B, Hkv, L, d)
    text_idx = np.array([[3, 9, 17, 29, 0], [0, 5, 6, 0, 0]], np.int32)
    text_len = np.array([4, 3], np.int32)
    q = np.zeros((B, 5, Hq, d))
    kv_len = np.array([30, 12], np.int32)
    sc = oracle.std_prefill_scores(q, k, kv_len, text_idx, text_len, Hkv, 0.3)
    for b in range(B):
        T = text_len[b]
        for g in range(Hkv):
            for j in range(kv_len[b]):
                want = sum(1.0 / (p + 1) for p in text_idx[b, :T] if j <= p) / T
                assert sc[b][g, j] == pytest.approx(want, rel=1e-14, abs=1e-16)


def test_one_token_one_head_is_a_library_softmax():
    rng = np.random.default_rng(1)
    d, L, p = 16, 40, 27
    k, _ = _kv(rng, 1, 1, L, d)
    q = rng.standard_normal((1, 1, 1, d))
    scale = 0.25
    sc = oracle.std_prefill_scores(q, k, np.array([L], np.int32), np.array([[p]], np.int32),
                                   np.array([1], np.int32), 1, scale)[0][0]
    want = np.zeros(L)
    want[:p + 1] = softmax(scale * (k[0, 0, :p + 1] @ q[0, 0, 0]))
    np.testing.assert_allclose(sc, want, rtol=1e-13, atol=1e-16)


def test_mean_runs_over_the_heads_of_the_group():
    """Two KV heads of two query heads each (heads 0, 1 -> KV head 0; 2, 3 ->
    KV head 1).  All queries are 0 (uniform over 0..p) except head 1, which
    points at one key of KV head 0 with a logit gap of ~1e3 (all its weight
    there): KV head 0 scores 1/2 * (1/(p+1) + [j == j*]), KV head 1 stays
    uniform."""
    rng = np.random.default_rng(2)
    d, L, p, js = 8, 20, 14, 6
    k, _ = _kv(rng, 1, 2, L, d, 0.01)
    k[0, 0, js] = 0.0
    k[0, 0, js, 0] = 10.0
    q = np.zeros((1, 1, 4, d))
    q[0, 0, 1, 0] = 100.0
    sc = oracle.std_prefill_scores(q, k, np.array([L], np.int32), np.array([[p]], np.int32),
                                   np.array([1], np.int32), 2, 1.0)[0]
    for j in range(L):
        uni = 1.0 / (p + 1) if j <= p else 0.0
        assert sc[0, j] == pytest.approx(0.5 * (uni + (1.0 if j == js else 0.0)), abs=1e-12)
        assert sc[1, j] == pytest.approx(uni, abs=1e-15)


@pytest.mark.parametrize("seed", range(3))
def test_scores_sum_to_one_and_vanish_after_the_last_text_token(seed):
    c = W.std_small(seed, 2, 4, 2, 32, (70, 45), W.F32, n_text=(9, 5))
    sc = oracle.std_prefill_scores(c.q_text.values, c.k.values, c.kv_len, c.text_idx, c.text_len,
                                   c.num_kv_heads, c.scale)
    for b in range(c.batch):
        last = c.text_idx[b, c.text_len[b] - 1]
        for g in range(c.num_kv_heads):
            assert sc[b][g].sum() == pytest.approx(1.0, abs=1e-13)
            assert np.all(sc[b][g][last + 1:] == 0.0)
            assert np.all(sc[b][g][:last + 1] > 0.0)


def test_selection_with_ties_is_exact():
    """q = 0: scores tie within each run of positions between text tokens.
    Text at 3, 7, 11 (L = 12): the visual runs are {0,1,2} > {4,5,6} > {8,9,10}
    by score, and ties go to the lower index."""
    rng = np.random.default_rng(3)
    k, _ = _kv(rng, 1, 1, 12, 4)
    q = np.zeros((1, 3, 1, 4))
    ti = np.array([[3, 7, 11]], np.int32)
    tl = np.array([3], np.int32)
    kv_len = np.array([12], np.int32)
    for K, want in [(1, [0]), (3, [0, 1, 2]), (4, [0, 1, 2, 4]), (7, [0, 1, 2, 4, 5, 6, 8]),
                    (9, [0, 1, 2, 4, 5, 6, 8, 9, 10]), (11, [0, 1, 2, 4, 5, 6, 8, 9, 10, -1, -1])]:
        sel, _ = oracle.std_prefill_select(q, k, kv_len, ti, tl, 1, K, 0.5)
        assert sel[0, 0].tolist() == want


@pytest.mark.parametrize("seed", range(4))
def test_selection_matches_rank_counting(seed):
    """Brute force on the scores: visual j is kept iff fewer than K visual
    positions beat it, where j' beats j if its score is higher or equal with a
    lower index."""
    c = W.std_small(seed, 2, 4, 2, 16, (40, 33), W.F32, n_text=(6, 4))
    for K in (1, 5, 17, 40):
        sel, sc = oracle.std_prefill_select(c.q_text.values, c.k.values, c.kv_len, c.text_idx,
                                            c.text_len, c.num_kv_heads, K, c.scale)
        for b in range(c.batch):
            text = set(c.text_idx[b, :c.text_len[b]].tolist())
            vis = [j for j in range(c.kv_len[b]) if j not in text]
            for g in range(c.num_kv_heads):
                s = sc[b][g]
                kept = [j for j in vis
                        if sum(1 for i in vis if s[i] > s[j] or (s[i] == s[j] and i < j)) < K]
                got = [x for x in sel[b, g].tolist() if x >= 0]
                assert got == kept
                assert all(x == -1 for x in sel[b, g, len(kept):])


def test_keep_list_is_the_sorted_union():
    sel = np.array([[[2, 9, 15, -1], [0, 1, -1, -1]]], np.int32)
    ti = np.array([[4, 10, 20, 0]], np.int32)
    tl = np.array([3], np.int32)
    keep, n = oracle.std_keep_list(sel, ti, tl)
    assert n.tolist() == [[6, 5]]
    assert keep[0, 0].tolist() == [2, 4, 9, 10, 15, 20, -1, -1]
    assert keep[0, 1].tolist() == [0, 1, 4, 10, 20, -1, -1, -1]


def test_no_text_gives_zero_scores_and_the_first_positions():
    rng = np.random.default_rng(5)
    k, _ = _kv(rng, 1, 2, 9, 4)
    q = rng.standard_normal((1, 2, 2, 4))
    sel, sc = oracle.std_prefill_select(q, k, np.array([9], np.int32),
                                        np.zeros((1, 2), np.int32), np.array([0], np.int32),
                                        2, 4, 0.5)
    assert np.all(sc[0] == 0.0)
    assert sel[0].tolist() == [[0, 1, 2, 3], [0, 1, 2, 3]]


def test_paged_layout_gives_the_same_scores():
    """The contiguous rows scattered into a shuffled page pool give the same
    scores bit for bit."""
    c = W.std_small(6, 2, 4, 2, 16, (50, 37), W.F32, n_text=(7, 3))
    ps, k = 8, c.k.values
    B, Hkv, Lm, d = k.shape
    npg = (Lm + ps - 1) // ps
    perm = np.random.default_rng(0).permutation(B * npg)
    pool = np.zeros((B * npg, Hkv, ps, d), k.dtype)
    table = perm.reshape(B, npg).astype(np.int32)
    for b in range(B):
        for j in range(Lm):
            pool[table[b, j // ps], :, j % ps] = k[b, :, j]
    a = oracle.std_prefill_scores(c.q_text.values, k, c.kv_len, c.text_idx, c.text_len,
                                  2, c.scale)
    p = oracle.std_prefill_scores(c.q_text.values, pool, c.kv_len, c.text_idx, c.text_len,
                                  2, c.scale, table, ps)
    for x, y in zip(a, p):
        assert np.array_equal(x, y)


def test_sparse_attention_reduces_to_vata_and_to_dense():
    c = W.small_attn(7, 2, 4, 2, 16, 3, (40, 29), W.F32)
    q, k, v = c.q.values, c.k.values, c.v.values
    # the same list for both heads and no tail: text-anchored attention
    lst = np.repeat(c.text_idx[:, None, :], 2, axis=1)
    ln = np.repeat(c.text_len[:, None], 2, axis=1)
    o1, l1 = oracle.sparse_attention(q, k, v, c.kv_len, c.q_len, lst, ln, None, 2, c.scale)
    o2, l2 = oracle.vata_attention(q, k, v, c.kv_len, c.q_len, c.text_idx, c.text_len, 2, c.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # an empty list and the whole sequence as the tail: dense attention
    o1, l1 = oracle.sparse_attention(q, k, v, c.kv_len, c.q_len, np.zeros((2, 2, 1), np.int32),
                                     np.zeros((2, 2), np.int32), np.zeros(2, np.int32), 2, c.scale)
    o2, l2 = oracle.verify_attention(q, k, v, c.kv_len, c.q_len, 2, c.scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-15)


def test_sparse_attention_per_head_lists_and_tail():
    """Each KV head attends to its own list plus the tail: head g alone equals
    text-anchored attention over (list of g) + tail positions."""
    c = W.small_attn(8, 1, 4, 2, 16, 2, (50,), W.F32)
    q, k, v = c.q.values, c.k.values, c.v.values
    lst = np.array([[[1, 5, 9, 30, -1], [0, 2, 3, 4, 39]]], np.int32)
    ln = np.array([[4, 5]], np.int32)
    tail = np.array([44], np.int32)
    o, l = oracle.sparse_attention(q, k, v, c.kv_len, c.q_len, lst, ln, tail, 2, c.scale)
    for g in range(2):
        ti = np.concatenate([lst[0, g, :ln[0, g]], np.arange(44, 50)]).astype(np.int32)[None]
        og, lg = oracle.vata_attention(q[:, :, 2 * g:2 * g + 2], k[:, g:g + 1], v[:, g:g + 1],
                                       c.kv_len, c.q_len, ti, np.array([ti.shape[1]], np.int32),
                                       1, c.scale)
        assert np.array_equal(o[:, :, 2 * g:2 * g + 2], og)
        assert np.array_equal(l[:, :, 2 * g:2 * g + 2], lg)


def test_sliding_window_is_attention_over_the_last_positions():
    """No list, a window of W: text-anchored attention over the last W
    positions (fewer when the sequence is shorter)."""
    c = W.small_attn(9, 2, 4, 2, 16, 3, (40, 7), W.F32)
    q, k, v = c.q.values, c.k.values, c.v.values
    Wn = 12
    o1, l1 = oracle.sparse_attention(q, k, v, c.kv_len, c.q_len, np.zeros((2, 2, 1), np.int32),
                                     np.zeros((2, 2), np.int32), None, 2, c.scale, window=Wn)
    ti = np.full((2, Wn), 0, np.int32)
    tl = np.zeros(2, np.int32)
    for b in range(2):
        x = np.arange(max(0, c.kv_len[b] - Wn), c.kv_len[b])
        ti[b, :len(x)] = x
        tl[b] = len(x)
    o2, l2 = oracle.vata_attention(q, k, v, c.kv_len, c.q_len, ti, tl, 2, c.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_list_entries_inside_the_tail_count_once():
    """Anchors that fall inside the window are the window's own positions:
    the result equals the same call with those anchors removed."""
    c = W.small_attn(10, 1, 4, 2, 16, 2, (50,), W.F32)
    q, k, v = c.q.values, c.k.values, c.v.values
    lst = np.array([[[3, 9, 41, 45, 48], [0, 44, 47, -1, -1]]], np.int32)
    ln = np.array([[5, 3]], np.int32)
    a = oracle.sparse_attention(q, k, v, c.kv_len, c.q_len, lst, ln, None, 2, c.scale, window=10)
    lst2 = np.array([[[3, 9, -1, -1, -1], [0, -1, -1, -1, -1]]], np.int32)
    b = oracle.sparse_attention(q, k, v, c.kv_len, c.q_len, lst2, np.array([[2, 1]], np.int32),
                                np.array([40], np.int32), 2, c.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
