"""Pins of the top-K oracle: exact integer brute force (selection and
tie-breaking), exactness of the fixed-order float64 score, and reduction of
the K >= L case to dense one-row decode."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W


def _int_case(seed, B=2, Hq=4, Hkv=2, d=6, L=16, dup=True):
    rng = np.random.default_rng(seed)
    q = rng.integers(-3, 4, size=(B, 1, Hq, d)).astype(np.float32)
    k = rng.integers(-3, 4, size=(B, Hkv, L, d)).astype(np.float32)
    if dup:
        for b in range(B):
            for g in range(Hkv):
                src = rng.integers(0, L, size=4)
                dst = rng.integers(0, L, size=4)
                k[b, g, dst] = k[b, g, src]
    v = rng.standard_normal((B, Hkv, L, d)).astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("top_k", [1, 4, 7, 16, 20])
def test_selection_integer_brute_force(seed, top_k):
    """Integer inputs make every score exact, so ties are exact.  Brute force:
    rank by exact score (Python ints), ties to the lower index, keep top_k,
    emit ascending, pad with -1."""
    q, k, v = _int_case(seed)
    B, _, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kv_len = np.full(B, L, np.int32)
    sel = oracle.topk_select(q, k, kv_len, Hkv, top_k)
    for b in range(B):
        for g in range(Hkv):
            qbar = [sum(int(q[b, 0, h, c]) for h in range(g * G, (g + 1) * G)) for c in range(d)]
            sc = [sum(qbar[c] * int(k[b, g, j, c]) for c in range(d)) for j in range(L)]
            best = sorted(range(L), key=lambda j: (-sc[j], j))[:min(top_k, L)]
            want = sorted(best) + [-1] * max(0, top_k - L)
            assert sel[b, g].tolist() == want


def test_ties_straddling_the_boundary_go_to_lower_index():
    # every key has the same score: the lowest indices win
    q = np.ones((1, 1, 2, 4), np.float32)
    k = np.ones((1, 1, 10, 4), np.float32)
    sel = oracle.topk_select(q, k, np.array([10]), 1, 3)
    assert sel[0, 0].tolist() == [0, 1, 2]
    # one key above, then a tie group straddling the cut
    k[0, 0, 7] = 2.0
    sel = oracle.topk_select(q, k, np.array([10]), 1, 3)
    assert sel[0, 0].tolist() == [0, 1, 7]


def test_ragged_lengths_only_rank_valid_keys():
    q, k, v = _int_case(3, B=2, L=16)
    kv_len = np.array([9, 16], np.int32)
    sel = oracle.topk_select(q, k, kv_len, 2, 12)
    assert sel[0, 0, 9:].tolist() == [-1, -1, -1]
    assert sel[0, 0, :9].tolist() == list(range(9))


def test_float64_score_is_exact_for_bf16_inputs():
    """For bf16 data at workload magnitudes the fixed-order float64 score is
    within a few ulp of the exact rational value."""
    c = W.small_attn(21, 1, 7, 1, 128, 1, 200, W.BF16)
    sc = oracle.topk_scores(c.q.values, c.k.values, c.kv_len, 1)[0][0]
    qv = c.q.values.astype(np.float64)
    kv = c.k.values.astype(np.float64)
    for j in range(0, 200, 13):
        qbar = [sum(Fraction(float(qv[0, 0, h, cc])) for h in range(7)) for cc in range(128)]
        exact = sum(qbar[cc] * Fraction(float(kv[0, 0, j, cc])) for cc in range(128))
        assert abs(Fraction(sc[j]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


def test_topk_covering_everything_equals_dense_decode():
    c = W.small_attn(22, 2, 6, 2, 16, 1, (40, 33), W.F32)
    sel, o, lse = oracle.topk_attention(c.q.values, c.k.values, c.v.values, c.kv_len, 2, 64,
                                        c.scale)
    o2, l2 = oracle.verify_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len, 2,
                                     c.scale)
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - l2)) < 1e-13
    assert sel[0, 0, :40].tolist() == list(range(40)) and sel[1, 0, 33:].tolist() == [-1] * 31


def test_topk_attention_only_reads_selected_rows():
    c = W.small_attn(23, 1, 4, 1, 16, 1, 64, W.F32)
    sel, o, lse = oracle.topk_attention(c.q.values, c.k.values, c.v.values, c.kv_len, 1, 8,
                                        c.scale)
    v = c.v.values.copy()
    mask = np.ones(64, bool)
    mask[sel[0, 0]] = False
    v[0, 0, mask] = 1e9
    _, o2, _ = oracle.topk_attention(c.q.values, c.k.values, v, c.kv_len, 1, 8, c.scale)
    assert np.array_equal(o, o2)


def _rounding_case(d: int = 8, L: int = 6, j1: int = 1, j2: int = 4):
    """Queries whose group sum needs 51 bits and two keys whose ranking
    depends on each product being rounded before it is added.

    qbar = (1, 1 + 2^-50, 2^-50 + 2^-58, 0, ...).  Key j1 = (-(1 + 2^-7),
    1 + 2^-7, 0, ...): the product (1 + 2^-50)(1 + 2^-7) = 1 + 2^-7 + 2^-50
    + 2^-57 rounds to 1 + 2^-7 + 2^-50 (2^-57 is below half an ulp of 1), so
    the chain gives exactly 2^-50.  Key j2 = (0, 0, 1, 0, ...) scores
    2^-50 + 2^-58.  A fused multiply-add would keep the 2^-57 and rank j1
    first.  Every other key is zero (score 0)."""
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, 0, :3] = [1.0, 1.0, 2.0 ** -50]
    q[0, 0, 1, :3] = [0.0, 2.0 ** -50, 2.0 ** -58]
    k = np.zeros((1, 1, L, d), np.float32)
    k[0, 0, j1, :2] = [-(1 + 2.0 ** -7), 1 + 2.0 ** -7]
    k[0, 0, j2, 2] = 1.0
    return q, k


def test_score_products_are_rounded_before_the_sum():
    q, k = _rounding_case()
    sc = oracle.topk_scores(q, k, np.array([6]), 1)[0][0]
    assert sc[1] == 2.0 ** -50
    assert sc[4] == 2.0 ** -50 + 2.0 ** -58
    fused = 2.0 ** -50 + 2.0 ** -57          # the same chain with the j1 product unrounded
    assert fused > sc[4] > sc[1]
    assert oracle.topk_select(q, k, np.array([6]), 1, 1)[0, 0].tolist() == [4]
    assert oracle.topk_select(q, k, np.array([6]), 1, 2)[0, 0].tolist() == [1, 4]
