"""GPU parity of top-K sparse draft attention: the selected index lists must
match the oracle bit for bit (ties to the lower index), the attention within
tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, kvcache

pytestmark = pytest.mark.gpu


def _run(c, top_k):
    import speculative_decoding_attention_amd as S
    q1 = dev(W.Stored(c.q.dtype, c.q.bits[:, -1:].copy()))
    sel, out, lse = S.spec_topk_attn(kvcache(c), q1, top_k, scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), out, lse


def _ref(c, top_k):
    q1 = c.q.values[:, -1:]
    return oracle.topk_attention(q1, c.k.values, c.v.values, c.kv_len, c.num_kv_heads, top_k,
                                 c.scale, c.page_table, c.page_size)


@pytest.mark.parametrize("cfg", [
    (1, 2, 28, 4, 128, (3000, 1900), W.BF16, 0, 256),
    (2, 3, 8, 2, 128, (700, 5000, 64), W.BF16, 16, 100),
    (3, 2, 4, 1, 64, (999, 300), W.F32, 0, 37),
    (4, 1, 28, 4, 128, (500,), W.BF16, 0, 1),
    (5, 2, 8, 2, 128, (120, 900), W.BF16, 0, 200),      # top_k > L for sequence 0
    (6, 2, 8, 2, 128, (1024, 640), W.BF16, 0, 600),     # K near L: the cut sits in the low tail
    (7, 3, 8, 2, 128, (4096, 33, 2051), W.BF16, 16, 32),  # 16-byte key rows, ragged lengths, paged
], ids=lambda c: f"s{c[0]}")
def test_small_topk(cfg):
    seed, B, Hq, Hkv, d, L, dt, page, K = cfg
    c = W.small_attn(seed, B, Hq, Hkv, d, 1, L, dt, page_size=page)
    sel, out, lse = _run(c, K)
    rs, ro, rl = _ref(c, K)
    assert np.array_equal(sel, rs)
    assert_attention_close(out, lse, ro, rl, np.ones(B, np.int32), dt, "topk small")


def _plant_boundary_ties(c, top_k, rng):
    """Copy the key row that ranks exactly K-th over several other rows (some
    before, some after it), so a tie group straddles the selection cut."""
    q1 = c.q.values[:, -1:]
    scores = oracle.topk_scores(q1, c.k.values, c.kv_len, c.num_kv_heads)
    kb = c.k.bits.copy()
    for b in range(c.batch):
        for g in range(c.num_kv_heads):
            s = scores[b][g]
            order = np.lexsort((np.arange(len(s)), -s))
            kth = order[top_k - 1]
            for dst in rng.choice(len(s), size=6, replace=False):
                kb[b, g, dst] = kb[b, g, kth]
    c.k = W.Stored(c.k.dtype, kb)
    return c


def test_topk_ties_straddling_the_cut():
    rng = np.random.default_rng(5)
    c = W.small_attn(21, 2, 28, 4, 128, 1, (6000, 4000), W.BF16)
    c = _plant_boundary_ties(c, 512, rng)
    sel, out, lse = _run(c, 512)
    rs, ro, rl = _ref(c, 512)
    assert np.array_equal(sel, rs)
    assert_attention_close(out, lse, ro, rl, np.ones(2, np.int32), W.BF16, "topk ties")


def test_topk_large_tie_group_at_the_cut():
    """2000 identical key rows spread over a 3000-key cache with the cut inside
    the group: the boundary holds more equal keys than counting ranks, so
    the candidates are sorted; the lowest indices of the group must win."""
    rng = np.random.default_rng(9)
    c = W.small_attn(23, 1, 8, 2, 128, 1, (3000,), W.BF16)
    kb = c.k.bits.copy()
    for g in range(2):
        rows = rng.choice(3000, size=2000, replace=False)
        kb[0, g, rows] = kb[0, g, rows[0]]
    c.k = W.Stored(W.BF16, kb)
    for top_k in (700, 1500):
        sel, out, lse = _run(c, top_k)
        rs, ro, rl = _ref(c, top_k)
        assert np.array_equal(sel, rs)
        assert_attention_close(out, lse, ro, rl, np.ones(1, np.int32), W.BF16, "topk tie group")


def test_topk_all_equal_scores_uses_exact_fallback():
    """Every key identical: more keys share the boundary bin than the sort
    buffer holds, so the exact radix path must pick the lowest indices."""
    c = W.small_attn(22, 1, 8, 2, 128, 1, (9000,), W.BF16)
    kb = c.k.bits.copy()
    kb[:, :, :] = kb[:, :, :1]
    c.k = W.Stored(W.BF16, kb)
    sel, out, lse = _run(c, 300)
    assert np.array_equal(sel[0, 0], np.arange(300)) and np.array_equal(sel[0, 1], np.arange(300))
    rs, ro, rl = _ref(c, 300)
    assert np.array_equal(sel, rs)
    assert_attention_close(out, lse, ro, rl, np.ones(1, np.int32), W.BF16, "topk all equal")


@pytest.fixture(scope="module")
def c4():
    return W.c4_topk(0)


def test_c4_topk_full(c4):
    sel, out, lse = _run(c4, 2048)
    rs, ro, rl = _ref(c4, 2048)
    assert np.array_equal(sel, rs)
    assert_attention_close(out, lse, ro, rl, np.ones(4, np.int32), W.BF16, "c4 topk")


def test_c4_topk_with_planted_ties(c4):
    rng = np.random.default_rng(9)
    c = W.AttnCase(**{**c4.__dict__})
    c = _plant_boundary_ties(c, 2048, rng)
    sel, out, lse = _run(c, 2048)
    rs, ro, rl = _ref(c, 2048)
    assert np.array_equal(sel, rs)


def test_c2_topk_full():
    c = W.c2_sparrow(0, with_hsr=False)[0]
    sel, out, lse = _run(c, 2048)
    rs, ro, rl = _ref(c, 2048)
    assert np.array_equal(sel, rs)
    assert_attention_close(out, lse, ro, rl, np.ones(1, np.int32), W.BF16, "c2 topk")


def test_topk_everything_equals_dense_decode():
    import speculative_decoding_attention_amd as S
    c = W.small_attn(23, 2, 28, 4, 128, 1, (700, 1100), W.BF16)
    sel, out, lse = _run(c, 4096)
    o2, l2 = S.spec_verify_attn(kvcache(c), dev(W.Stored(W.BF16, c.q.bits[:, -1:].copy())),
                                scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(sel[0, 0, :700], np.arange(700)) and np.all(sel[0, :, 700:] == -1)
    assert (out - o2).abs().max().item() <= 1e-2 * o2.abs().max().item()


def test_topk_longer_than_the_selection_bitmask():
    """140,000 keys: more than the 131,072 selection bits the ranking kernel
    keeps in LDS, so the ordered output comes from its score-based path."""
    c = W.small_attn(31, 1, 4, 1, 128, 1, (140000,), W.BF16)
    sel, out, lse = _run(c, 512)
    rs, ro, rl = _ref(c, 512)
    assert np.array_equal(sel, rs)
    assert_attention_close(out, lse, ro, rl, np.ones(1, np.int32), W.BF16, "topk long")


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("j1,j2", [(37, 201), (250, 3)])
def test_score_products_are_rounded_before_the_sum(dt, d, j1, j2):
    """Two keys whose order flips if a product is fused into its sum (see
    the oracle's pin of the same case): top-1 must be j2, top-2 both."""
    from test_oracle_topk import _rounding_case
    q, k = _rounding_case(d, 300, j1, j2)
    c = W.small_attn(31, 1, 2, 1, d, 1, (300,), dt)
    c.q, c.k = W.Stored.from_f32(q, dt), W.Stored.from_f32(k, dt)
    for K, want in ((1, [j2]), (2, sorted([j1, j2]))):
        sel, _, _ = _run(c, K)
        assert sel[0, 0].tolist() == want
        assert np.array_equal(sel, _ref(c, K)[0])
