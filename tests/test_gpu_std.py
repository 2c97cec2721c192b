"""Sparse-to-Dense prefill selection and the sparse draft attention over the
kept lists, on the GPU through the C ABI, against the oracle.

Selection parity: the mean attention is compared within its tolerance
(relative 1e-4 plus 1e-9 absolute: fp32 scores and exponentials against
fp64).  The selected set must equal the oracle's except for positions whose
oracle scores lie within twice that tolerance of the oracle's K-th visual
score (near-ties that fp32 may order either way); it must also be a top-K of
the library's own returned scores, and the kept list must be exactly the
sorted union of the selection and the text list."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-9


def _kv(c):
    from speculative_decoding_attention_amd import KVCache
    return KVCache(dev(c.k), dev(c.v), dev(c.kv_len.astype(np.int32)),
                   page_table=dev(c.page_table.astype(np.int32)) if c.page_size else None,
                   page_size=c.page_size, max_len=c.max_len)


def _check_selection(c, sel, keep, keep_len, score, units=None, ref=None):
    """Compare one call's outputs with the oracle on the listed units."""
    K = c.top_k
    if ref is None:
        ref = oracle.std_prefill_select(c.q_text.values, c.k.values, c.kv_len, c.text_idx,
                                        c.text_len, c.num_kv_heads, K, c.scale, c.page_table,
                                        c.page_size)
    sel_ref, sc_ref = ref
    todo = units or [(b, g) for b in range(c.batch) for g in range(c.num_kv_heads)]
    for b, g in todo:
        L, T = int(c.kv_len[b]), int(c.text_len[b])
        text = c.text_idx[b, :T]
        s_ref = sc_ref[b][g]
        s_got = score[b, g, :L].astype(np.float64)
        err = np.abs(s_got - s_ref)
        bad = err > RTOL * s_ref + ATOL
        assert not bad.any(), f"unit {b},{g}: score err {err[bad][:4]} at {np.flatnonzero(bad)[:4]}"
        # selection
        vis = np.setdiff1d(np.arange(L), text)
        n_sel = min(K, len(vis))
        got = sel[b, g]
        assert np.all(got[n_sel:] == -1)
        got = got[:n_sel]
        assert np.all(np.diff(got) > 0) and np.isin(got, vis).all()
        want = sel_ref[b, g, :n_sel]
        diff = np.setxor1d(got, want)
        if diff.size:
            kth = np.sort(s_ref[vis])[::-1][n_sel - 1]
            near = np.abs(s_ref[diff] - kth) <= 2 * (RTOL * kth + ATOL)
            assert near.all(), f"unit {b},{g}: selection differs beyond near-ties: {diff[~near][:8]}"
        # a top-K of the library's own scores
        if n_sel < len(vis):
            rest = np.setdiff1d(vis, got)
            assert score[b, g, got].min() >= score[b, g, rest].max()
        # kept list: ascending union
        u = np.union1d(got, text)
        assert keep_len[b, g] == len(u)
        assert np.array_equal(keep[b, g, :len(u)], u)
        assert np.all(keep[b, g, len(u):] == -1)


CASES = [
    # seed, B, Hq, Hkv, d, L, dtype, n_text, page_size, top_k
    (0, 2, 8, 2, 128, (700, 433), W.BF16, (40, 17), 0, 64),
    (1, 1, 28, 4, 128, (1500,), W.BF16, (150,), 0, 128),     # 7 heads per group, several row blocks
    (2, 2, 4, 1, 64, (520, 300), W.BF16, (33, 60), 0, 40),
    (3, 2, 4, 2, 64, (300, 211), W.F32, (21, 9), 0, 32),
    (4, 2, 8, 2, 128, (900, 611), W.BF16, (50, 20), 16, 100),  # paged
    (5, 2, 4, 2, 128, (260, 140), W.F32, (12, 30), 16, 24),    # paged fp32
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}_d{c[4]}_{c[6]}_ps{c[8]}")
def test_std_select_matches_oracle(case):
    import speculative_decoding_attention_amd as S
    seed, B, Hq, Hkv, d, L, dt, nt, ps, K = case
    c = W.std_small(seed, B, Hq, Hkv, d, L, dt, n_text=nt, page_size=ps, top_k=K)
    kv = _kv(c)
    sel, keep, keep_len, score = S.spec_std_select(kv, dev(c.q_text), dev(c.text_idx),
                                                   dev(c.text_len), K, scale=c.scale,
                                                   want_score=True)
    torch.cuda.synchronize()
    _check_selection(c, sel.cpu().numpy(), keep.cpu().numpy(), keep_len.cpu().numpy(),
                     score.cpu().numpy())


def test_std_select_edge_cases():
    """K above the number of visual positions (every visual position kept,
    the kept list is the whole sequence), one text token at position 0, and a
    sequence without text (scores 0, the first K positions)."""
    import speculative_decoding_attention_amd as S
    c = W.std_small(11, 3, 8, 2, 128, (300, 200, 180), W.BF16, n_text=(20, 1, 0), top_k=290)
    c.text_idx[1, 0] = 0
    kv = _kv(c)
    sel, keep, keep_len, score = S.spec_std_select(kv, dev(c.q_text), dev(c.text_idx),
                                                   dev(c.text_len), c.top_k, scale=c.scale,
                                                   want_score=True)
    torch.cuda.synchronize()
    sel, keep, keep_len, score = (x.cpu().numpy() for x in (sel, keep, keep_len, score))
    _check_selection(c, sel, keep, keep_len, score)
    assert np.array_equal(keep[0, 0, :300], np.arange(300)) and keep_len[0, 0] == 300
    assert np.all(score[2, :, :180] == 0) and np.array_equal(sel[2, 0, :180], np.arange(180))
    # one text token at position 0 sees only itself
    assert score[1, 0, 0] == pytest.approx(1.0, abs=1e-6) and np.all(score[1, 0, 1:200] == 0)


def test_std_select_ties_go_to_the_lower_index():
    """Duplicated key rows placed before every text token score exactly alike,
    on both sides; the cut falls inside the duplicate group."""
    import speculative_decoding_attention_amd as S
    c = W.std_small(12, 1, 8, 2, 128, (600,), W.BF16, n_text=(10,), top_k=40)
    c.text_idx[0, :5] = [200, 250, 300, 350, 400]       # the other 5 trail at 595..599
    bits = c.k.bits
    # one strong key (position 5) copied to 60 positions before the first text token
    src = bits[0, :, 5].copy()
    dst = np.arange(10, 10 + 60)
    bits[0, :, dst] = src
    q = c.q_text.values.copy()
    for g in range(2):
        q[0, :, 4 * g:4 * g + 4] += 4.0 * W.bf16_bits_to_f32(src[g])[None, None, :]
    c.q_text = W.Stored.from_f32(q, W.BF16)
    kv = _kv(c)
    sel, keep, keep_len, score = S.spec_std_select(kv, dev(c.q_text), dev(c.text_idx),
                                                   dev(c.text_len), c.top_k, scale=c.scale,
                                                   want_score=True)
    torch.cuda.synchronize()
    sel, keep, keep_len, score = (x.cpu().numpy() for x in (sel, keep, keep_len, score))
    for g in range(2):
        vals = score[0, g, dst]
        assert np.all(vals == vals[0]), "duplicated keys must score identically"
    _check_selection(c, sel, keep, keep_len, score)


def test_std_select_full_size():
    """The 25k-visual-token prefill (25,512 positions, 512 text tokens, 28/4
    heads, K = 2048): every unit's scores sum to 1, and all four units are
    checked against the oracle in full."""
    import speculative_decoding_attention_amd as S
    c = W.c2_std(0)
    kv = _kv(c)
    sel, keep, keep_len, score = S.spec_std_select(kv, dev(c.q_text), dev(c.text_idx),
                                                   dev(c.text_len), c.top_k, scale=c.scale,
                                                   want_score=True)
    torch.cuda.synchronize()
    sel, keep, keep_len, score = (x.cpu().numpy() for x in (sel, keep, keep_len, score))
    for g in range(4):
        assert abs(score[0, g].astype(np.float64).sum() - 1.0) < 1e-4
    for g in range(4):
        k1 = W.Stored(W.BF16, c.k.bits[:, g:g + 1].copy())
        q1 = W.Stored(W.BF16, c.q_text.bits[:, :, 7 * g:7 * g + 7].copy())
        one = W.StdCase(c.name, c.dtype, q1, k1, k1, c.q, c.kv_len, c.q_len, c.text_idx,
                        c.text_len, 7, 1, c.head_dim, c.max_len, c.top_k)
        _check_selection(one, sel[:, g:g + 1], keep[:, g:g + 1], keep_len[:, g:g + 1],
                         score[:, g:g + 1])


def _random_lists(rng, c, list_max, tail):
    """Per-head ascending position lists below each sequence's tail start."""
    B, Hkv = c.batch, c.num_kv_heads
    lst = np.full((B, Hkv, list_max), -1, np.int32)
    ln = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        t0 = int(c.kv_len[b]) - tail[b]
        for g in range(Hkv):
            n = int(rng.integers(0, min(list_max, t0) + 1)) if g else min(list_max, t0)
            x = np.sort(rng.choice(t0, size=n, replace=False)).astype(np.int32)
            lst[b, g, :n] = x
            ln[b, g] = n
    return lst, ln


SPARSE = [
    # seed, B, Hq, Hkv, d, L, n, dtype, page_size, list_max, tail
    (0, 2, 8, 2, 128, (900, 700), 1, W.BF16, 0, 300, (5, 0)),
    (1, 2, 28, 4, 128, (3000, 2100), 6, W.BF16, 0, 1200, (40, 9)),
    (2, 2, 4, 2, 64, (500, 333), 3, W.BF16, 0, 120, (3, 17)),
    (3, 2, 4, 2, 64, (400, 250), 2, W.F32, 0, 90, (0, 4)),
    (4, 3, 8, 2, 128, (1200, 900, 64), 1, W.BF16, 16, 500, (10, 1, 8)),
    (5, 1, 8, 2, 128, (20000,), 1, W.BF16, 0, 4500, (300,)),   # several gathered splits
]


@pytest.mark.parametrize("case", SPARSE, ids=lambda c: f"s{c[0]}_d{c[4]}_{c[7]}_ps{c[8]}_n{c[6]}")
@pytest.mark.parametrize("with_tail", [True, False])
def test_sparse_attn_matches_oracle(case, with_tail):
    import speculative_decoding_attention_amd as S
    seed, B, Hq, Hkv, d, L, n, dt, ps, list_max, tail = case
    c = W.std_small(seed, B, Hq, Hkv, d, L, dt, n_text=1, page_size=ps, n=n)
    rng = np.random.default_rng(100 + seed)
    tail = np.asarray(tail if with_tail else (0,) * B, np.int32)
    lst, ln = _random_lists(rng, c, list_max, tail)
    t0 = (c.kv_len - tail).astype(np.int32)
    kv = _kv(c)
    o, l = S.spec_sparse_attn(kv, dev(c.q), dev(lst), dev(ln),
                              tail_start=dev(t0) if with_tail else None,
                              tail_max=int(tail.max()) if with_tail else 0, scale=c.scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len, lst,
                                     ln, t0 if with_tail else None, Hkv, c.scale, c.page_table,
                                     c.page_size)
    assert_attention_close(o, l, ro, rl, c.q_len, dt, tag=str(case))


WINDOW = [
    # seed, B, Hq, Hkv, d, L, n, dtype, page_size, list_max, window
    (20, 2, 8, 2, 128, (900, 700), 1, W.BF16, 0, 64, 128),
    (21, 2, 28, 4, 128, (3000, 40), 6, W.BF16, 0, 300, 256),   # window longer than one sequence
    (22, 2, 4, 2, 64, (500, 333), 3, W.F32, 0, 50, 32),
    (23, 3, 8, 2, 128, (1200, 900, 64), 2, W.BF16, 16, 200, 100),
]


@pytest.mark.parametrize("case", WINDOW, ids=lambda c: f"s{c[0]}_d{c[4]}_{c[7]}_ps{c[8]}_w{c[10]}")
@pytest.mark.parametrize("anchors", ["none", "shared", "per_head"])
def test_window_variants_match_oracle(case, anchors):
    """Text-anchored window variants: a sliding window of the last W
    positions alone, with the same anchor list for every head, or with
    per-head anchor lists; anchors may fall inside the window (counted
    once)."""
    import speculative_decoding_attention_amd as S
    seed, B, Hq, Hkv, d, L, n, dt, ps, list_max, win = case
    c = W.std_small(seed, B, Hq, Hkv, d, L, dt, n_text=1, page_size=ps, n=n)
    rng = np.random.default_rng(200 + seed)
    lst = np.full((B, Hkv, list_max), -1, np.int32)
    ln = np.zeros((B, Hkv), np.int32)
    if anchors != "none":
        for b in range(B):
            Lb = int(c.kv_len[b])
            m = min(list_max, Lb)
            base = np.sort(rng.choice(Lb, size=m, replace=False))
            for g in range(Hkv):
                x = base if anchors == "shared" else np.sort(rng.choice(Lb, size=m, replace=False))
                lst[b, g, :m] = x
                ln[b, g] = m
    kv = _kv(c)
    o, l = S.spec_sparse_attn(kv, dev(c.q), dev(lst), dev(ln), tail_start=None, tail_max=win,
                              scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len, lst,
                                     ln, None, Hkv, c.scale, c.page_table, c.page_size, window=win)
    assert_attention_close(o, l, ro, rl, c.q_len, dt, tag=f"{case} {anchors}")


def test_select_then_sparse_decode_end_to_end():
    """Prefill selection followed by a decode step over the kept lists and the
    tokens written since, both on the GPU, against the same two steps of the
    oracle (the selections agree exactly on this seeded case)."""
    import speculative_decoding_attention_amd as S
    c = W.std_small(21, 2, 8, 2, 128, (1400, 1000), W.BF16, n_text=(60, 30), top_k=200, n=4)
    prefill = (c.kv_len - 6).astype(np.int32)      # 6 tokens decoded since the prefill
    pre_len = dev(prefill)
    from speculative_decoding_attention_amd import KVCache
    kv_pre = KVCache(dev(c.k), dev(c.v), pre_len, max_len=c.max_len)
    ti = c.text_idx.copy()
    # the text tokens of the prefill: the leading entries of each ascending list
    tl = np.array([np.sum(ti[b, :c.text_len[b]] < prefill[b]) for b in range(c.batch)], np.int32)
    sel, keep, keep_len, _ = S.spec_std_select(kv_pre, dev(c.q_text), dev(ti), dev(tl), c.top_k,
                                               scale=c.scale)
    kv = _kv(c)
    o, l = S.spec_sparse_attn(kv, dev(c.q), keep, keep_len, tail_start=pre_len, tail_max=6,
                              scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rsel, _ = oracle.std_prefill_select(c.q_text.values, c.k.values, prefill, ti, tl, 2,
                                        c.top_k, c.scale)
    assert np.array_equal(sel.cpu().numpy(), rsel)
    rkeep, rlen = oracle.std_keep_list(rsel, ti, tl)
    assert np.array_equal(keep.cpu().numpy(), rkeep) and np.array_equal(keep_len.cpu().numpy(), rlen)
    ro, rl = oracle.sparse_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len, rkeep,
                                     rlen, prefill, 2, c.scale)
    assert_attention_close(o, l, ro, rl, c.q_len, W.BF16, tag="e2e")


def test_std_select_longer_than_the_selection_bitmask():
    """140,000 positions (past the ranking kernel's LDS bit mask) with 24 text
    tokens, K = 1000."""
    import speculative_decoding_attention_amd as S
    c = W.std_small(33, 1, 4, 2, 128, (140000,), W.BF16, n_text=(24,), top_k=1000)
    kv = _kv(c)
    sel, keep, keep_len, score = S.spec_std_select(kv, dev(c.q_text), dev(c.text_idx),
                                                   dev(c.text_len), c.top_k, scale=c.scale,
                                                   want_score=True)
    torch.cuda.synchronize()
    _check_selection(c, sel.cpu().numpy(), keep.cpu().numpy(), keep_len.cpu().numpy(),
                     score.cpu().numpy())
