"""Pins of the attention oracles against facts that do not come from the
oracle itself: closed forms, invariants of softmax attention, a library
routine (torch's scaled-dot-product attention on the CPU in float64), and the
consistency checks the method fixes (text-anchored attention with every
position listed equals dense attention; the first verification row equals
one-token decode)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _case(seed=1, B=2, Hq=4, Hkv=2, d=16, n=3, L=(37, 50), page=0, dtype=W.F32):
    return W.small_attn(seed, B, Hq, Hkv, d, n, L, dtype, page_size=page)


def _verify(c, **kw):
    return oracle.verify_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len,
                                   c.num_kv_heads, c.scale, c.page_table, c.page_size, **kw)


def _sdpa_reference(c):
    """torch SDPA (float64, CPU) on logical rows with an explicit boolean mask."""
    B, n, Hq, d = c.q.shape
    G = Hq // c.num_kv_heads
    out = np.zeros((B, n, Hq, d))
    for b in range(B):
        L, nb = int(c.kv_len[b]), int(c.q_len[b])
        k = oracle.paged_rows(c.k.values, c.page_table, b, L, c.page_size) if c.page_size \
            else c.k.values[b, :, :L]
        v = oracle.paged_rows(c.v.values, c.page_table, b, L, c.page_size) if c.page_size \
            else c.v.values[b, :, :L]
        q = torch.tensor(c.q.values[b, :nb], dtype=torch.float64).permute(1, 0, 2)  # [Hq, nb, d]
        kt = torch.tensor(np.repeat(k, G, axis=0), dtype=torch.float64)             # [Hq, L, d]
        vt = torch.tensor(np.repeat(v, G, axis=0), dtype=torch.float64)
        mask = torch.tensor(np.arange(L)[None, :] <= (L - nb + np.arange(nb))[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(q, kt, vt, attn_mask=mask,
                                                             scale=c.scale)
        out[b, :nb] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("page", [0, 16])
def test_verify_matches_torch_sdpa_fp64(page):
    c = _case(page=page)
    o, lse = _verify(c)
    ref = _sdpa_reference(c)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_verify_lse_normalises_probabilities():
    """Check (2): with p_j = exp(s_j - LSE), sum_j p_j = 1, using scores from
    torch's matmul rather than the oracle's."""
    c = _case(seed=3)
    o, lse = _verify(c)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.batch):
        L, nb = int(c.kv_len[b]), int(c.q_len[b])
        for i in range(nb):
            for h in range(c.num_q_heads):
                k = torch.tensor(c.k.values[b, h // G, :L - nb + i + 1], dtype=torch.float64)
                s = c.scale * (k @ torch.tensor(c.q.values[b, i, h], dtype=torch.float64))
                assert abs(float(torch.exp(s - lse[b, i, h]).sum()) - 1.0) < 1e-12


def test_values_all_one_give_one():
    c = _case(seed=4)
    c.v = W.Stored.from_f32(np.ones_like(c.v.values), W.F32)
    o, _ = _verify(c)
    nb = c.q_len
    for b in range(c.batch):
        assert np.allclose(o[b, :nb[b]], 1.0, atol=1e-14, rtol=0)


def test_zero_query_is_uniform_over_visible_prefix():
    """Q = 0 makes every visible score 0: row i averages V[0..P_i] and
    LSE = ln(P_i + 1).  Pins the mask count exactly."""
    c = _case(seed=5)
    c.q = W.Stored.from_f32(np.zeros_like(c.q.values), W.F32)
    o, lse = _verify(c)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.batch):
        L, nb = int(c.kv_len[b]), int(c.q_len[b])
        for i in range(nb):
            P = L - nb + i
            for h in range(c.num_q_heads):
                mean = c.v.values[b, h // G, :P + 1].astype(np.float64).mean(axis=0)
                assert np.max(np.abs(o[b, i, h] - mean)) < 1e-13
                assert abs(lse[b, i, h] - math.log(P + 1)) < 1e-13


def test_single_key_returns_its_value():
    c = W.small_attn(6, 1, 2, 1, 8, 1, 1, W.F32)
    o, lse = _verify(c)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], c.v.values[0, 0, 0].astype(np.float64))
        s = c.scale * float(np.dot(c.q.values[0, 0, h].astype(np.float64),
                                   c.k.values[0, 0, 0].astype(np.float64)))
        assert abs(lse[0, 0, h] - s) < 1e-14


def test_two_key_closed_form():
    """d = 1, keys k0, k1, values v0, v1, one query q at position 1:
    o = (v0 + e^{x} v1) / (1 + e^{x}) with x = scale*q*(k1 - k0)."""
    q, k0, k1, v0, v1, scale = 0.75, -1.25, 2.5, 3.0, -2.0, 0.5
    c = W.small_attn(7, 1, 1, 1, 1, 1, 2, W.F32)
    c.q = W.Stored.from_f32(np.array([[[[q]]]]), W.F32)
    c.k = W.Stored.from_f32(np.array([[[[k0], [k1]]]]), W.F32)
    c.v = W.Stored.from_f32(np.array([[[[v0], [v1]]]]), W.F32)
    o, lse = oracle.verify_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len,
                                     1, scale)
    x = scale * q * (k1 - k0)
    assert abs(o[0, 0, 0, 0] - (v0 + math.exp(x) * v1) / (1 + math.exp(x))) < 1e-14
    assert abs(lse[0, 0, 0] - (scale * q * k0 + math.log1p(math.exp(x)))) < 1e-14


def test_first_verify_row_equals_decode():
    """Check (3): verification row i equals a one-row decode over the prefix
    that ends at its own position."""
    c = _case(seed=8, n=4)
    o, lse = _verify(c)
    for i in range(4):
        q1 = c.q.values[:, i:i + 1]
        L1 = c.kv_len - c.q_len + i + 1
        o1, l1 = oracle.verify_attention(q1, c.k.values, c.v.values, L1, np.ones(c.batch, np.int32),
                                         c.num_kv_heads, c.scale)
        assert np.max(np.abs(o1[:, 0] - o[:, i])) < 1e-14
        assert np.max(np.abs(l1[:, 0] - lse[:, i])) < 1e-14


def test_gqa_equals_replicated_heads():
    c = _case(seed=9, Hq=6, Hkv=2)
    o, lse = _verify(c)
    G = 3
    k_rep = np.repeat(c.k.values, G, axis=1)
    v_rep = np.repeat(c.v.values, G, axis=1)
    o2, l2 = oracle.verify_attention(c.q.values, k_rep, v_rep, c.kv_len, c.q_len, 6, c.scale)
    assert np.max(np.abs(o - o2)) < 1e-14 and np.max(np.abs(lse - l2)) < 1e-14


def test_padded_rows_are_zero_and_minus_inf():
    c = W.small_attn(10, 2, 2, 1, 8, 4, (20, 30), W.F32, q_len=[2, 4])
    o, lse = _verify(c)
    assert np.all(o[0, 2:] == 0) and np.all(np.isneginf(lse[0, 2:]))
    assert np.all(np.isfinite(lse[1]))


def test_paged_equals_contiguous():
    c = _case(seed=11, page=16, L=(45, 64))
    o, lse = _verify(c)
    B, Hkv, d = c.batch, c.num_kv_heads, c.head_dim
    Lmax = int(c.kv_len.max())
    kc = np.zeros((B, Hkv, Lmax, d), np.float32)
    vc = np.zeros((B, Hkv, Lmax, d), np.float32)
    for b in range(B):
        L = int(c.kv_len[b])
        kc[b, :, :L] = oracle.paged_rows(c.k.values, c.page_table, b, L, 16)
        vc[b, :, :L] = oracle.paged_rows(c.v.values, c.page_table, b, L, 16)
    o2, l2 = oracle.verify_attention(c.q.values, kc, vc, c.kv_len, c.q_len, Hkv, c.scale)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_paged_rows_brute_force():
    pool = np.arange(5 * 1 * 4 * 1, dtype=np.float32).reshape(5, 1, 4, 1)
    table = np.array([[3, 0, 4]], np.int32)
    rows = oracle.paged_rows(pool, table, 0, 10, 4)
    expect = [pool[3, 0, s, 0] for s in range(4)] + [pool[0, 0, s, 0] for s in range(4)] + \
             [pool[4, 0, s, 0] for s in range(2)]
    assert rows[0, :, 0].tolist() == expect


# ---------------------------------------------------------------- VATA ----

def _vata(c, idx=None, tlen=None):
    idx = c.text_idx if idx is None else idx
    tlen = c.text_len if tlen is None else tlen
    return oracle.vata_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len, idx, tlen,
                                 c.num_kv_heads, c.scale, c.page_table, c.page_size)


@pytest.mark.parametrize("page", [0, 16])
def test_vata_all_positions_equals_dense(page):
    """Check (1): with every position listed, text-anchored attention is dense
    attention."""
    c = _case(seed=12, page=page)
    Lmax = int(c.kv_len.max())
    idx = np.tile(np.arange(Lmax, dtype=np.int32), (c.batch, 1))
    o1, l1 = _vata(c, idx, c.kv_len)
    o2, l2 = _verify(c)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14


def test_vata_matches_sdpa_on_gathered_rows():
    c = _case(seed=13)
    o, lse = _vata(c)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.batch):
        L, nb, T = int(c.kv_len[b]), int(c.q_len[b]), int(c.text_len[b])
        idx = c.text_idx[b, :T]
        q = torch.tensor(c.q.values[b, :nb], dtype=torch.float64).permute(1, 0, 2)
        kt = torch.tensor(np.repeat(c.k.values[b][:, idx], G, axis=0), dtype=torch.float64)
        vt = torch.tensor(np.repeat(c.v.values[b][:, idx], G, axis=0), dtype=torch.float64)
        mask = torch.tensor(idx[None, :] <= (L - nb + np.arange(nb))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(q, kt, vt, attn_mask=mask,
                                                               scale=c.scale)
        assert np.max(np.abs(o[b, :nb] - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_vata_own_position_only_returns_own_value():
    c = _case(seed=14, n=1)
    idx = (c.kv_len - 1).astype(np.int32)[:, None]
    o, _ = _vata(c, idx, np.ones(c.batch, np.int32))
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.batch):
        for h in range(c.num_q_heads):
            assert np.array_equal(o[b, 0, h], c.v.values[b, h // G, c.kv_len[b] - 1])


def test_vata_never_reads_unlisted_rows():
    """Poisoning every unlisted K/V row leaves the result unchanged."""
    c = _case(seed=15)
    o1, l1 = _vata(c)
    k = c.k.values.copy()
    v = c.v.values.copy()
    for b in range(c.batch):
        listed = np.zeros(k.shape[2], bool)
        listed[c.text_idx[b, :c.text_len[b]]] = True
        k[b, :, ~listed] = 1e6
        v[b, :, ~listed] = -1e6
    o2, l2 = oracle.vata_attention(c.q.values, k, v, c.kv_len, c.q_len, c.text_idx, c.text_len,
                                   c.num_kv_heads, c.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_vata_empty_set_gives_zero():
    c = _case(seed=16, n=2)
    idx = np.full((c.batch, 1), 0, np.int32)
    o, lse = _vata(c, idx, np.zeros(c.batch, np.int32))
    assert np.all(o == 0) and np.all(np.isneginf(lse[:, :2]))


def test_vata_repeated_position_counts_twice():
    """A position listed twice carries double weight: d = 1, keys 0 and 1 with
    position 1 listed twice gives o = (v0 + 2 e^x v1) / (1 + 2 e^x)."""
    q, k0, k1, v0, v1, scale = 1.0, 0.0, 1.0, 1.0, 5.0, 1.0
    qa = np.array([[[[q]]]], np.float32)
    ka = np.array([[[[k0], [k1]]]], np.float32)
    va = np.array([[[[v0], [v1]]]], np.float32)
    o, _ = oracle.vata_attention(qa, ka, va, np.array([2]), np.array([1]),
                                 np.array([[0, 1, 1]], np.int32), np.array([3]), 1, scale)
    x = math.exp(scale * q * (k1 - k0))
    assert abs(o[0, 0, 0, 0] - (v0 + 2 * x * v1) / (1 + 2 * x)) < 1e-14
