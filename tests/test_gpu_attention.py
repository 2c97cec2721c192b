"""GPU parity of verification and text-anchored attention against the CPU
oracle, at test sizes that span several tiles and splits with ragged tails,
and at the full workload sizes the bench times."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV, assert_attention_close, dev, kvcache

pytestmark = pytest.mark.gpu


def _lib():
    import speculative_decoding_attention_amd as S
    return S


def _verify_pair(c, out_dtype=torch.float32):
    S = _lib()
    kv = kvcache(c)
    q_len = dev(c.q_len.astype(np.int32))
    out, lse = S.spec_verify_attn(kv, dev(c.q), q_len=q_len, scale=c.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len,
                                     c.num_kv_heads, c.scale, c.page_table, c.page_size)
    return out, lse, ro, rl


def _vata_pair(c, out_dtype=torch.float32, idx=None, tlen=None):
    S = _lib()
    idx = c.text_idx if idx is None else idx
    tlen = c.text_len if tlen is None else tlen
    kv = kvcache(c)
    out, lse = S.spec_vata_attn(kv, dev(c.q), dev(idx.astype(np.int32)),
                                dev(tlen.astype(np.int32)), q_len=dev(c.q_len.astype(np.int32)),
                                scale=c.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.vata_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len, idx,
                                   tlen, c.num_kv_heads, c.scale, c.page_table, c.page_size)
    return out, lse, ro, rl


# ------------------------------------------------------------ tiny (C1) ----

def test_c1_verify_fp32():
    c, _ = W.c1_tiny()
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.F32, "c1 verify")


@pytest.mark.parametrize("n", [1, 5])
def test_c1_vata_fp32(n):
    c, _ = W.c1_tiny()
    if n == 1:
        c.q = W.Stored(W.F32, c.q.bits[:, -1:].copy())
        c.q_len = np.array([1], np.int32)
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.F32, f"c1 vata n={n}")


# ------------------------------------------------------- small ragged ----

SMALL = [
    # seed, B, Hq, Hkv, d, n, L, dtype, page
    (1, 2, 8, 2, 128, 5, (700, 1333), W.BF16, 0),
    (2, 3, 28, 4, 128, 6, (2000, 77, 1029), W.BF16, 16),
    (3, 2, 4, 1, 64, 3, (300, 901), W.BF16, 0),
    (4, 2, 14, 2, 128, 8, (517, 1500), W.BF16, 32),     # 56 rows per unit
    (5, 2, 4, 2, 64, 4, (250, 999), W.F32, 0),
    (6, 1, 6, 2, 128, 2, (1025,), W.F32, 16),
    (7, 2, 16, 1, 128, 4, (64, 1), W.BF16, 0),          # 64 rows; a 1-key sequence
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"s{c[0]}")
def test_small_verify(cfg):
    seed, B, Hq, Hkv, d, n, L, dt, page = cfg
    n_eff = [min(n, x) for x in np.broadcast_to(L, (B,))]
    c = W.small_attn(seed, B, Hq, Hkv, d, n, L, dt, page_size=page, q_len=n_eff)
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, dt, f"small verify {seed}")


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"s{c[0]}")
def test_small_vata(cfg):
    seed, B, Hq, Hkv, d, n, L, dt, page = cfg
    n_eff = [min(n, x) for x in np.broadcast_to(L, (B,))]
    c = W.small_attn(seed, B, Hq, Hkv, d, n, L, dt, page_size=page, q_len=n_eff)
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, dt, f"small vata {seed}")


# One sequence, many splits: the grouped merge takes one output column per
# thread below 128 merged rows (3 KV heads x 42 rows = 126) and two columns
# per thread, one workgroup per row, from 128 on (4 x 42 = 168).
@pytest.mark.parametrize("Hq,Hkv", [(21, 3), (28, 4)])
@pytest.mark.parametrize("page,q_len", [(0, None), (16, None), (0, [4])])
def test_grouped_merge_both_widths(Hq, Hkv, page, q_len):
    # q_len [4] of 6: the merged rows of the two padded query positions are 0, LSE -inf
    c = W.small_attn(91 + Hkv, 1, Hq, Hkv, 128, 6, 6000, W.BF16, page_size=page, q_len=q_len)
    for out_dtype in (torch.float32, torch.bfloat16):
        out, lse, ro, rl = _verify_pair(c, out_dtype)
        assert_attention_close(out.float(), lse, ro, rl, c.q_len, W.BF16,
                               f"grouped merge {Hq}/{Hkv} page {page} {out_dtype}")


@pytest.mark.parametrize("n,page", [(1, 0), (3, 16), (6, 0)])
def test_many_short_units(n, page):
    """A batch of 32 short ragged sequences: 128 units of one or two splits,
    so the split kernel's waves write their own partials and the merge takes
    the one-thread-per-column path (at most 8 partials per unit)."""
    rng = np.random.default_rng(50 + n)
    L = tuple(int(x) for x in rng.integers(max(n, 100), 601, size=32))
    c = W.small_attn(60 + n, 32, 28, 4, 128, n, L, W.BF16, page_size=page)
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"short units verify n={n}")
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"short units vata n={n}")


@pytest.mark.parametrize("page", [0, 16])
def test_balanced_splits_of_very_uneven_lengths(page):
    """Balanced splits from the device lengths: one long sequence beside
    very short ones (and a 1-position one) in a batch of 5, so the long
    sequence takes most of the splits and the short ones one each;
    verification and text-anchored attention, paged and contiguous."""
    L = (30000, 7, 1, 650, 129)
    c = W.small_attn(91 + page, 5, 28, 4, 128, 6, L, W.BF16, page_size=page,
                     q_len=[6, 6, 1, 6, 6])
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "uneven verify")
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "uneven vata")


@pytest.mark.parametrize("B,Hkv,lmax,page", [(64, 2, 1200, 0), (64, 2, 1200, 16),
                                              (2, 4, 40000, 0), (47, 4, 3000, 0)])
def test_balanced_plan_over_batch_sizes(B, Hkv, lmax, page):
    """Balanced splits for a batch that gives every lane of the plan's
    wave-wide sums a length (64 sequences, so lanes in all four 16-lane rows
    count; two KV heads, so the capacity plan has two splits per unit and
    the balanced plan applies), two very unequal sequences, and an odd
    batch, each verified against the oracle (one or two query rows)."""
    rng = np.random.default_rng(700 + B + page)
    L = [int(x) for x in rng.integers(1, lmax + 1, size=B)]
    if B == 2:
        L = [lmax, 3]
    ql = [min(2, x) for x in L]
    c = W.small_attn(710 + B + page, B, 4 * Hkv, Hkv, 128, 2, tuple(L), W.BF16,
                     page_size=page, q_len=ql)
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"balanced B={B} page={page}")


def test_padded_query_rows_and_bf16_output():
    c = W.small_attn(11, 3, 8, 2, 128, 6, (900, 450, 1200), W.BF16, q_len=[6, 2, 4])
    out, lse, ro, rl = _verify_pair(c, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "padded rows")


def test_vata_empty_and_partial_lists():
    """text_len = 0 gives O = 0, LSE = -inf; a list whose entries all lie
    after the first rows' positions leaves those rows empty."""
    c = W.small_attn(12, 2, 8, 2, 128, 4, (600, 600), W.BF16)
    idx = np.zeros((2, 8), np.int32)
    idx[1, :3] = [597, 598, 599]            # rows 0..2 of seq 1 see 0..2 entries
    tlen = np.array([0, 3], np.int32)
    out, lse, ro, rl = _vata_pair(c, idx=idx, tlen=tlen)
    o = out.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0].cpu().numpy()))
    assert np.all(np.isneginf(lse[1, 0].cpu().numpy()))
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "vata partial")



@pytest.mark.parametrize("n,page", [(1, 0), (6, 0), (6, 16)])
def test_vata_unordered_list_with_repeats(n, page):
    """A list in no particular order, with repeated positions: 32-entry
    blocks whose positions all precede every query row alternate with blocks
    that hide one of the last n positions (visible to some rows only) at a
    random place, so whole-block visibility is decided per block."""
    L = (2400, 1900)
    c = W.small_attn(21 + n, 2, 28, 4, 128, n, L, W.BF16, page_size=page)
    rng = np.random.default_rng(77 + n)
    T = 1200
    idx = np.zeros((2, T), np.int32)
    for b, Lb in enumerate(L):
        early = rng.integers(0, Lb - n, size=T).astype(np.int32)
        early[5:9] = early[1]                        # repeats
        for blk in range(1, T // 32, 2):             # every other block hides a late one
            idx_in = blk * 32 + int(rng.integers(0, 32))
            early[idx_in] = Lb - 1 - int(rng.integers(0, n))
        idx[b] = early
    tlen = np.array([T, T - 45], np.int32)           # a ragged final block
    out, lse, ro, rl = _vata_pair(c, idx=idx, tlen=tlen)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"vata unordered n={n}")

# -------------------------------------------------------- invariants ----

def test_values_one_gives_one_and_lse_normalises():
    c = W.small_attn(13, 2, 28, 4, 128, 6, (3000, 2111), W.BF16)
    c.v = W.Stored.from_f32(np.ones(c.v.shape, np.float32), W.BF16)
    out, lse, ro, rl = _verify_pair(c)
    dev1 = float(np.abs(out.cpu().numpy() - 1.0).max())
    assert dev1 < 1e-6, dev1
    # sum_j exp(s_j - LSE) = 1 with scores from torch fp64 on the device data
    b, i, h = 1, 3, 17
    L, n = int(c.kv_len[b]), int(c.q_len[b])
    k = torch.tensor(c.k.values[b, h // 7, :L - n + i + 1], dtype=torch.float64)
    s = c.scale * (k @ torch.tensor(c.q.values[b, i, h], dtype=torch.float64))
    assert abs(float(torch.exp(s - float(lse[b, i, h])).sum()) - 1.0) < 1e-5


def test_vata_all_positions_equals_verify_on_device():
    S = _lib()
    c = W.small_attn(14, 2, 28, 4, 128, 6, (1800, 2500), W.BF16)
    kv = kvcache(c)
    q = dev(c.q)
    o1, l1 = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    idx = torch.arange(c.max_len, dtype=torch.int32, device=DEV).repeat(2, 1).contiguous()
    o2, l2 = S.spec_vata_attn(kv, q, idx, dev(c.kv_len.astype(np.int32)), scale=c.scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_first_verify_row_equals_decode_on_device():
    S = _lib()
    c = W.small_attn(15, 2, 28, 4, 128, 6, (2222, 1111), W.BF16)
    kv = kvcache(c)
    o, l = S.spec_verify_attn(kv, dev(c.q), scale=c.scale, out_dtype=torch.float32)
    kv1 = kvcache(c)
    kv1_len = dev((c.kv_len - 5).astype(np.int32))
    from speculative_decoding_attention_amd import KVCache
    kvd = KVCache(kv1.k, kv1.v, kv1_len)
    od, ld = S.spec_verify_attn(kvd, dev(c.q)[:, :1].contiguous(), scale=c.scale,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the two calls tile the keys differently, so bf16 probability rounding
    # differs: same scale-aware bound as the oracle parity checks
    assert (o[:, 0] - od[:, 0]).abs().max().item() < 1e-2 * o.abs().max().item()
    assert (l[:, 0] - ld[:, 0]).abs().max().item() < 1e-4


@pytest.mark.parametrize("d", [64, 128])
def test_every_verify_row_equals_decode_fp32(d):
    """fp32 inputs: verification row i equals a one-row decode over the
    prefix it sees (kv_len = L - n + i + 1) within 1e-5, for every row i.
    fp32 probabilities are not rounded, so the two tilings differ only in
    summation order."""
    S = _lib()
    from speculative_decoding_attention_amd import KVCache
    n = 6
    c = W.small_attn(18 + d, 2, 8, 2, d, n, (2222, 1111), W.F32)
    kv = kvcache(c)
    q = dev(c.q)
    o, l = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    for i in range(n):
        kvd = KVCache(kv.k, kv.v, dev((c.kv_len - n + i + 1).astype(np.int32)))
        od, ld = S.spec_verify_attn(kvd, q[:, i:i + 1].contiguous(), scale=c.scale,
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert (o[:, i] - od[:, 0]).abs().max().item() <= 1e-5, f"row {i}"
        assert (l[:, i] - ld[:, 0]).abs().max().item() <= 1e-5, f"row {i} lse"


def test_paged_equals_contiguous_on_device():
    S = _lib()
    c = W.small_attn(16, 2, 28, 4, 128, 6, (1700, 2600), W.BF16, page_size=16)
    o1, l1 = S.spec_verify_attn(kvcache(c), dev(c.q), scale=c.scale, out_dtype=torch.float32)
    B, Hkv, d, Lm = 2, 4, 128, c.max_len
    kc = np.zeros((B, Hkv, Lm, d), np.uint16)
    vc = np.zeros((B, Hkv, Lm, d), np.uint16)
    for b in range(B):
        L = int(c.kv_len[b])
        kc[b, :, :L] = oracle.paged_rows(c.k.bits, c.page_table, b, L, 16)
        vc[b, :, :L] = oracle.paged_rows(c.v.bits, c.page_table, b, L, 16)
    from speculative_decoding_attention_amd import KVCache
    kv2 = KVCache(dev(W.Stored(W.BF16, kc)), dev(W.Stored(W.BF16, vc)),
                  dev(c.kv_len.astype(np.int32)))
    o2, l2 = S.spec_verify_attn(kv2, dev(c.q), scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
@pytest.mark.parametrize("L,max_len", [((5000, 3100, 130), 5600), ((904, 2017, 130), 5600),
                                       ((938, 997, 1300), 5600), ((1064, 1131, 2400), 5600),
                                       ((2017,), 18432), ((5000,), 18432), ((997,), 18432),
                                       ((1064,), 18432), ((1131,), 18432)])
def test_rows_past_the_length_are_never_used(dt, L, max_len):
    """Cache capacity beyond kv_len holds NaN keys and infinite values: the
    output must still match the oracle (which never reads those rows).
    Batches of several sequences split the lengths present.  A single
    sequence is split over the capacity: with 256 CUs, 18,432 positions plan
    288-key splits whose first two 64-key tiles the dense bf16 kernel
    requests before the length is known; 2017 ends inside a split's tile 0
    and 5000 inside tile 1, so those tiles are requested again; 997, 1064
    and 1131 end inside tiles 2, 3 and 4, which are requested only after the
    length is known."""
    B = len(L)
    c = W.small_attn(41, B, 28, 4, 128, 6, L, dt, max_len=max_len)
    kb, vb = c.k.bits.copy(), c.v.bits.copy()
    nan, inf = (0x7FC0, 0x7F80) if dt == W.BF16 else (np.nan, np.inf)   # bf16 bits / fp32 values
    for b_ in range(B):
        kb[b_, :, L[b_]:] = nan
        vb[b_, :, L[b_]:] = inf
    c.k, c.v = W.Stored(dt, kb), W.Stored(dt, vb)
    out, lse, ro, rl = _verify_pair(c)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    assert_attention_close(out, lse, ro, rl, c.q_len, dt, "rows past the length")


def test_repeated_calls_are_bitwise_identical():
    S = _lib()
    c = W.small_attn(17, 1, 28, 4, 128, 6, (25512,), W.BF16)
    kv = kvcache(c)
    q = dev(c.q)
    ref = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    for _ in range(3):
        o, l = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])


# ------------------------------------------------- full workload sizes ----

@pytest.fixture(scope="module")
def c2():
    return W.c2_sparrow(0, with_hsr=False)[0]


def test_c2_verify_full(c2):
    out, lse, ro, rl = _verify_pair(c2)
    assert_attention_close(out, lse, ro, rl, c2.q_len, W.BF16, "c2 verify")


def test_c2_verify_bf16_output_as_benched(c2):
    out, lse, ro, rl = _verify_pair(c2, out_dtype=torch.bfloat16)
    assert_attention_close(out, lse, ro, rl, c2.q_len, W.BF16, "c2 verify bf16 out")


@pytest.mark.parametrize("n", [1, 6])
def test_c2_vata_full(c2, n):
    c = c2
    if n == 1:
        c = W.AttnCase(**{**c2.__dict__})
        c.q = W.Stored(W.BF16, c2.q.bits[:, -1:].copy())
        c.q_len = np.array([1], np.int32)
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"c2 vata n={n}")


@pytest.fixture(scope="module")
def c3():
    return W.c3_ragged_paged(0)


def test_c3_verify_full(c3):
    out, lse, ro, rl = _verify_pair(c3)
    assert_attention_close(out, lse, ro, rl, c3.q_len, W.BF16, "c3 verify")


def test_c3_vata_full(c3):
    out, lse, ro, rl = _vata_pair(c3)
    assert_attention_close(out, lse, ro, rl, c3.q_len, W.BF16, "c3 vata")


def test_c4_verify_full():
    """Dense verification at L = 32768, B = 4: every output of all 16
    (sequence, KV head) units against the oracle."""
    c = W.c4_topk(0)
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "c4 verify")


def test_verify_and_vata_long_context():
    """A 300,000-position sequence next to a short one (4 query rows, 4 heads
    per group): the split plan and the merge at long length."""
    c = W.small_attn(32, 2, 4, 1, 128, 4, (300000, 700), W.BF16, text_frac=0.01)
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "long verify")
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "long vata")


@pytest.mark.parametrize("page_size", [1, 2, 256])
@pytest.mark.parametrize("G", [1, 7])
def test_page_size_limits_and_group_sizes(page_size, G):
    """The smallest and largest page sizes, one query head per KV head (plain
    multi-head attention) and seven; verification and text-anchored attention."""
    c = W.small_attn(40 + page_size + G, 2, 2 * G, 2, 128, 3, (611, 300), W.BF16,
                     page_size=page_size)
    out, lse, ro, rl = _verify_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"verify ps{page_size} G{G}")
    out, lse, ro, rl = _vata_pair(c)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, f"vata ps{page_size} G{G}")
