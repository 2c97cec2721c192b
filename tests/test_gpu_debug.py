"""Debug mode (spec_set_debug / SPEC_DEBUG=1): valid inputs give the same
results as with debug off, and each out-of-range device index array is
reported as SPEC_ERR_SHAPE before anything is launched.

Every invalid input below is chosen so that, were it to reach the kernels, all
accesses would still stay inside allocated memory (an over-long first
sequence reads into the next one's rows, a negative page number lands on a
spare page placed in front of the pool)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, kvcache

pytestmark = pytest.mark.gpu

SHAPE = 2


@pytest.fixture
def S():
    import speculative_decoding_attention_amd as S
    prev = S.spec_set_debug(True)
    yield S
    S.spec_set_debug(prev)


def _case(page_size=0):
    return W.small_attn(41, 2, 8, 2, 128, 6, (900, 700), W.BF16, page_size=page_size,
                        max_len=1024 if not page_size else None)


def _rejects(fn):
    import speculative_decoding_attention_amd as S
    with pytest.raises(S.SpecError) as e:
        fn()
    assert e.value.status == SHAPE, str(e.value)


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_valid_inputs_match_debug_off(S):
    c = _case()
    kv = kvcache(c)
    q = dev(c.q)
    q1 = q[:, -1:].contiguous()
    idx, tl = dev(c.text_idx), dev(c.text_len)
    rng = np.random.default_rng(2)
    logits = dev(W.Stored.from_f32(rng.standard_normal((2, 6, 5000)).astype(np.float32), W.BF16))
    draft = dev(rng.integers(0, 5000, size=(2, 5)).astype(np.int32))
    gamma = dev(np.array([5, 2], np.int32))
    calls = [
        lambda: S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32),
        lambda: S.spec_vata_attn(kv, q, idx, tl, scale=c.scale, out_dtype=torch.float32),
        lambda: S.spec_topk_attn(kv, q1, 64, scale=c.scale, out_dtype=torch.float32),
        lambda: S.spec_accept(logits, draft, gamma),
    ]
    on = [f() for f in calls]
    torch.cuda.synchronize()
    S.spec_set_debug(False)
    off = [f() for f in calls]
    torch.cuda.synchronize()
    for a, b in zip(on, off):
        _same(a, b)


def test_bad_lengths_are_rejected(S):
    c = _case()
    q = dev(c.q)
    q1 = q[:, -1:].contiguous()

    def with_len(l0, l1=700):
        c2 = _case()
        c2.kv_len = np.array([l0, l1], np.int32)
        return kvcache(c2)

    over = with_len(1025)              # kv_len[0] > max_len
    _rejects(lambda: S.spec_verify_attn(over, q, scale=c.scale))
    _rejects(lambda: S.spec_topk_attn(over, q1, 64, scale=c.scale))
    short = with_len(900, 3)           # fewer keys than the 6 query rows
    _rejects(lambda: S.spec_verify_attn(short, q, scale=c.scale))
    kv = kvcache(c)
    _rejects(lambda: S.spec_verify_attn(kv, q, q_len=dev(np.array([0, 6], np.int32)),
                                        scale=c.scale))
    # q_len within bounds is fine
    S.spec_verify_attn(kv, q, q_len=dev(np.array([1, 6], np.int32)), scale=c.scale)
    torch.cuda.synchronize()


def test_bad_text_lists_are_rejected(S):
    c = _case()
    kv = kvcache(c)
    q = dev(c.q)
    idx = c.text_idx.copy()
    idx[0, 0] = c.kv_len[0]            # one past the last position, still < max_len
    _rejects(lambda: S.spec_vata_attn(kv, q, dev(idx), dev(c.text_len), scale=c.scale))
    tl = c.text_len.copy()
    tl[0] = c.text_idx.shape[1] + 1    # longer than the list's row
    _rejects(lambda: S.spec_vata_attn(kv, q, dev(c.text_idx), dev(tl), scale=c.scale))


def test_bad_gamma_is_rejected(S):
    rng = np.random.default_rng(3)
    logits = dev(W.Stored.from_f32(rng.standard_normal((2, 6, 5000)).astype(np.float32), W.BF16))
    draft = dev(rng.integers(0, 5000, size=(2, 5)).astype(np.int32))
    _rejects(lambda: S.spec_accept(logits, draft, dev(np.array([6, 1], np.int32))))
    S.spec_accept(logits, draft, dev(np.array([5, 0], np.int32)))
    torch.cuda.synchronize()


def test_negative_page_is_rejected(S):
    from speculative_decoding_attention_amd import KVCache
    c = _case(page_size=16)
    k, v = dev(c.k), dev(c.v)
    # a spare page in front of the pool, so page -1 is allocated memory
    kf = torch.zeros((k.shape[0] + 1,) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    vf = torch.zeros_like(kf)
    kf[1:] = k
    vf[1:] = v
    pt = c.page_table.copy()
    pt[0, 3] = -1
    kv = KVCache(kf[1:], vf[1:], dev(c.kv_len), page_table=dev(pt), page_size=16,
                 max_len=c.max_len)
    _rejects(lambda: S.spec_verify_attn(kv, dev(c.q), scale=c.scale))


def test_std_and_sparse_lists_are_checked(S):
    """A text list out of order for the prefill selection, and a kept list
    that reaches past the sequence, a list longer than its row, or a tail
    start before the stated bound.  Reached anyway, each would stay inside the
    arrays: the positions are below kv_len and the lengths within the row."""
    c = W.std_small(13, 2, 8, 2, 128, (600, 500), W.BF16, n_text=(12, 8), top_k=32, n=1)
    kv = kvcache_std(c)
    ti = c.text_idx.copy()
    ti[0, 2], ti[0, 3] = ti[0, 3], ti[0, 2]
    _rejects(lambda: S.spec_std_select(kv, dev(c.q_text), dev(ti), dev(c.text_len), 32,
                                       scale=c.scale))
    sel, keep, keep_len, _ = S.spec_std_select(kv, dev(c.q_text), dev(c.text_idx),
                                               dev(c.text_len), 32, scale=c.scale)
    torch.cuda.synchronize()
    lst = np.full((2, 2, 40), -1, np.int32)
    ln = np.full((2, 2), 10, np.int32)
    for b in range(2):
        for g in range(2):
            lst[b, g, :10] = np.arange(100, 110)
    t0 = (c.kv_len - 20).astype(np.int32)
    q = dev(c.q)
    S.spec_sparse_attn(kv, q, dev(lst), dev(ln), tail_start=dev(t0), tail_max=20, scale=c.scale)
    torch.cuda.synchronize()
    inside = lst.copy()
    inside[1, 1, 3] = t0[1]              # inside the tail: allowed, counted once
    S.spec_sparse_attn(kv, q, dev(inside), dev(ln), tail_start=dev(t0), tail_max=20,
                       scale=c.scale)
    torch.cuda.synchronize()
    bad = lst.copy()
    bad[1, 1, 3] = c.kv_len[1]           # past the sequence (row 500 of 600 exists)
    _rejects(lambda: S.spec_sparse_attn(kv, q, dev(bad), dev(ln), tail_start=dev(t0),
                                        tail_max=20, scale=c.scale))
    long = ln.copy()
    long[0, 1] = 41                      # longer than the row of 40
    _rejects(lambda: S.spec_sparse_attn(kv, q, dev(lst), dev(long), tail_start=dev(t0),
                                        tail_max=20, scale=c.scale))
    early = t0.copy()
    early[0] -= 1                        # a 21-position tail with tail_max = 20
    _rejects(lambda: S.spec_sparse_attn(kv, q, dev(lst), dev(ln), tail_start=dev(early),
                                        tail_max=20, scale=c.scale))


def kvcache_std(c):
    from speculative_decoding_attention_amd import KVCache
    return KVCache(dev(c.k), dev(c.v), dev(c.kv_len.astype(np.int32)), max_len=c.max_len)


def test_commit_inputs_are_checked(S):
    """An accepted prefix longer than gamma, a verification length shorter
    than the verified rows, or an output length past its capacity.  Reached
    anyway, the kernel clamps each of them to its range."""
    draft = dev(np.array([[1, 2, 3], [4, 5, 6]], np.int32))
    nxt = dev(np.array([7, 8], np.int32))
    toks = torch.zeros((2, 5), dtype=torch.int32, device="cuda:0")

    def run(acc, kv, tl):
        S.spec_commit(draft, dev(np.array(acc, np.int32)), nxt, dev(np.array(kv, np.int32)),
                      tokens=toks, tok_len=dev(np.array(tl, np.int32)))

    run([1, 3], [10, 12], [0, 2])                 # valid
    torch.cuda.synchronize()
    _rejects(lambda: run([4, 0], [10, 12], [0, 2]))
    _rejects(lambda: run([1, 0], [10, 3], [0, 2]))
    _rejects(lambda: run([1, 0], [10, 12], [0, 6]))
