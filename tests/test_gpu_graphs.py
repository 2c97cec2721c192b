"""Every entry point inside a captured HIP graph: each replay (with eager work
and synchronisation between replays) reproduces the eager result bit for bit.
The library's counters live in the zero-once sync region of the workspace, so
no replay depends on a clearing launch."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, kvcache

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _check_replays(fn, outs, replays=4):
    """fn writes into the tensors `outs`; compare graph replays to eager."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = _capture(fn)
    for r in range(replays):
        for o in outs:
            o.fill_(-7)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), f"replay {r} differs"


def test_attention_entry_points_in_graphs():
    import speculative_decoding_attention_amd as S
    c = W.small_attn(31, 2, 28, 4, 128, 6, (3000, 1700), W.BF16, page_size=16)
    kv = kvcache(c)
    q = dev(c.q)
    B, n, Hq, d = c.q.shape
    ws = S.Workspace()
    o = torch.empty((B, n, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, n, Hq), dtype=torch.float32, device="cuda:0")
    _check_replays(lambda: S.spec_verify_attn(kv, q, scale=c.scale, out=o, lse=lse, workspace=ws),
                   [o, lse])

    idx = np.stack([np.arange(c.kv_len[b] - 300, c.kv_len[b]) for b in range(B)]).astype(np.int32)
    tlen = np.full((B,), 300, np.int32)
    di, dl = dev(idx), dev(tlen)
    _check_replays(lambda: S.spec_vata_attn(kv, q, di, dl, scale=c.scale, out=o, lse=lse,
                                            workspace=ws), [o, lse])

    q1 = q[:, -1:].contiguous()
    sel = torch.empty((B, 4, 256), dtype=torch.int32, device="cuda:0")
    o1 = torch.empty((B, 1, Hq, d), dtype=torch.float32, device="cuda:0")
    l1 = torch.empty((B, 1, Hq), dtype=torch.float32, device="cuda:0")
    _check_replays(lambda: S.spec_topk_attn(kv, q1, 256, scale=c.scale, sel_idx=sel, out=o1,
                                            lse=l1, workspace=ws), [sel, o1, l1])


def test_hsr_and_accept_in_graphs():
    import speculative_decoding_attention_amd as S
    rng = np.random.default_rng(4)
    ws = S.Workspace()
    for m, dm in ((1, 512), (40, 256)):            # small-M stream and split-K MFMA paths
        e = dev(W.Stored.from_f32(rng.standard_normal((m, dm)).astype(np.float32) * 0.02, W.BF16))
        h = dev(W.Stored.from_f32(rng.standard_normal((m, dm)).astype(np.float32) * 0.02, W.BF16))
        w = dev(W.Stored.from_f32(rng.standard_normal((dm, 2 * dm)).astype(np.float32) * 0.02,
                                  W.BF16))
        y = torch.empty((m, dm), dtype=torch.float32, device="cuda:0")
        _check_replays(lambda: S.spec_hsr_fuse(e, h, w, y=y, workspace=ws), [y])

    logits = dev(W.Stored.from_f32(rng.standard_normal((3, 6, 50000)).astype(np.float32),
                                   W.BF16))
    draft = torch.from_numpy(rng.integers(0, 50000, size=(3, 5)).astype(np.int32)).cuda()
    t = torch.empty((3, 6), dtype=torch.int32, device="cuda:0")
    n_acc = torch.empty((3,), dtype=torch.int32, device="cuda:0")
    nxt = torch.empty((3,), dtype=torch.int32, device="cuda:0")
    _check_replays(lambda: S.spec_accept(logits, draft, target_tok=t, accept_len=n_acc,
                                         next_tok=nxt, workspace=ws), [t, n_acc, nxt])


def test_std_select_and_sparse_attention_in_graphs():
    import speculative_decoding_attention_amd as S
    from speculative_decoding_attention_amd import KVCache
    c = W.std_small(3, 2, 8, 2, 128, (700, 700), W.BF16, n_text=(30, 12), top_k=64, n=2)
    kv = KVCache(dev(c.k), dev(c.v), dev(c.kv_len), max_len=c.max_len)
    ws = S.Workspace()
    B, Hkv, K, T = 2, 2, 64, c.t_max
    sel = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda:0")
    keep = torch.empty((B, Hkv, K + T), dtype=torch.int32, device="cuda:0")
    klen = torch.empty((B, Hkv), dtype=torch.int32, device="cuda:0")
    score = torch.empty((B, Hkv, c.max_len), dtype=torch.float32, device="cuda:0")
    qt, ti, tl = dev(c.q_text), dev(c.text_idx), dev(c.text_len)
    _check_replays(lambda: S.spec_std_select(kv, qt, ti, tl, K, scale=c.scale, sel_idx=sel,
                                             keep_idx=keep, keep_len=klen, score=score,
                                             workspace=ws), [sel, keep, klen, score])
    q = dev(c.q)
    o = torch.empty((B, 2, 8, 128), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, 2, 8), dtype=torch.float32, device="cuda:0")
    t0 = dev(c.kv_len - 40)
    _check_replays(lambda: S.spec_sparse_attn(kv, q, keep, klen, tail_start=t0, tail_max=40,
                                              scale=c.scale, out=o, lse=lse, workspace=ws),
                   [o, lse])
    _check_replays(lambda: S.spec_sparse_attn(kv, q, keep, klen, tail_max=32, scale=c.scale,
                                              out=o, lse=lse, workspace=ws), [o, lse])
