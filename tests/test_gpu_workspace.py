"""The workspace contract on the device: one zero-filled workspace shared by
every entry point, in any order and with changing shapes, gives the same
results as fresh workspaces, and its synchronisation region is all zero
again after each call."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, kvcache

pytestmark = pytest.mark.gpu


def _sync_region_is_zero(ws):
    import speculative_decoding_attention_amd as S
    torch.cuda.synchronize()
    head = ws.buf[:S.SPEC_WS_SYNC_BYTES]
    return int(torch.count_nonzero(head).item()) == 0


def test_shared_workspace_all_entry_points():
    import speculative_decoding_attention_amd as S
    c, hsr, acc = W.c2_sparrow(0)
    kv = kvcache(c)
    q = dev(c.q)
    q1 = q[:, -1:].contiguous()      # the draft row
    ws = S.Workspace()

    def verify():
        return S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32, workspace=ws)

    def vata1():
        return S.spec_vata_attn(kv, q1, dev(c.text_idx), dev(c.text_len),
                                scale=c.scale, out_dtype=torch.float32, workspace=ws)

    def topk():
        return S.spec_topk_attn(kv, q1, c.top_k, scale=c.scale, out_dtype=torch.float32,
                                workspace=ws)

    def fuse(m):
        return S.spec_hsr_fuse(dev(W.Stored(W.BF16, hsr.e.bits[:m].copy())),
                               dev(W.Stored(W.BF16, hsr.h.bits[:m].copy())), dev(hsr.w),
                               out_dtype=torch.float32, workspace=ws)

    def accept():
        return S.spec_accept(dev(acc.logits), dev(acc.draft), dev(acc.gamma), workspace=ws)

    # fresh-workspace results first
    ref = {"verify": S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32,
                                        workspace=S.Workspace()),
           "vata1": S.spec_vata_attn(kv, q1, dev(c.text_idx),
                                     dev(c.text_len), scale=c.scale, out_dtype=torch.float32,
                                     workspace=S.Workspace()),
           "topk": S.spec_topk_attn(kv, q1, c.top_k, scale=c.scale, out_dtype=torch.float32,
                                    workspace=S.Workspace()),
           "accept": S.spec_accept(dev(acc.logits), dev(acc.draft), dev(acc.gamma),
                                   workspace=S.Workspace())}
    torch.cuda.synchronize()
    # a split-K fusion case with a workspace of its own (40 rows, d = 256)
    rng = np.random.default_rng(5)
    e40 = W.Stored.from_f32(rng.standard_normal((40, 256)).astype(np.float32) * 0.02, W.BF16)
    h40 = W.Stored.from_f32(rng.standard_normal((40, 256)).astype(np.float32) * 0.02, W.BF16)
    w40 = W.Stored.from_f32(rng.standard_normal((256, 512)).astype(np.float32) * 0.02, W.BF16)
    y40_ref = oracle.hsr_fuse(e40.values, h40.values, w40.values)

    order = ["topk", "verify", "accept", "vata1", "hsr40", "verify", "hsr1", "topk", "accept",
             "vata1", "verify"]
    for name in order:
        if name == "hsr40":
            y = S.spec_hsr_fuse(dev(e40), dev(h40), dev(w40), out_dtype=torch.float32,
                                workspace=ws)
            torch.cuda.synchronize()
            assert np.abs(y.cpu().numpy() - y40_ref).max() <= 1e-4
        elif name == "hsr1":
            y = fuse(1)
            torch.cuda.synchronize()
            ry = oracle.hsr_fuse(hsr.e.values[:1], hsr.h.values[:1], hsr.w.values)
            assert np.abs(y.cpu().numpy() - ry).max() <= 1e-4
        else:
            got = {"verify": verify, "vata1": vata1, "topk": topk, "accept": accept}[name]()
            torch.cuda.synchronize()
            for x, r in zip(got, ref[name]):
                assert torch.equal(x, r), name
        assert _sync_region_is_zero(ws), f"sync region dirty after {name}"
