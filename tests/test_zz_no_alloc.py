"""The allocation-free verification entry point: through the C ABI it must
give exactly the results of spec_verify_attn (same kernels and split plan,
partials in the library's own scratch instead of a caller workspace), on two
calls in a row, the second smaller than the first."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, kvcache

pytestmark = pytest.mark.gpu


def _both(c, out_dtype):
    import speculative_decoding_attention_amd as S
    kv = kvcache(c)
    q = dev(c.q)
    q_len = dev(c.q_len.astype(np.int32))
    ref_o, ref_l = S.spec_verify_attn(kv, q, q_len=q_len, scale=c.scale, out_dtype=out_dtype)
    B, n, Hq, d = c.q.shape
    out = torch.full((B, n, Hq, d), float("nan"), dtype=out_dtype, device=q.device)
    lse = torch.full((B, n, Hq), float("nan"), dtype=torch.float32, device=q.device)
    S.spec_verify_attn_noalloc(kv, q, out, lse, q_len=q_len, scale=c.scale)
    torch.cuda.synchronize()
    return ref_o, ref_l, out, lse


def test_noalloc_matches_verify_on_two_calls_second_smaller():
    big = W.c2_sparrow(0, with_hsr=False)[0]                  # 25,512 positions, 6.5 MB scratch
    small = W.small_attn(81, 3, 8, 2, 128, 5, (1300, 700, 2100), W.BF16, page_size=16,
                         q_len=[5, 3, 4])
    for c, odt in ((big, torch.bfloat16), (small, torch.float32)):
        ro, rl, o, l = _both(c, odt)
        assert torch.equal(o, ro), c.name
        assert torch.equal(l, rl), c.name


def test_noalloc_fp32_head_dim_64():
    c = W.small_attn(82, 2, 4, 2, 64, 3, (900, 333), W.F32)
    ro, rl, o, l = _both(c, torch.float32)
    assert torch.equal(o, ro) and torch.equal(l, rl)
