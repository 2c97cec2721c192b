"""The measurement hook records its two events around the main kernel of
the next call only, and changes no result."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, kvcache

pytestmark = pytest.mark.gpu


def test_marked_call_times_its_main_kernel_and_computes_the_same():
    import speculative_decoding_attention_amd as S
    c = W.small_attn(3, 2, 28, 4, 128, 6, (9000, 4100), W.BF16)
    kv, q = kvcache(c), dev(c.q)
    ref_o, ref_l = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    S.mark_main_kernel(e0, e1)
    t0.record()
    o, l = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    t1.record()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    main_ms, call_ms = e0.elapsed_time(e1), t0.elapsed_time(t1)
    assert 0.0 < main_ms <= call_ms
    # one-shot: a second call leaves the events where they were
    S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == main_ms


@pytest.mark.parametrize("which", ["topk", "accept", "hsr"])
def test_every_entry_point_marks_its_main_kernel(which):
    import speculative_decoding_attention_amd as S
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d = torch.device("cuda:0")
    if which == "topk":
        c = W.small_attn(5, 1, 8, 2, 128, 1, (3000,), W.BF16)
        S.mark_main_kernel(e0, e1)
        S.spec_topk_attn(kvcache(c), dev(c.q), 256, scale=c.scale)
    elif which == "accept":
        lg = torch.randn(4, 3, 5000, device=d).to(torch.bfloat16)
        S.mark_main_kernel(e0, e1)
        S.spec_accept(lg, torch.zeros(4, 2, dtype=torch.int32, device=d))
    else:
        e = torch.randn(40, 512, device=d).to(torch.bfloat16)
        w = torch.randn(512, 1024, device=d).to(torch.bfloat16)
        S.mark_main_kernel(e0, e1)
        S.spec_hsr_fuse(e, e, w)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) > 0.0


def test_timing_events_bracket_the_main_kernel_inside_the_call():
    """Fence-free timing events work with the hook as torch's events do: the
    main kernel's span is positive and inside the whole call's span."""
    import speculative_decoding_attention_amd as S
    c = W.small_attn(3, 2, 28, 4, 128, 6, (9000, 4100), W.BF16)
    kv, q = kvcache(c), dev(c.q)
    ref_o, ref_l = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    e0, e1, t0, t1 = (S.TimingEvent() for _ in range(4))
    S.mark_main_kernel(t0, t1)                 # the whole call: two hooks in a row
    S.mark_main_kernel(e0, e1)                 # the later hook wins
    o, l = S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    assert e0.elapsed_ms(e1) > 0.0
    # bracket a whole call with a pair recorded through torch's own events
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    S.mark_main_kernel(t0, t1)
    w0.record()
    S.spec_verify_attn(kv, q, scale=c.scale, out_dtype=torch.float32)
    w1.record()
    torch.cuda.synchronize()
    assert 0.0 < t0.elapsed_ms(t1) <= w0.elapsed_time(w1)


@pytest.mark.parametrize("words", [4, 4 * 12345, 13_107_200])
def test_read_probe_reads_every_word_once(words):
    import speculative_decoding_attention_amd as S
    g = torch.Generator().manual_seed(words)
    x = torch.randint(-2**31, 2**31 - 1, (words,), dtype=torch.int32, generator=g)
    sink = S.read_probe(x.to("cuda:0"))
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(x.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want

