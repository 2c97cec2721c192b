"""GPU parity of the HSR fusion GEMM (tolerance) and greedy acceptance
(bit-exact), including the full HSR draft step: HSR output -> text-anchored
attention."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev

pytestmark = pytest.mark.gpu


def _hsr(case, out_dtype):
    import speculative_decoding_attention_amd as S
    y = S.spec_hsr_fuse(dev(case.e), dev(case.h), dev(case.w), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def _hsr_check(case, y):
    ref = oracle.hsr_fuse(case.e.values, case.h.values, case.w.values)
    yy = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(yy - ref).max()
    bound = 2e-3 if y.dtype == torch.bfloat16 else 1e-4
    assert err <= bound, f"HSR max err {err}"
    assert err <= 2e-2
    return ref


@pytest.mark.parametrize("m,d", [(1, 256), (2, 128), (5, 128), (16, 64), (17, 192), (40, 256),
                                 (64, 128), (65, 128), (77, 384), (130, 64), (200, 512),
                                 # 257..320 rows: one tile spans every row
                                 (257, 192), (300, 128), (320, 64), (320, 512), (290, 1024)])
def test_hsr_small(m, d):
    rng = np.random.default_rng(m * 1000 + d)
    case = W.HsrCase("small",
                     W.Stored.from_f32(rng.standard_normal((m, d)).astype(np.float32) * 0.02, W.BF16),
                     W.Stored.from_f32(rng.standard_normal((m, d)).astype(np.float32) * 0.02, W.BF16),
                     W.Stored.from_f32(rng.standard_normal((d, 2 * d)).astype(np.float32) * 0.02,
                                       W.BF16))
    _hsr_check(case, _hsr(case, torch.float32))
    _hsr_check(case, _hsr(case, torch.bfloat16))


def test_hsr_identity_halves():
    d, m = 128, 20
    rng = np.random.default_rng(3)
    e = rng.standard_normal((m, d)).astype(np.float32)
    h = rng.standard_normal((m, d)).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    z = np.zeros_like(eye)
    for wmat, want in ((np.concatenate([eye, z], 1), e), (np.concatenate([z, eye], 1), h)):
        case = W.HsrCase("id", W.Stored.from_f32(e, W.BF16), W.Stored.from_f32(h, W.BF16),
                         W.Stored.from_f32(wmat, W.BF16))
        y = _hsr(case, torch.float32).cpu().numpy()
        assert np.array_equal(y, W.Stored.from_f32(want, W.BF16).values)


def test_c2_hsr_draft_rows():
    """The 25k-token step's HSR inputs, one row per draft step (M = 1) and all
    five rows at once."""
    _, hsr, _ = W.c2_sparrow(0)
    _hsr_check(hsr, _hsr(hsr, torch.float32))
    for k in range(hsr.e.shape[0]):
        one = W.HsrCase("row", W.Stored(W.BF16, hsr.e.bits[k:k + 1].copy()),
                        W.Stored(W.BF16, hsr.h.bits[k:k + 1].copy()), hsr.w)
        _hsr_check(one, _hsr(one, torch.bfloat16))


@pytest.fixture(scope="module")
def c5():
    return W.c5_hsr_accept(0)


def test_c5_hsr_then_vata(c5):
    """The full HSR draft step: Y = FC([e;h]) in bf16 becomes the draft
    queries of text-anchored attention over 2048 text positions."""
    import speculative_decoding_attention_amd as S
    from speculative_decoding_attention_amd import KVCache
    hsr = c5["hsr"]
    y = _hsr(hsr, torch.bfloat16)
    _hsr_check(hsr, y)
    ybits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    c = W.c5_attn_case(c5["kv"], ybits)
    kv = KVCache(dev(c.k), dev(c.v), dev(c.kv_len))
    out, lse = S.spec_vata_attn(kv, y.view(64, 5, 28, 128), dev(c.text_idx), dev(c.text_len),
                                q_len=dev(c.q_len), scale=c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.vata_attention(c.q.values, c.k.values, c.v.values, c.kv_len, c.q_len,
                                   c.text_idx, c.text_len, c.num_kv_heads, c.scale)
    assert_attention_close(out, lse, ro, rl, c.q_len, W.BF16, "c5 vata")


def _accept(case):
    import speculative_decoding_attention_amd as S
    t, n, nxt = S.spec_accept(dev(case.logits), dev(case.draft), dev(case.gamma))
    torch.cuda.synchronize()
    return t.cpu().numpy(), n.cpu().numpy(), nxt.cpu().numpy()


def test_c5_accept_bit_exact(c5):
    case = c5["accept"]
    t, n, nxt = _accept(case)
    rt, rn, rnx = oracle.accept(case.logits.values, case.draft, case.gamma)
    assert np.array_equal(t, rt) and np.array_equal(n, rn) and np.array_equal(nxt, rnx)
    # repeated calls reuse the workspace (counters must come back to zero)
    t2, n2, nxt2 = _accept(case)
    assert np.array_equal(t2, rt) and np.array_equal(n2, rn) and np.array_equal(nxt2, rnx)


def test_c1_accept_planted():
    _, case = W.c1_tiny()
    t, n, nxt = _accept(case)
    rt, rn, rnx = oracle.accept(case.logits.values, case.draft, case.gamma)
    assert n[0] == 2 and np.array_equal(t, rt) and nxt[0] == rnx[0]


@pytest.mark.parametrize("B", [9, 16, 8])
@pytest.mark.parametrize("V,dt", [(1000, W.F32), (1003, W.BF16), (7, W.F32), (50001, W.BF16)])
def test_accept_ragged_gamma_and_ties(V, dt, B):
    rng = np.random.default_rng(V + B)
    n_max = 6
    logits = rng.integers(-3, 4, size=(B, n_max, V)).astype(np.float32)   # heavy ties
    logits[0, 1, :] = 0.0
    logits[0, 1, 5 % V] = -0.0
    t_ref = logits.argmax(-1)
    draft = rng.integers(0, V, size=(B, n_max - 1)).astype(np.int32)
    for b in range(B):
        m = b % n_max
        draft[b, :m] = t_ref[b, :m]
    gamma = np.resize(np.array([5, 0, 1, 2, 3, 4, 5, 5, 3], np.int32), B)
    case = W.AcceptCase("ragged", W.Stored.from_f32(logits, dt), draft, gamma)
    t, n, nxt = _accept(case)
    rt, rn, rnx = oracle.accept(case.logits.values, case.draft, case.gamma)
    assert np.array_equal(t, rt) and np.array_equal(n, rn) and np.array_equal(nxt, rnx)


# vocabularies at and just past one chunk (4,096 bf16 or 2,048 fp32 logits per
# 256-thread chunk): one full chunk, a one-element tail chunk, and a
# vectorised tail chunk of one 16-byte word
@pytest.mark.parametrize("V,dt", [(4096, W.BF16), (4097, W.BF16), (4104, W.BF16),
                                  (2048, W.F32), (2049, W.F32), (2052, W.F32)])
def test_accept_chunk_boundaries(V, dt):
    rng = np.random.default_rng(V)
    B, n_max = 3, 4
    logits = rng.standard_normal((B, n_max, V)).astype(np.float32)
    logits[:, :, V - 1] = 9.0                      # the maximum in the last element
    logits[1, 2, V - 1] = 0.0
    logits[1, 2, 0] = 9.0                          # the maximum in the first element
    draft = np.full((B, n_max - 1), V - 1, np.int32)
    draft[2, 1] = 0
    case = W.AcceptCase("chunk", W.Stored.from_f32(logits, dt), draft, np.full(B, n_max - 1, np.int32))
    t, n, nxt = _accept(case)
    rt, rn, rnx = oracle.accept(case.logits.values, case.draft, case.gamma)
    assert np.array_equal(t, rt) and np.array_equal(n, rn) and np.array_equal(nxt, rnx)


def test_accept_batches_in_turn():
    """Calls of several batch sizes in a row on one workspace, vectorised and
    scalar vocabularies, ragged gamma."""
    rng = np.random.default_rng(11)
    for B in (64, 8, 9, 24, 64):
        V = 32000 + B
        logits = rng.standard_normal((B, 4, V)).astype(np.float32)
        t_ref = logits.argmax(-1)
        draft = t_ref[:, :3].astype(np.int32).copy()
        draft[::3, 1] = (draft[::3, 1] + 1) % V
        gamma = rng.integers(0, 4, size=B).astype(np.int32)
        case = W.AcceptCase("turns", W.Stored.from_f32(logits, W.BF16), draft, gamma)
        t, n, nxt = _accept(case)
        rt, rn, rnx = oracle.accept(case.logits.values, case.draft, case.gamma)
        assert np.array_equal(t, rt) and np.array_equal(n, rn) and np.array_equal(nxt, rnx), B


def test_accept_single_row_no_draft():
    import speculative_decoding_attention_amd as S
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((3, 1, 333)).astype(np.float32)
    t, n, nxt = S.spec_accept(dev(logits), torch.zeros((3, 0), dtype=torch.int32, device="cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy()[:, 0], logits[:, 0].argmax(-1))
    assert np.all(n.cpu().numpy() == 0)
