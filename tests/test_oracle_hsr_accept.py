"""Pins of the HSR-fusion and acceptance oracles, and of the bf16 storage
rounding the input generators use."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W


# ------------------------------------------------------------------ HSR ----

def test_hsr_identity_weights_select_each_half():
    rng = np.random.default_rng(0)
    M, D = 5, 7
    e = rng.standard_normal((M, D))
    h = rng.standard_normal((M, D))
    eye, zero = np.eye(D), np.zeros((D, D))
    assert np.array_equal(oracle.hsr_fuse(e, h, np.concatenate([eye, zero], 1)), e)
    assert np.array_equal(oracle.hsr_fuse(e, h, np.concatenate([zero, eye], 1)), h)


def test_hsr_matches_torch_linear_and_explicit_loops():
    rng = np.random.default_rng(1)
    M, D = 4, 6
    e, h = rng.standard_normal((M, D)), rng.standard_normal((M, D))
    w = rng.standard_normal((D, 2 * D))
    y = oracle.hsr_fuse(e, h, w)
    ref = torch.nn.functional.linear(torch.cat([torch.tensor(e), torch.tensor(h)], 1),
                                     torch.tensor(w)).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12
    assert np.max(np.abs(y - oracle.hsr_fuse_loops(e, h, w))) < 1e-12


def test_hsr_order_is_embedding_then_hidden():
    """Swapping e and h changes the result unless W's halves are equal."""
    rng = np.random.default_rng(2)
    e, h = rng.standard_normal((2, 3)), rng.standard_normal((2, 3))
    w = np.concatenate([np.eye(3), 2 * np.eye(3)], 1)
    assert np.allclose(oracle.hsr_fuse(e, h, w), e + 2 * h)


# --------------------------------------------------------------- accept ----

@pytest.mark.parametrize("seed", range(4))
def test_accept_brute_force_all_drafts(seed):
    """Check (4): for vocab 3 and gamma 3, every one of the 27 drafts against
    logits with planted ties; the expected length is found by trying every
    prefix length, the argmax with torch.argmax (first maximal index)."""
    rng = np.random.default_rng(seed)
    V, gamma = 3, 3
    logits = rng.integers(-2, 3, size=(1, gamma + 1, V)).astype(np.float32)  # many ties
    t_ref = [int(torch.argmax(torch.tensor(logits[0, i]))) for i in range(gamma + 1)]
    for draft in itertools.product(range(V), repeat=gamma):
        d = np.array([draft], np.int32)
        t, n, nxt = oracle.accept(logits, d)
        want_n = max(m for m in range(gamma + 1) if list(draft[:m]) == t_ref[:m])
        assert t[0].tolist() == t_ref
        assert n[0] == want_n and nxt[0] == t_ref[want_n]
        t2, n2, nxt2 = oracle.accept(logits, d, fast=False)
        assert np.array_equal(t, t2) and n2[0] == n[0] and nxt2[0] == nxt[0]


def test_accept_ties_take_lowest_index_and_signed_zero_is_equal():
    logits = np.array([[[0.0, 2.0, 2.0, 1.0], [-0.0, 0.0, -1.0, -3.0]]], np.float32)
    t, n, nxt = oracle.accept(logits, np.array([[1]], np.int32))
    assert t[0].tolist() == [1, 0] and n[0] == 1 and nxt[0] == 0
    t, n, nxt = oracle.accept(logits, np.array([[2]], np.int32), fast=False)
    assert t[0].tolist() == [1, 0] and n[0] == 0 and nxt[0] == 1


def test_accept_all_match_and_first_mismatch():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((2, 5, 50)).astype(np.float32)
    t_ref = logits.argmax(-1)
    draft = np.stack([t_ref[0, :4], t_ref[1, :4]]).astype(np.int32)
    draft[1, 0] = (draft[1, 0] + 1) % 50
    t, n, nxt = oracle.accept(logits, draft)
    assert n.tolist() == [4, 0]
    assert nxt.tolist() == [t_ref[0, 4], t_ref[1, 0]]


def test_accept_per_sequence_gamma():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((2, 6, 20)).astype(np.float32)
    t_ref = logits.argmax(-1)
    draft = t_ref[:, :5].astype(np.int32).copy()
    t, n, nxt = oracle.accept(logits, draft, np.array([2, 5], np.int32))
    assert n.tolist() == [2, 5] and t[0, 3:].tolist() == [-1, -1, -1]
    assert nxt.tolist() == [t_ref[0, 2], t_ref[1, 5]]


def test_c1_planted_acceptance():
    """The tiny workload plants two matching draft tokens then a mismatch."""
    _, acc = W.c1_tiny()
    t, n, nxt = oracle.accept(acc.logits.values, acc.draft, acc.gamma)
    assert n[0] == 2
    assert t[0, :2].tolist() == acc.draft[0, :2].tolist()
    assert t[0, 2] != acc.draft[0, 2] and nxt[0] == t[0, 2]


# ----------------------------------------------------------- bf16 store ----

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                  3.3895313892515355e38], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.tensor(x).to(torch.bfloat16).float().numpy())
