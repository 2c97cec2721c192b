"""Pins of the commit bookkeeping: a hand-worked round, capacity saturation,
and the lossless invariant of the whole greedy loop -- speculative decoding
with any draft emits exactly the target's own greedy sequence -- run with the
oracle's accept and commit on a table-driven toy target."""
import numpy as np
import pytest

import oracle


def test_one_round_by_hand():
    # cache held 10 positions during verification, gamma = 3: the last
    # committed token sits at C = 6, drafts at 7, 8, 9; two drafts accepted
    kv, last, toks, tl, ti, tn = oracle.commit(
        kv_len=[10], draft=[[11, 12, 13]], accept_len=[2], next_tok=[99],
        tokens=np.full((1, 8), -1), tok_len=[1], text_idx=np.full((1, 6), -1), text_len=[2])
    assert kv.tolist() == [9]                      # rows 6, 7, 8 stay
    assert last.tolist() == [99]
    assert toks[0].tolist() == [-1, 11, 12, 99, -1, -1, -1, -1] and tl.tolist() == [4]
    assert ti[0].tolist() == [-1, -1, 6, 7, 8, -1] and tn.tolist() == [5]


def test_rejection_at_the_first_draft_and_per_sequence_gamma():
    kv, last, toks, tl, ti, tn = oracle.commit(
        kv_len=[20, 7], draft=[[1, 2, 3, 4], [5, 6, 7, 8]], accept_len=[0, 2], next_tok=[40, 41],
        gamma=[4, 2], tokens=np.zeros((2, 4), int), tok_len=[0, 3],
        text_idx=np.zeros((2, 3), int), text_len=[0, 2])
    assert kv.tolist() == [16, 7]                  # b=0: C=15, n=0; b=1: C=4, n=2
    assert toks[0, :1].tolist() == [40] and tl.tolist() == [1, 4]   # b=1 saturates at 4
    assert toks[1, 3] == 5
    assert ti[0, :1].tolist() == [15] and tn.tolist() == [1, 3]
    assert ti[1, 2] == 4


def _toy(V, seed):
    rng = np.random.default_rng(seed)
    table = rng.integers(0, V, size=(V, V))          # target: next = table[prev2, prev1]
    dtable = np.where(rng.random((V, V)) < 0.6, table, rng.integers(0, V, size=(V, V)))
    return table, dtable


def _logits_for(ctx_rows, table, V, rng):
    """Rows whose unique argmax is the table's next token, over noise."""
    out = rng.standard_normal((len(ctx_rows), V))
    for i, ctx in enumerate(ctx_rows):
        out[i, table[ctx[-2], ctx[-1]]] = 10.0
    return out


@pytest.mark.parametrize("gamma", [1, 3, 6])
@pytest.mark.parametrize("seed", range(3))
def test_speculative_loop_is_lossless(gamma, seed):
    V, N = 13, 60
    table, dtable = _toy(V, seed)
    rng = np.random.default_rng(100 + seed)
    prompt = [int(x) for x in rng.integers(0, V, size=5)]
    greedy = list(prompt)
    while len(greedy) < len(prompt) + N:
        greedy.append(int(table[greedy[-2], greedy[-1]]))

    ctx = list(prompt)
    kv_len = np.array([len(ctx) - 1], np.int32)    # the last token's K/V is not written yet
    tokens = np.full((1, N + gamma + 2), -1, np.int32)
    tok_len = np.zeros(1, np.int32)
    rounds = 0
    while tok_len[0] < N:
        d = []
        for _ in range(gamma):
            c = ctx + d
            d.append(int(dtable[c[-2], c[-1]]))
        rows = [ctx + d[:i] for i in range(gamma + 1)]
        logits = _logits_for(rows, table, V, rng)[None]
        t, n, nxt = oracle.accept(logits, np.array([d], np.int32))
        verify_len = kv_len + gamma + 1               # rows C..C+gamma written by verification
        kv_len, last, tokens, tok_len, _, _ = oracle.commit(verify_len, np.array([d]), n, nxt,
                                                            tokens=tokens, tok_len=tok_len)
        ctx = ctx + d[:int(n[0])] + [int(nxt[0])]
        assert kv_len[0] == len(ctx) - 1 and last[0] == ctx[-1]
        rounds += 1
    assert tokens[0, :N].tolist() == greedy[len(prompt):len(prompt) + N]
    assert rounds <= N                                # at least one token per round
