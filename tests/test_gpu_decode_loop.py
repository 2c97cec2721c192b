"""Whole speculative-decoding loops on the GPU with a random-weight toy target
(tests/toy_lm.py): drafting with each sparse attention of the library
(dense self-draft, text-anchored, per-step top-K, Sparse-to-Dense kept lists),
dense verification, greedy acceptance and the device-side commit.  The
pages' lossless claim is the check: the emitted tokens equal the target's
own one-token-at-a-time greedy decode, for every draft.  One variant runs
each round as a captured HIP graph, which proves a round needs no host
synchronisation.  Also: spec_commit against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev
from toy_lm import ToyLM

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_NEW = 40


def test_commit_matches_oracle():
    import speculative_decoding_attention_amd as S
    rng = np.random.default_rng(3)
    B, n_max = 7, 6
    gamma = rng.integers(0, n_max, size=B).astype(np.int32)
    kv_len = (rng.integers(50, 90, size=B) + gamma + 1).astype(np.int32)
    acc = np.array([rng.integers(0, g + 1) for g in gamma], np.int32)
    nxt = rng.integers(0, 1000, size=B).astype(np.int32)
    draft = rng.integers(0, 1000, size=(B, n_max - 1)).astype(np.int32)
    tokens = rng.integers(-5, 0, size=(B, 9)).astype(np.int32)
    tok_len = rng.integers(0, 9, size=B).astype(np.int32)
    text_idx = rng.integers(-5, 0, size=(B, 12)).astype(np.int32)
    text_len = rng.integers(0, 12, size=B).astype(np.int32)
    want = oracle.commit(kv_len, draft, acc, nxt, gamma, tokens, tok_len, text_idx, text_len)
    d_kv, d_tok, d_tl, d_ti, d_tn = dev(kv_len), dev(tokens), dev(tok_len), dev(text_idx), dev(text_len)
    last = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    S.spec_commit(dev(draft), dev(acc), dev(nxt), d_kv, gamma=dev(gamma), last_tok=last,
                  tokens=d_tok, tok_len=d_tl, text_idx=d_ti, text_len=d_tn)
    torch.cuda.synchronize()
    got = (d_kv, last, d_tok, d_tl, d_ti, d_tn)
    for g, w in zip(got, want):
        assert np.array_equal(g.cpu().numpy(), w)


class Loop:
    """Prompt, cache and bookkeeping state for one batch of sequences."""

    def __init__(self, seed, L0=(300, 221), n_text=(24, 17), gamma=4, top_k=64, std_k=48):
        import speculative_decoding_attention_amd as S
        self.S = S
        self.m = ToyLM(seed=seed)
        m = self.m
        rng = np.random.default_rng(seed)
        self.B, self.gamma, self.top_k = len(L0), gamma, top_k
        self.L0 = np.array(L0, np.int32)
        self.max_len = int(self.L0.max()) + (N_NEW + 2) * (gamma + 1)
        B = self.B
        prompt = rng.integers(0, m.V, size=(B, int(self.L0.max()))).astype(np.int32)
        self.prompt = torch.from_numpy(prompt).to(DEV)
        # text positions: trailing n_text, plus 6 spread over the rest
        texts = []
        for b in range(B):
            L = int(self.L0[b])
            inter = np.sort(rng.choice(L - n_text[b], size=6, replace=False))
            texts.append(np.concatenate([inter, np.arange(L - n_text[b], L)]).astype(np.int32))
        self.t_cap = max(len(t) for t in texts) + (N_NEW + 2) * (gamma + 1)
        self.K = torch.zeros((B, m.Hkv, self.max_len, m.d), device=DEV)
        self.V = torch.zeros_like(self.K)
        # prefill: every prompt position's K/V
        pos = torch.arange(prompt.shape[1], device=DEV).unsqueeze(0).expand(B, -1)
        h = m.embed(self.prompt, pos)
        q, k, v = m.qkv(h)
        m.write_kv(self.K, self.V, k, v, pos)
        # prefill selection over the prompt's text tokens (Sparse-to-Dense)
        t_max = max(len(t) for t in texts)
        ti = np.zeros((B, t_max), np.int32)
        tl = np.array([len(t) for t in texts], np.int32)
        for b in range(B):
            ti[b, :tl[b]] = texts[b]
        q_text = torch.stack([q[b, torch.from_numpy(ti[b]).long().to(DEV)] for b in range(B)])
        kv_pref = S.KVCache(self.K, self.V, dev(self.L0), max_len=self.max_len)
        _, self.keep, self.keep_len, _ = S.spec_std_select(kv_pref, q_text.contiguous(), dev(ti),
                                                           dev(tl), std_k, scale=m.scale)
        self.tail_start = dev(self.L0)
        # committed text list for the text-anchored draft: prompt text positions
        # below the last prompt token (whose K/V each round rewrites first)
        self.text_idx = torch.full((B, self.t_cap), -1, dtype=torch.int32, device=DEV)
        self.text_len = torch.zeros(B, dtype=torch.int32, device=DEV)
        for b in range(B):
            keep = texts[b][texts[b] < self.L0[b] - 1]
            self.text_idx[b, :len(keep)] = torch.from_numpy(keep).to(DEV)
            self.text_len[b] = len(keep)
        # decode state: the last prompt token is the first verified row
        self.kv_len = dev(self.L0 - 1)
        self.last_tok = self.prompt[torch.arange(B, device=DEV), self.kv_len.long()].contiguous()
        self.cur_len = self.kv_len.clone()
        self.kv = S.KVCache(self.K, self.V, self.cur_len, max_len=self.max_len)
        self.tokens = torch.full((B, N_NEW + gamma + 1), -1, dtype=torch.int32, device=DEV)
        self.tok_len = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.tl_tmp = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.ar = torch.arange(B, device=DEV)

    def greedy(self, n):
        """The target's own greedy decode, one token per dense call."""
        S, m = self.S, self.m
        kv_len = self.kv_len.clone()
        cur = kv_len.clone()
        kv = S.KVCache(self.K.clone(), self.V.clone(), cur, max_len=self.max_len)
        x = self.last_tok.clone()
        out = []
        for _ in range(n):
            pos = kv_len.unsqueeze(1)
            h = m.embed(x.unsqueeze(1), pos)
            q, k, v = m.qkv(h)
            m.write_kv(kv.k, kv.v, k, v, pos)
            cur.copy_(kv_len + 1)
            o, _ = S.spec_verify_attn(kv, q, scale=m.scale, out_dtype=torch.float32)
            x = m.logits(h, o)[:, 0].argmax(-1).to(torch.int32)
            out.append(x)
            kv_len.copy_(cur)
        return torch.stack(out, 1)

    def draft_attn(self, kind, q, j):
        S, m = self.S, self.m
        if kind == "dense":
            return S.spec_verify_attn(self.kv, q, scale=m.scale, out_dtype=torch.float32)[0]
        if kind == "vata":
            self.text_idx[self.ar, (self.text_len + j).long()] = self.kv_len + j
            self.tl_tmp.copy_(self.text_len + j + 1)
            return S.spec_vata_attn(self.kv, q, self.text_idx, self.tl_tmp, scale=m.scale,
                                    out_dtype=torch.float32)[0]
        if kind == "topk":
            return S.spec_topk_attn(self.kv, q, self.top_k, scale=m.scale,
                                    out_dtype=torch.float32)[1]
        if kind == "std":
            return S.spec_sparse_attn(self.kv, q, self.keep, self.keep_len,
                                      tail_start=self.tail_start,
                                      tail_max=(N_NEW + 2) * (self.gamma + 1) + 1,
                                      scale=m.scale, out_dtype=torch.float32)[0]
        raise ValueError(kind)

    def round(self, kind):
        """One speculative round; returns accept_len (device)."""
        S, m, g = self.S, self.m, self.gamma
        draft = torch.empty((self.B, g), dtype=torch.int32, device=DEV)
        x = self.last_tok
        for j in range(g):
            pos = (self.kv_len + j).unsqueeze(1)
            h = m.embed(x.unsqueeze(1), pos)
            q, k, v = m.qkv(h)
            m.write_kv(self.K, self.V, k, v, pos)
            self.cur_len.copy_(self.kv_len + j + 1)
            o = self.draft_attn(kind, q, j)
            x = m.logits(h, o)[:, 0].argmax(-1).to(torch.int32)
            draft[:, j] = x
        toks = torch.cat([self.last_tok.unsqueeze(1), draft], 1)
        pos = self.kv_len.unsqueeze(1) + torch.arange(g + 1, device=DEV, dtype=torch.int32)
        h = m.embed(toks, pos)
        q, k, v = m.qkv(h)
        m.write_kv(self.K, self.V, k, v, pos)
        self.cur_len.copy_(self.kv_len + g + 1)
        o, _ = S.spec_verify_attn(self.kv, q, scale=m.scale, out_dtype=torch.float32)
        logits = m.logits(h, o).contiguous()
        _, n, nxt = S.spec_accept(logits, draft)
        S.spec_commit(draft, n, nxt, self.cur_len, last_tok=self.last_tok, tokens=self.tokens,
                      tok_len=self.tok_len, text_idx=self.text_idx, text_len=self.text_len)
        self.kv_len.copy_(self.cur_len)
        return n


@pytest.mark.parametrize("kind", ["dense", "vata", "topk", "std"])
@pytest.mark.parametrize("seed", [0, 1])
def test_speculative_loop_is_lossless(kind, seed):
    lp = Loop(seed)
    ref = lp.greedy(N_NEW)
    accepted = []
    for _ in range(N_NEW):
        accepted.append(lp.round(kind))
        if int(lp.tok_len.min().item()) >= N_NEW:
            break
    torch.cuda.synchronize()
    got = lp.tokens[:, :N_NEW]
    assert torch.equal(got, ref), f"{kind}: first mismatch at {(got != ref).nonzero()[:1].tolist()}"
    acc = torch.stack(accepted).cpu().numpy()
    if kind == "dense":
        assert np.all(acc == lp.gamma), "a draft identical to the target must be fully accepted"
    if kind == "topk":
        assert acc.min() < lp.gamma, "the rejection path was not exercised"
    # committed length = prompt + emitted tokens - 1 (the last token's K/V is pending)
    emitted = np.minimum(np.cumsum(acc + 1, axis=0)[-1], 10 ** 9)
    assert np.array_equal(lp.kv_len.cpu().numpy(), lp.L0 - 1 + emitted)


@pytest.mark.parametrize("kind", ["vata", "std"])
def test_graph_captured_rounds_are_lossless(kind):
    """One eager round sizes every workspace; each later round replays one
    captured graph (draft, verification, acceptance, commit) with no host
    synchronisation in between."""
    lp = Loop(5)
    ref = lp.greedy(N_NEW)
    lp.round(kind)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lp.round(kind)
    for _ in range(N_NEW - 1):
        g.replay()
    torch.cuda.synchronize()
    assert int(lp.tok_len.min().item()) >= N_NEW
    assert torch.equal(lp.tokens[:, :N_NEW], ref)
