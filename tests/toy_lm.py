"""A one-layer random-weight language model used only as test scaffolding for
whole speculative-decoding loops.  The projections, embeddings and the LM
head are plain torch fp32 matmuls on the device; every attention call,
acceptance and commit goes through the library's C ABI.  fp32 throughout, so
the dense verification rows and the one-token greedy reference differ only by
summation order (far below any argmax gap the seeds produce).

Token x at position p: h = E[x] + P[p]; q, k, v = h Wq, h Wk, h Wv (per head);
o = attention(q, cache); logits = (h + o Wo) Wlm.
"""
from __future__ import annotations

import torch


class ToyLM:
    def __init__(self, vocab=512, Hq=8, Hkv=2, d=64, max_pos=1024, seed=0, device="cuda:0"):
        g = torch.Generator().manual_seed(seed)
        D = Hq * d
        self.V, self.Hq, self.Hkv, self.d, self.D = vocab, Hq, Hkv, d, D
        self.scale = d ** -0.5
        r = lambda *s: torch.randn(*s, generator=g)
        self.E = r(vocab, D).to(device)
        self.P = (0.5 * r(max_pos, D)).to(device)
        self.Wq = (r(D, Hq * d) / D ** 0.5).to(device)
        self.Wk = (r(D, Hkv * d) / D ** 0.5).to(device)
        self.Wv = (r(D, Hkv * d) / D ** 0.5).to(device)
        self.Wo = (r(Hq * d, D) / (Hq * d) ** 0.5).to(device)
        self.Wlm = (4.0 * r(D, vocab) / D ** 0.5).to(device)

    def embed(self, tok, pos):
        """tok, pos: [B, n] int -> h [B, n, D]."""
        return self.E[tok.long()] + self.P[pos.long()]

    def qkv(self, h):
        B, n, _ = h.shape
        q = (h @ self.Wq).view(B, n, self.Hq, self.d).contiguous()
        k = (h @ self.Wk).view(B, n, self.Hkv, self.d)
        v = (h @ self.Wv).view(B, n, self.Hkv, self.d)
        return q, k, v

    @staticmethod
    def write_kv(K, V, k, v, pos):
        """Cache rows K[b, :, pos[b, i]] <- k[b, i] (device indices, no sync)."""
        bi = torch.arange(K.shape[0], device=K.device).unsqueeze(1).expand_as(pos)
        K[bi, :, pos.long()] = k
        V[bi, :, pos.long()] = v

    def logits(self, h, o):
        B, n = h.shape[:2]
        return (h + o.reshape(B, n, self.Hq * self.d) @ self.Wo) @ self.Wlm
