"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This module holds no arithmetic of the method itself: it only draws random
numbers, rounds them to their storage dtype, and lays them out (contiguous or
paged KV, index lists, planted argmaxes).  Both the CPU oracle and the HIP
path consume exactly what is produced here.

Draw order per workload (one ``numpy.random.default_rng(seed)`` each):
lengths -> gamma -> page permutation -> Q -> K -> V -> text layout ->
HSR inputs -> logits -> draft tokens.

Shapes follow the workloads the pages measure on: tens of thousands of visual
tokens (Sparrow explainer, technical summary "5. Results": 25k visual tokens),
7B-class targets with 28 query / 4 KV heads of dim 128 and hidden size 3584,
a ~2k-token draft context (Sparrow pt explainer, "1. O Problema"), draft
lengths gamma of 3..9 (Sparse-to-Dense pt explainer, "Resultados
Experimentais", hyper-parameters).  No benchmark item is reproduced: all
values are synthetic normals.
"""
from __future__ import annotations

import dataclasses
from typing import NamedTuple, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# storage helpers
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Stored:
    """A tensor in its storage dtype.

    ``bits`` is uint16 for bf16 and float32 for f32; ``values`` is the exact
    float32 value of every element (what both sides compute on).
    """

    dtype: str
    bits: np.ndarray

    @property
    def values(self) -> np.ndarray:
        if self.dtype == BF16:
            return bf16_bits_to_f32(self.bits)
        return self.bits

    @property
    def shape(self):
        return self.bits.shape

    @staticmethod
    def from_f32(x: np.ndarray, dtype: str) -> "Stored":
        x = np.ascontiguousarray(x, dtype=np.float32)
        if dtype == BF16:
            return Stored(BF16, f32_to_bf16_bits(x))
        if dtype == F32:
            return Stored(F32, x)
        raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


# --------------------------------------------------------------------------
# workload records
# --------------------------------------------------------------------------

@dataclasses.dataclass
class AttnCase:
    """Inputs for verify / VATA / top-K attention.

    K/V are either contiguous ``[B, Hkv, L_max, d]`` (page_size == 0) or a
    paged pool ``[P, Hkv, page_size, d]`` with ``page_table [B, max_pages]``.
    ``q`` is ``[B, n_max, Hq, d]``; ``q_len[b]`` rows are real, the rest pad.
    Query row i of sequence b sits at absolute position kv_len[b]-q_len[b]+i.
    """

    name: str
    dtype: str
    q: Stored
    k: Stored
    v: Stored
    kv_len: np.ndarray
    q_len: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_len: int
    page_size: int = 0
    page_table: Optional[np.ndarray] = None
    text_idx: Optional[np.ndarray] = None
    text_len: Optional[np.ndarray] = None
    top_k: int = 0

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_max(self) -> int:
        return int(self.q.shape[1])

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))


@dataclasses.dataclass
class HsrCase:
    name: str
    e: Stored      # [M, D]
    h: Stored      # [M, D]
    w: Stored      # [D, 2D]  (output-major)


@dataclasses.dataclass
class AcceptCase:
    name: str
    logits: Stored          # [B, n_max, V]
    draft: np.ndarray       # [B, n_max-1] int32
    gamma: np.ndarray       # [B] int32
    planted_len: Optional[np.ndarray] = None


@dataclasses.dataclass
class StdCase:
    """Inputs for Sparse-to-Dense prefill selection and its sparse decode.

    ``q_text [B, t_max, Hq, d]``: row t is the prefill query of the text token
    at ``text_idx[b, t]`` (ascending, distinct, t < text_len[b]).  K/V are laid
    out as in AttnCase.  ``q [B, n, Hq, d]`` are draft query rows for the
    decode that follows (row i at position kv_len[b] - q_len[b] + i).
    """

    name: str
    dtype: str
    q_text: Stored
    k: Stored
    v: Stored
    q: Stored
    kv_len: np.ndarray
    q_len: np.ndarray
    text_idx: np.ndarray
    text_len: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_len: int
    top_k: int = 0
    page_size: int = 0
    page_table: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return int(self.q_text.shape[0])

    @property
    def t_max(self) -> int:
        return int(self.q_text.shape[1])

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def c1_tiny(seed: int = 0):
    """Tiny single-layer step, fp32: B=1, 2 query / 1 KV head, d=64,
    512 visual + 64 text positions, gamma=4 (5 verify rows), vocab 1000.
    Acceptance logits have draft tokens 0 and 1 planted as row argmaxes and
    draft token 2 planted as a mismatch."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, Lvis, Ltxt, gamma, V = 1, 2, 1, 64, 512, 64, 4, 1000
    L = Lvis + Ltxt
    n = gamma + 1
    q = _normal(rng, (B, n, Hq, d))
    k = _normal(rng, (B, Hkv, L, d))
    v = _normal(rng, (B, Hkv, L, d))
    text_idx = np.arange(Lvis, L, dtype=np.int32)[None, :]
    logits = _normal(rng, (B, n, V))
    draft = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    # plant: rows 0 and 1 take the draft token as a strict maximum
    for i in range(2):
        logits[0, i, draft[0, i]] = logits[0, i].max() + np.float32(1.0)
    # row 2: a strict maximum at a drawn column; the draft token is the next
    # column, so it misses
    col2 = int(rng.integers(0, V))
    logits[0, 2, col2] = logits[0, 2].max() + np.float32(1.0)
    draft[0, 2] = (col2 + 1) % V
    attn = AttnCase(
        name="c1", dtype=F32,
        q=Stored.from_f32(q, F32), k=Stored.from_f32(k, F32), v=Stored.from_f32(v, F32),
        kv_len=np.array([L], np.int32), q_len=np.array([n], np.int32),
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=L,
        text_idx=text_idx, text_len=np.array([Ltxt], np.int32))
    acc = AcceptCase(name="c1", logits=Stored.from_f32(logits, F32), draft=draft,
                     gamma=np.array([gamma], np.int32),
                     planted_len=np.array([2], np.int32))
    return attn, acc


def c2_text_layout(Lvis: int = 25000, Ltxt: int = 512, n_interleaved: int = 64) -> np.ndarray:
    """Text positions of the 25k-visual-token step: ``n_interleaved`` prompt
    positions spread evenly over the first Lvis + n_interleaved slots, then
    the trailing Ltxt - n_interleaved positions."""
    span = Lvis + n_interleaved
    inter = (np.arange(n_interleaved, dtype=np.int64) * span) // n_interleaved
    trail = np.arange(span, Lvis + Ltxt, dtype=np.int64)
    return np.concatenate([inter, trail]).astype(np.int32)


def c2_sparrow(seed: int = 0, Lvis: int = 25000, with_hsr: bool = True):
    """Sparrow-scale step, bf16: B=1, 28/4 heads, d=128, Lvis visual + 512
    text positions (64 interleaved + 448 trailing), gamma=5.  Also returns
    HSR inputs (one row of hidden size 3584 per draft step) and bf16
    acceptance logits (vocab 152064) so that one speculative iteration can
    run on it end to end."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, Ltxt, gamma = 1, 28, 4, 128, 512, 5
    L = Lvis + Ltxt
    n = gamma + 1
    q = _normal(rng, (B, n, Hq, d))
    k = _normal(rng, (B, Hkv, L, d), 0.5)
    v = _normal(rng, (B, Hkv, L, d), 0.5)
    text_idx = c2_text_layout(Lvis, Ltxt)[None, :]
    attn = AttnCase(
        name=f"c2_lvis{Lvis}", dtype=BF16,
        q=Stored.from_f32(q, BF16), k=Stored.from_f32(k, BF16), v=Stored.from_f32(v, BF16),
        kv_len=np.array([L], np.int32), q_len=np.array([n], np.int32),
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=L,
        text_idx=text_idx, text_len=np.array([Ltxt], np.int32), top_k=2048)
    if not with_hsr:
        return attn, None, None
    D, V = Hq * d, 152064
    e = _normal(rng, (gamma, D), 0.02)      # one (e_t, h_{t-1}) row per draft step
    h = _normal(rng, (gamma, D), 0.02)
    w = _normal(rng, (D, 2 * D), 0.02)
    hsr = HsrCase("c2_hsr", Stored.from_f32(e, BF16), Stored.from_f32(h, BF16),
                  Stored.from_f32(w, BF16))
    logits = _normal(rng, (B, n, V))
    draft = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    acc = AcceptCase("c2_accept", Stored.from_f32(logits, BF16), draft,
                     np.array([gamma], np.int32))
    return attn, hsr, acc


class C3Layout(NamedTuple):
    lvis: np.ndarray
    ltxt: np.ndarray
    gamma: np.ndarray
    L: np.ndarray          # int32 kv lengths
    pages: int             # pool size
    page_table: np.ndarray


def _c3_layout(rng: np.random.Generator, B: int, ps: int = 16) -> C3Layout:
    """Lengths, gammas and page table of the ragged batch (the first draws)."""
    lvis = rng.integers(8000, 25001, size=B)
    ltxt = rng.integers(256, 1025, size=B)
    gam = rng.integers(3, 8, size=B)
    L = (lvis + ltxt).astype(np.int32)
    npg = (L + ps - 1) // ps
    P = int(npg.sum())
    perm = rng.permutation(P).astype(np.int32)
    page_table = np.zeros((B, int(npg.max())), np.int32)
    off = 0
    for b in range(B):
        page_table[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    return C3Layout(lvis, ltxt, gam, L, P, page_table)


def c3_layout(seed: int = 0, batch: int = 16) -> C3Layout:
    """The ragged batch's layout alone (no Q/K/V draws)."""
    return _c3_layout(np.random.default_rng(seed), batch)


def c3_ragged_paged(seed: int = 0, batch: int = 16):
    """Ragged paged batch, bf16: per sequence Lvis ~ U[8000, 25000], Ltxt ~
    U[256, 1024], gamma ~ U{3..7}; 16-token pages in a random pool order.
    Text positions are each sequence's trailing Ltxt."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, ps = batch, 28, 4, 128, 16
    lay = _c3_layout(rng, B, ps)
    lvis, ltxt, gam, L, P, page_table = lay
    n_max = 8                      # gamma <= 7, so blocks are padded to 8 rows
    q = _normal(rng, (B, n_max, Hq, d))
    k = _normal(rng, (P, Hkv, ps, d), 0.5)
    v = _normal(rng, (P, Hkv, ps, d), 0.5)
    t_max = int(ltxt.max())
    text_idx = np.zeros((B, t_max), np.int32)
    for b in range(B):
        text_idx[b, :ltxt[b]] = np.arange(lvis[b], L[b], dtype=np.int32)
    return AttnCase(
        name="c3", dtype=BF16,
        q=Stored.from_f32(q, BF16), k=Stored.from_f32(k, BF16), v=Stored.from_f32(v, BF16),
        kv_len=L, q_len=(gam + 1).astype(np.int32),
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=int(L.max()),
        page_size=ps, page_table=page_table,
        text_idx=text_idx, text_len=ltxt.astype(np.int32))


def c4_topk(seed: int = 0, batch: int = 4, L: int = 32768, top_k: int = 2048):
    """Top-K sparse draft + dense verify, bf16: B=4, 28/4 heads, d=128,
    L = 32768 (28672 visual + 4096 text), K = 2048, gamma = 5.  The top-K
    draft query is the last of the 6 verify rows (position L-1)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, gamma = batch, 28, 4, 128, 5
    n = gamma + 1
    q = _normal(rng, (B, n, Hq, d))
    k = _normal(rng, (B, Hkv, L, d), 0.5)
    v = _normal(rng, (B, Hkv, L, d), 0.5)
    return AttnCase(
        name="c4", dtype=BF16,
        q=Stored.from_f32(q, BF16), k=Stored.from_f32(k, BF16), v=Stored.from_f32(v, BF16),
        kv_len=np.full(B, L, np.int32), q_len=np.full(B, n, np.int32),
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=L, top_k=top_k)


def c5_hsr_accept(seed: int = 0, batch: int = 64, vocab: int = 152064, Ltxt: int = 2048,
                  with_kv: bool = True, with_logits: bool = True):
    """HSR draft step + acceptance, bf16: E, H [64*5, 3584] ~ N(0,1)*0.02,
    W [3584, 7168] ~ N(0,1)*0.02; text-anchored attention over Ltxt = 2048
    (identity index list, 28/4 heads, d=128, 5 query rows whose Q is the HSR
    output); acceptance over logits [64, 6, vocab].

    Acceptance planting: per sequence a target length n_b ~ U{0..5}; rows
    i <= n_b get a strict maximum at a chosen column; draft[i] equals that
    column for i < n_b and differs from it at i = n_b.  About one row in eight
    also gets a second column set to the same maximum (a planted tie)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, gamma = batch, 28, 4, 128, 5
    D = Hq * d
    M = B * gamma
    n = gamma + 1
    out = {}
    if with_kv:
        k = _normal(rng, (B, Hkv, Ltxt, d), 0.5)
        v = _normal(rng, (B, Hkv, Ltxt, d), 0.5)
    e = _normal(rng, (M, D), 0.02)
    h = _normal(rng, (M, D), 0.02)
    w = _normal(rng, (D, 2 * D), 0.02)
    out["hsr"] = HsrCase("c5_hsr", Stored.from_f32(e, BF16), Stored.from_f32(h, BF16),
                         Stored.from_f32(w, BF16))
    if with_kv:
        out["kv"] = dict(k=Stored.from_f32(k, BF16), v=Stored.from_f32(v, BF16),
                         kv_len=np.full(B, Ltxt, np.int32), q_len=np.full(B, gamma, np.int32),
                         text_idx=np.tile(np.arange(Ltxt, dtype=np.int32), (B, 1)),
                         text_len=np.full(B, Ltxt, np.int32),
                         num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=Ltxt)
    if with_logits:
        logits = _normal(rng, (B, n, vocab))
        draft = rng.integers(0, vocab, size=(B, gamma)).astype(np.int32)
        plant = rng.integers(0, gamma + 1, size=B).astype(np.int32)
        cols = rng.integers(0, vocab, size=(B, n))
        tie_row = rng.random(size=(B, n)) < 0.125
        tie_col = rng.integers(0, vocab, size=(B, n))
        for b in range(B):
            for i in range(n):
                if i <= plant[b]:
                    top = logits[b, i].max() + np.float32(1.0)
                    logits[b, i, cols[b, i]] = top
                    if tie_row[b, i] and tie_col[b, i] != cols[b, i]:
                        logits[b, i, tie_col[b, i]] = top
                if i < plant[b]:
                    draft[b, i] = cols[b, i]
                elif i == plant[b] and i < gamma:
                    draft[b, i] = (cols[b, i] + 1 + rng.integers(0, vocab - 1)) % vocab
        out["accept"] = AcceptCase("c5_accept", Stored.from_f32(logits, BF16), draft,
                                   np.full(B, gamma, np.int32), planted_len=plant)
    return out


def c5_attn_case(kv: dict, q_bits_bf16: np.ndarray, batch: int = 64, gamma: int = 5) -> AttnCase:
    """Text-anchored attention case of the HSR step: Q is the HSR output
    (bf16 bits, [M, 3584]) viewed as [B, gamma, 28, 128]."""
    q = Stored(BF16, np.ascontiguousarray(q_bits_bf16).reshape(batch, gamma, 28, 128))
    return AttnCase(name="c5_vata", dtype=BF16, q=q, k=kv["k"], v=kv["v"],
                    kv_len=kv["kv_len"], q_len=kv["q_len"], num_q_heads=kv["num_q_heads"],
                    num_kv_heads=kv["num_kv_heads"], head_dim=kv["head_dim"],
                    max_len=kv["max_len"], text_idx=kv["text_idx"], text_len=kv["text_len"])


def small_attn(seed: int, B: int, Hq: int, Hkv: int, d: int, n: int, L, dtype: str,
               page_size: int = 0, kv_scale: float = 0.5, max_len: Optional[int] = None,
               q_len=None, text_frac: float = 0.25) -> AttnCase:
    """Random attention case at test sizes: ragged lengths, optional paging,
    a sorted text-position list per sequence that always includes the query
    rows' own positions (the trailing ones)."""
    rng = np.random.default_rng(seed)
    L = np.broadcast_to(np.asarray(L, dtype=np.int32), (B,)).copy()
    ql = np.full(B, n, np.int32) if q_len is None else np.asarray(q_len, np.int32)
    max_len = int(L.max()) if max_len is None else max_len
    if page_size:
        npg = (L + page_size - 1) // page_size
        P = int(npg.sum())
        perm = rng.permutation(P).astype(np.int32)
        page_table = np.zeros((B, int(npg.max()) + 1), np.int32)
        off = 0
        for b in range(B):
            page_table[b, :npg[b]] = perm[off:off + npg[b]]
            off += npg[b]
        kv_shape = (P, Hkv, page_size, d)
    else:
        page_table = None
        kv_shape = (B, Hkv, max_len, d)
    q = _normal(rng, (B, n, Hq, d))
    k = _normal(rng, kv_shape, kv_scale)
    v = _normal(rng, kv_shape, kv_scale)
    lists = []
    for b in range(B):
        Lb = int(L[b])
        tail = np.arange(max(0, Lb - int(ql[b])), Lb)
        extra = np.flatnonzero(rng.random(max(0, Lb - int(ql[b]))) < text_frac)
        lists.append(np.union1d(extra, tail).astype(np.int32))
    t_max = max(1, max(len(x) for x in lists))
    text_idx = np.zeros((B, t_max), np.int32)
    text_len = np.zeros(B, np.int32)
    for b, x in enumerate(lists):
        text_idx[b, :len(x)] = x
        text_len[b] = len(x)
    return AttnCase(
        name=f"small_s{seed}", dtype=dtype,
        q=Stored.from_f32(q, dtype), k=Stored.from_f32(k, dtype), v=Stored.from_f32(v, dtype),
        kv_len=L, q_len=ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=max_len,
        page_size=page_size, page_table=page_table, text_idx=text_idx, text_len=text_len)


def _text_positions(rng: np.random.Generator, L: int, n: int) -> np.ndarray:
    """n distinct ascending text positions below L: half of them (rounded
    up) trail the sequence, the rest are spread at random before them."""
    n = min(n, L)
    trail = (n + 1) // 2
    inter = np.sort(rng.choice(L - trail, size=n - trail, replace=False)) if n > trail else \
        np.zeros(0, np.int64)
    return np.concatenate([inter, np.arange(L - trail, L)]).astype(np.int32)


def std_small(seed: int, B: int, Hq: int, Hkv: int, d: int, L, dtype: str, n_text,
              page_size: int = 0, top_k: int = 16, n: int = 1, max_len: Optional[int] = None,
              q_scale: float = 1.0) -> StdCase:
    """Random prefill-selection case at test sizes: ragged lengths, text
    tokens interleaved with the visual ones and trailing them, optional
    paging.  Draw order: K -> V -> text layout -> text queries -> draft rows."""
    rng = np.random.default_rng(seed)
    L = np.broadcast_to(np.asarray(L, dtype=np.int32), (B,)).copy()
    nt = np.broadcast_to(np.asarray(n_text, dtype=np.int32), (B,)).copy()
    max_len = int(L.max()) if max_len is None else max_len
    if page_size:
        npg = (L + page_size - 1) // page_size
        P = int(npg.sum())
        perm = rng.permutation(P).astype(np.int32)
        page_table = np.zeros((B, int(npg.max()) + 1), np.int32)
        off = 0
        for b in range(B):
            page_table[b, :npg[b]] = perm[off:off + npg[b]]
            off += npg[b]
        kv_shape = (P, Hkv, page_size, d)
    else:
        page_table = None
        kv_shape = (B, Hkv, max_len, d)
    k = _normal(rng, kv_shape, 0.5)
    v = _normal(rng, kv_shape, 0.5)
    t_max = max(1, int(nt.max()))
    text_idx = np.zeros((B, t_max), np.int32)
    text_len = np.zeros(B, np.int32)
    for b in range(B):
        x = _text_positions(rng, int(L[b]), int(nt[b]))
        text_idx[b, :len(x)] = x
        text_len[b] = len(x)
    q_text = _normal(rng, (B, t_max, Hq, d), q_scale)
    q = _normal(rng, (B, n, Hq, d))
    return StdCase(
        name=f"std_s{seed}", dtype=dtype, q_text=Stored.from_f32(q_text, dtype),
        k=Stored.from_f32(k, dtype), v=Stored.from_f32(v, dtype), q=Stored.from_f32(q, dtype),
        kv_len=L, q_len=np.full(B, n, np.int32), text_idx=text_idx, text_len=text_len,
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=max_len, top_k=top_k,
        page_size=page_size, page_table=page_table)


def c2_std(seed: int = 0, top_k: int = 2048) -> StdCase:
    """Sparse-to-Dense prefill selection at the 25k-visual-token shape, bf16:
    B=1, 28/4 heads, d=128, 25000 visual + 512 text positions in the same
    layout as the Sparrow-scale step (64 interleaved, 448 trailing), one
    prefill query row per text token, K = 2048 kept visual positions, one
    draft row.  Draw order: K -> V -> text queries -> draft row."""
    rng = np.random.default_rng([seed, 2])
    B, Hq, Hkv, d, Lvis, Ltxt = 1, 28, 4, 128, 25000, 512
    L = Lvis + Ltxt
    k = _normal(rng, (B, Hkv, L, d), 0.5)
    v = _normal(rng, (B, Hkv, L, d), 0.5)
    q_text = _normal(rng, (B, Ltxt, Hq, d))
    q = _normal(rng, (B, 1, Hq, d))
    return StdCase(
        name="c2_std", dtype=BF16, q_text=Stored.from_f32(q_text, BF16),
        k=Stored.from_f32(k, BF16), v=Stored.from_f32(v, BF16), q=Stored.from_f32(q, BF16),
        kv_len=np.array([L], np.int32), q_len=np.array([1], np.int32),
        text_idx=c2_text_layout(Lvis, Ltxt)[None, :], text_len=np.array([Ltxt], np.int32),
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_len=L, top_k=top_k)
