"""The oracle still reproduces the stored C1 fixture (tests/golden)."""
import json
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c1_expected.json")


def test_c1_golden_fixture():
    with open(GOLDEN) as f:
        g = json.load(f)
    attn, acc = W.c1_tiny(0)
    t, n, nxt = oracle.accept(acc.logits.values, acc.draft, acc.gamma)
    assert t[0].tolist() == g["accept"]["target_tok"]
    assert int(n[0]) == g["accept"]["accept_len"] == 2
    assert int(nxt[0]) == g["accept"]["next_tok"]
    o, lse = oracle.verify_attention(attn.q.values, attn.k.values, attn.v.values, attn.kv_len,
                                     attn.q_len, attn.num_kv_heads, attn.scale)
    assert np.max(np.abs(lse[0] - np.array(g["verify_lse"]))) < 1e-12
    assert np.max(np.abs(o[0].sum(-1) - np.array(g["verify_out_row_sums"]))) < 1e-12
    ov, lv = oracle.vata_attention(attn.q.values, attn.k.values, attn.v.values, attn.kv_len,
                                   attn.q_len, attn.text_idx, attn.text_len,
                                   attn.num_kv_heads, attn.scale)
    assert np.max(np.abs(lv[0] - np.array(g["vata_lse"]))) < 1e-12
    assert np.max(np.abs(ov[0].sum(-1) - np.array(g["vata_out_row_sums"]))) < 1e-12
