"""Writes tests/golden/c1_expected.json from the oracle only.

The pages print no worked numeric example, so the stored values here come
from the CPU oracle on the tiny fp32 workload (seed 0): the acceptance result
the workload plants (two matching draft tokens, then a miss) and a few
attention outputs.  They pin the oracle against silent drift; each value is
re-derivable by running this script.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def main():
    attn, acc = W.c1_tiny(0)
    t, n, nxt = oracle.accept(acc.logits.values, acc.draft, acc.gamma)
    o, lse = oracle.verify_attention(attn.q.values, attn.k.values, attn.v.values, attn.kv_len,
                                     attn.q_len, attn.num_kv_heads, attn.scale)
    ov, lv = oracle.vata_attention(attn.q.values, attn.k.values, attn.v.values, attn.kv_len,
                                   attn.q_len, attn.text_idx, attn.text_len,
                                   attn.num_kv_heads, attn.scale)
    doc = {
        "source": "oracle on workloads.c1_tiny(seed=0); see make_golden.py",
        "accept": {"target_tok": t[0].tolist(), "accept_len": int(n[0]),
                   "next_tok": int(nxt[0])},
        "verify_lse": lse[0].tolist(),
        "verify_out_row_sums": o[0].sum(axis=-1).tolist(),
        "vata_lse": lv[0].tolist(),
        "vata_out_row_sums": ov[0].sum(axis=-1).tolist(),
    }
    with open(os.path.join(HERE, "c1_expected.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
