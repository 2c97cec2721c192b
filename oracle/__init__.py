"""CPU fp64 oracle for the speculative-decoding attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and never imports it.

Each function is the plain definition of one step, evaluated in float64 on the
exact (widened) values of the stored inputs:

* ``verify_attention``  -- dense verification of gamma+1 draft rows over the
  full KV cache (Sparse-to-Dense pt explainer, "Metodologia", decoding
  procedure: the dense model checks all speculative tokens in parallel with a
  single I/O pass over the full KV cache, using standard attention).
* ``vata_attention``    -- text-anchored draft attention over an index list of
  text positions; the visual KV is never touched (Sparrow zh explainer,
  technical summary 3.1 HSR-VATA; Sparrow pt explainer 3.A).
* ``topk_select`` / ``topk_attention`` -- top-K sparse draft attention
  (Sparse-to-Dense pt explainer, "Metodologia": the sparse model attends to the
  most relevant KV entries only; "Seleção de Cache KV" for the group-mean
  score).
* ``hsr_fuse``          -- FC over the concatenation [e_t ; h_{t-1}] (Sparrow zh
  explainer 3.1, hidden-state reuse).
* ``std_prefill_scores`` / ``std_prefill_select`` / ``std_keep_list`` --
  Sparse-to-Dense's prefill selection: per (sequence, KV head), the top-K
  visual positions by the mean attention of the text tokens, kept with the
  text positions (Sparse-to-Dense pt explainer, "Seleção de Cache KV").
* ``sparse_attention``  -- the sparse draft attention over such a per-head
  list plus a dense tail: the positions written since, or a sliding window
  (same page, "Metodologia"; the window variants of Sparrow's text anchors).
* ``commit``            -- the bookkeeping that follows acceptance: keep
  the accepted rows of the cache, roll back the rest, append the emitted
  tokens and the new text positions (same page, decoding procedure).
* ``accept``            -- greedy acceptance: longest prefix of draft tokens that
  match the dense model's argmax, plus one bonus token (Sparse-to-Dense pt
  explainer, "Metodologia", decoding procedure).

Pins (closed forms, invariants, brute force) live in ``tests/test_oracle_*``.
One function is "parity unpinned" in part: the aggregation rule of the top-K
score (sum of the group's queries) is a reading, fixed by the workload
definition rather than the pages; its selection and attention steps are pinned.
The prefill selection's granularity (one list per KV head, the group's heads
averaged) is likewise a reading; its arithmetic is pinned.
"""
from .attention import (verify_attention, vata_attention, topk_scores, topk_select,
                        topk_attention, paged_rows)
from .hsr import hsr_fuse, hsr_fuse_loops
from .accept import accept, argmax_lowest, commit
from .std import sparse_attention, std_keep_list, std_prefill_scores, std_prefill_select

__all__ = ["verify_attention", "vata_attention", "topk_scores", "topk_select",
           "topk_attention", "paged_rows", "hsr_fuse", "hsr_fuse_loops", "accept",
           "argmax_lowest", "commit", "std_prefill_scores", "std_prefill_select", "std_keep_list",
           "sparse_attention"]
