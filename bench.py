"""Benchmark of the speculative-decoding hot path on one MI355X.

Workload: the 25k-visual-token step -- one sequence, 28 query / 4 KV heads of
dim 128, 25,000 visual + 512 text KV positions (64 interleaved + 448
trailing), gamma = 5, hidden size 3584, vocabulary 152,064, bf16 inputs with
fp32 accumulation.  Inputs are seeded synthetic normals (the pages measure on
video benchmarks and trained models that are not used here).

One step = one speculative iteration through every hot-path entry point:
  5 x [ spec_hsr_fuse (one row, 7168 -> 3584)  ->  spec_vata_attn (n = 1) ]
  spec_topk_attn  (one query, K = 2048 over all 25,512 keys)
  spec_verify_attn (gamma + 1 = 6 rows over all 25,512 keys)
  spec_accept      (argmax over [6, 152,064] bf16 logits + prefix)

Timing: every timed unit is a captured HIP graph replayed on one stream, with
HIP events around the replays; KV caches, HSR weights and logits rotate over
enough copies that each call streams from HBM, not the 256 MiB Infinity
Cache.  The headline value is the verification attention's algorithmic HBM
bandwidth; draft steps/s is 1 / (HSR + text-anchored attention time).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=10, help="buffer copies cycled through")
    ap.add_argument("--reps", type=int, default=40, help="replays of each per-entry-point graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["verify", "vata", "hsr", "topk", "accept", "step", "c5",
                                       "std", "verify_b16", "c3", "c4", "lvis", "ceiling"],
                    default=None, help="time one part only (for counter passes)")
    return ap.parse_args()


def expected_tokens(alpha: float, gamma: int) -> float:
    """Tokens emitted per round when each draft token is accepted
    independently with probability alpha: the accepted prefix n has
    P(n = k) = alpha^k (1 - alpha) for k < gamma and P(n = gamma) = alpha^gamma,
    and every round adds the bonus token, so E = sum_k (k + 1) P(n = k) =
    (1 - alpha^(gamma+1)) / (1 - alpha)."""
    if alpha >= 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def io_model(alpha, gamma, draft_us, verify_us, dense_us, draft_bytes, verify_bytes,
             dense_bytes):
    """Sparse-to-Dense's I/O argument for the attention of one layer: a round
    is gamma sparse draft steps plus one dense verification of gamma + 1 rows
    and yields expected_tokens(alpha, gamma) tokens; plain decoding reads the
    whole cache once per token.  Returns per-token KV bytes and attention
    time for both."""
    e = expected_tokens(alpha, gamma)
    return {"alpha": alpha, "gamma": gamma, "tokens_per_round": round(e, 3),
            "kv_bytes_per_token": round((gamma * draft_bytes + verify_bytes) / e),
            "dense_kv_bytes_per_token": dense_bytes,
            "attn_us_per_token": round((gamma * draft_us + verify_us) / e, 3),
            "dense_attn_us_per_token": round(dense_us, 3),
            "attn_speedup": round(dense_us * e / (gamma * draft_us + verify_us), 3)}


def cpu_verify_baseline(oracle, attn, Hkv, scale, call_bytes, seconds):
    """Times the oracle on whole verification calls for about `seconds`: the
    (sequence, KV head) units of several calls at once go to a thread pool as
    wide as the CPUs this process may use, with BLAS pinned to one thread per
    worker (numpy releases the GIL inside its kernels).  Returns the
    cpu_baseline object (throughput over every call finished)."""
    import concurrent.futures as cf
    host = len(os.sched_getaffinity(0))
    units = [(b, g) for b in range(attn.q.shape[0]) for g in range(Hkv)]
    per_round = max(1, host // len(units))          # calls in flight together
    threads = min(host, per_round * len(units))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:
        limit = None

    q, k, v = attn.q.values, attn.k.values, attn.v.values     # inputs widened once

    def one(u):
        oracle.verify_attention(q, k, v, attn.kv_len, attn.q_len, Hkv, scale, units=[u])

    t_start = time.perf_counter()
    calls = 0
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(one, units * per_round))
            calls += per_round
            if time.perf_counter() - t_start >= seconds:
                break
    secs = (time.perf_counter() - t_start) / calls
    if limit is not None:
        limit.restore_original_limits()
    return {"value": round(call_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cores": host, "blas_threads_per_worker": 1, "kind": "oracle",
            "sample": f"{calls} full verification calls of this workload ({len(units)} "
                      f"(sequence, KV head) units x 42 rows x 25,512 keys each, fp64 numpy), "
                      f"{per_round} in flight at a time on {threads} pool threads; "
                      f"{secs:.3f} s per call"}


def break_even_alpha(gamma, draft_us, verify_us, dense_us):
    """Smallest acceptance rate at which a round of gamma draft steps and one
    verification costs no more attention time per token than plain decoding:
    dense_us * expected_tokens(alpha, gamma) = gamma * draft_us + verify_us.
    expected_tokens rises from 1 (alpha = 0) to gamma + 1 (alpha = 1), so the
    root is found by bisection; None when even alpha = 1 does not pay."""
    need = (gamma * draft_us + verify_us) / dense_us
    if need <= 1.0:
        return 0.0
    if need > gamma + 1:
        return None
    lo, hi = 0.0, 1.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if expected_tokens(mid, gamma) < need:
            lo = mid
        else:
            hi = mid
    return round(hi, 4)


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_decoding_attention_amd as S
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = max(1, args.rotate)

    # ------------------------------------------------------------- inputs --
    attn, hsr, acc = W.c2_sparrow(0)
    B, n, Hq, d = attn.q.shape
    Hkv, L, gamma, top_k = attn.num_kv_heads, attn.max_len, n - 1, attn.top_k
    D = hsr.e.shape[1]
    V = acc.logits.shape[2]

    def to_dev(st):
        if st.dtype == W.BF16:
            return torch.from_numpy(st.bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(st.bits).to(dev)

    k0, v0 = to_dev(attn.k), to_dev(attn.v)
    kv_len = torch.tensor(attn.kv_len, dtype=torch.int32, device=dev)
    kvs = [S.KVCache(k0 if r == 0 else k0.clone(), v0 if r == 0 else v0.clone(), kv_len)
           for r in range(R)]
    q = to_dev(attn.q)
    q_last = q[:, -1:].contiguous()
    text_idx = torch.tensor(attn.text_idx, dtype=torch.int32, device=dev)
    text_len = torch.tensor(attn.text_len, dtype=torch.int32, device=dev)
    e, h = to_dev(hsr.e), to_dev(hsr.h)
    w0 = to_dev(hsr.w)
    ws = [w0 if r == 0 else w0.clone() for r in range(R)]
    lg0 = to_dev(acc.logits)
    logits = [lg0 if r == 0 else lg0.clone() for r in range(R)]
    draft = torch.tensor(acc.draft, dtype=torch.int32, device=dev)
    scale = attn.scale

    # outputs, preallocated so captured graphs allocate nothing
    o_ver = torch.empty((B, n, Hq, d), dtype=torch.bfloat16, device=dev)
    l_ver = torch.empty((B, n, Hq), dtype=torch.float32, device=dev)
    y_hsr = torch.empty((gamma, D), dtype=torch.bfloat16, device=dev)
    o_vata = torch.empty((gamma, 1, Hq, d), dtype=torch.bfloat16, device=dev)
    l_vata = torch.empty((gamma, 1, Hq), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=dev)
    o_topk = torch.empty((B, 1, Hq, d), dtype=torch.bfloat16, device=dev)
    l_topk = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
    t_tok = torch.empty((B, n), dtype=torch.int32, device=dev)
    a_len = torch.empty((B,), dtype=torch.int32, device=dev)
    n_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    wsp = {k: S.Workspace(dev) for k in ("verify", "vata", "topk", "hsr", "accept")}

    def call_hsr(r, k):
        S.spec_hsr_fuse(e[k:k + 1], h[k:k + 1], ws[r], y=y_hsr[k:k + 1], workspace=wsp["hsr"])

    def call_vata(r, k):
        S.spec_vata_attn(kvs[r], y_hsr[k:k + 1].view(1, 1, Hq, d), text_idx, text_len,
                         scale=scale, out=o_vata[k:k + 1], lse=l_vata[k:k + 1],
                         workspace=wsp["vata"])

    def call_topk(r):
        S.spec_topk_attn(kvs[r], q_last, top_k, scale=scale, sel_idx=sel, out=o_topk,
                         lse=l_topk, workspace=wsp["topk"])

    def call_verify(r):
        S.spec_verify_attn(kvs[r], q, scale=scale, out=o_ver, lse=l_ver,
                           workspace=wsp["verify"])

    def call_accept(r):
        S.spec_accept(logits[r], draft, target_tok=t_tok, accept_len=a_len, next_tok=n_tok,
                      workspace=wsp["accept"])

    def step(r):
        for k in range(gamma):
            call_hsr(r, k)
            call_vata(r, k)
        call_topk(r)
        call_verify(r)
        call_accept(r)

    # eager warm-up of the headline calls (sizes their workspaces before
    # capture); the other sections size their own with eager calls, so a
    # profile of one of them holds only that section's kernels
    if args.only in (None, "verify", "vata", "hsr", "topk", "accept", "step"):
        for r in range(R):
            step(r)
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    stream = torch.cuda.current_stream(dev)

    def time_graph(g, replays, warm_ms=30.0, timed_ms=10.0):
        # untimed replays first, for at least warm_ms of GPU time and half
        # the timed count: calls under continuous load settle over the first
        # tens of milliseconds (the ragged paged batch: 141, 125, 122, 120,
        # 119 us per call in successive 6.5 ms loops; the C2 verification
        # 20.7 us in its first loop, 20.0 after), and steady-state calls are
        # what is reported.  The timed loop then covers at least timed_ms:
        # the first few launches after a long burst of queued replays start
        # late (a text-anchored graph of 98 us read 124-162 us per replay
        # over 4 replays there, 97 us over 100).
        g.replay()
        torch.cuda.synchronize()
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        g.replay()
        w1.record(stream)
        w1.synchronize()
        one_ms = max(w0.elapsed_time(w1), 1e-3)
        for _ in range(min(4000, max(replays // 2, int(warm_ms / one_ms) + 1))):
            g.replay()
        torch.cuda.synchronize()
        replays = min(4000, max(replays, int(timed_ms / one_ms) + 1))
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(replays):
            g.replay()
        t1.record(stream)
        t1.synchronize()
        return t0.elapsed_time(t1) / replays   # ms per replay

    def main_kernel_us(call, count, warm=2):
        """Mean duration (us) of the main kernel of call(i), i = 0, 1, ...:
        the library's measurement hook records two events on the call's
        stream right before and right after that kernel (eager calls).  The
        events are timing-only HIP events (no system-scope fence when
        recorded), so the pair spans the kernel's dispatch and the command
        processor's handling of the two event packets, but no cache
        write-back or invalidation."""
        pairs = []
        for i in range(warm + count):
            e0, e1 = S.TimingEvent(), S.TimingEvent()
            # a spin ahead of the call keeps the GPU busy while the host
            # enqueues the events and the call's launches, so the kernel
            # starts right after `before` instead of waiting for the host
            torch.cuda._sleep(1_000_000)
            S.mark_main_kernel(e0, e1)
            call(i)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([a_.elapsed_ms(b_) for a_, b_ in pairs[warm:]])) * 1e3

    from speculative_decoding_attention_amd.profiling import source_hash
    src_hash = source_hash()
    counters = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == src_hash:
            counters = tr.get("kernels", {})

    def roofline(key, bound, work, us):
        """Roofline of one main kernel: `work` algorithmic bytes (hbm) or
        flops (mfma) per launch over its measured duration; `traffic` is the
        HBM bytes per launch the FETCH_SIZE / WRITE_SIZE counters saw for
        this kernel with the same sources (None otherwise)."""
        if bound == "hbm":
            ach, peak, unit = work / (us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
        else:
            ach, peak, unit = work / (us * 1e-6) / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s"
        c = counters.get(key)
        return {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": c.get("bytes") if c else None,
                "kernel": key, "kernel_us": round(us, 3), "work_per_launch": work,
                # the same kernel's mean duration in the committed kernel trace
                "trace_us": c.get("mean_us") if c else None}

    result = {}
    parts = {}
    only = args.only

    # ---- per-entry-point graphs: R back-to-back calls over R buffer copies
    if only in (None, "verify"):
        g = capture(lambda: [call_verify(r) for r in range(R)])
        parts["verify_us"] = time_graph(g, args.reps) * 1e3 / R
    if only in (None, "vata"):
        g = capture(lambda: [call_vata(r, 0) for r in range(R)])
        parts["vata_us"] = time_graph(g, args.reps) * 1e3 / R
    if only in (None, "hsr"):
        g = capture(lambda: [call_hsr(r, 0) for r in range(R)])
        parts["hsr_us"] = time_graph(g, args.reps) * 1e3 / R
    if only in (None, "topk"):
        g = capture(lambda: [call_topk(r) for r in range(R)])
        parts["topk_us"] = time_graph(g, args.reps) * 1e3 / R
    if only in (None, "accept"):
        g = capture(lambda: [call_accept(r) for r in range(R)])
        parts["accept_us"] = time_graph(g, args.reps) * 1e3 / R
    if only in (None, "vata", "hsr"):
        g = capture(lambda: [(call_hsr(r, 0), call_vata(r, 0)) for r in range(R)])
        parts["draft_step_us"] = time_graph(g, args.reps) * 1e3 / R

    # ---- the timed region: exactly `steps` whole steps, one graph per copy
    ms_per_step = None
    if only in (None, "step"):
        graphs = [capture(lambda r=r: step(r)) for r in range(R)]
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(args.steps):
            graphs[i % R].replay()
        t1.record(stream)
        t1.synchronize()
        ms_per_step = t0.elapsed_time(t1) / args.steps

    # ---- the batched draft workload (64 sequences, gamma = 5): the fusion FC
    # on the matrix cores (M = 320), text-anchored attention over 2048 text
    # rows per sequence and acceptance over [64, 6, vocab] logits.  Seeded
    # device-side normals of the workload's shapes and scales.
    c5 = None
    if only in (None, "c5"):
        torch.manual_seed(0)
        Bc, Lt, Mc = 64, 2048, 64 * gamma
        ec = torch.randn(Mc, D, device=dev).mul_(0.02).to(torch.bfloat16)
        hc = torch.randn(Mc, D, device=dev).mul_(0.02).to(torch.bfloat16)
        yc = torch.empty(Mc, D, dtype=torch.bfloat16, device=dev)
        S.spec_hsr_fuse(ec, hc, ws[0], y=yc, workspace=wsp["hsr"])   # sizes the workspace
        torch.cuda.synchronize()
        g = capture(lambda: [S.spec_hsr_fuse(ec, hc, ws[r], y=yc, workspace=wsp["hsr"])
                             for r in range(R)])
        hsr_c5_us = time_graph(g, max(4, args.reps // 4)) * 1e3 / R
        # context, not the library's path: the vendor GEMM (hipBLASLt through
        # torch) at the same shape and weight layout, on the rows already
        # concatenated, over the same rotated weight copies
        xcat = torch.cat([ec, hc], 1)
        torch.nn.functional.linear(xcat, ws[0])      # the library's own set-up, eager
        torch.cuda.synchronize()
        g = capture(lambda: [torch.nn.functional.linear(xcat, ws[r]) for r in range(R)])
        vendor_c5_us = time_graph(g, max(4, args.reps // 4)) * 1e3 / R
        del xcat, g
        kvc = []
        for _ in range(2):      # two copies: 2 x 268 MB, more than the 256 MiB cache
            kc = torch.randn(Bc, Hkv, Lt, d, device=dev).mul_(0.5).to(torch.bfloat16)
            vc = torch.randn(Bc, Hkv, Lt, d, device=dev).mul_(0.5).to(torch.bfloat16)
            kvc.append(S.KVCache(kc, vc, torch.full((Bc,), Lt, dtype=torch.int32, device=dev)))
        qc = yc.view(Bc, gamma, Hq, d)
        tic = torch.arange(Lt, dtype=torch.int32, device=dev).repeat(Bc, 1)
        tlc = torch.full((Bc,), Lt, dtype=torch.int32, device=dev)
        oc = torch.empty((Bc, gamma, Hq, d), dtype=torch.bfloat16, device=dev)
        lc = torch.empty((Bc, gamma, Hq), dtype=torch.float32, device=dev)
        g = capture(lambda: [S.spec_vata_attn(kv, qc, tic, tlc, scale=scale, out=oc, lse=lc,
                                              workspace=wsp["vata"]) for kv in kvc])
        vata_c5_us = time_graph(g, max(4, args.reps // 4)) * 1e3 / len(kvc)
        vata_main_us = main_kernel_us(lambda i: S.spec_vata_attn(kvc[i % 2], qc, tic, tlc,
                                                                 scale=scale, out=oc, lse=lc,
                                                                 workspace=wsp["vata"]), 6)
        del kvc
        lgc = [torch.randn(Bc, n, V, device=dev).to(torch.bfloat16) for _ in range(3)]
        drc = torch.randint(0, V, (Bc, gamma), dtype=torch.int32, device=dev)
        tc = torch.empty((Bc, n), dtype=torch.int32, device=dev)
        ac = torch.empty((Bc,), dtype=torch.int32, device=dev)
        nc = torch.empty((Bc,), dtype=torch.int32, device=dev)
        g = capture(lambda: [S.spec_accept(lg, drc, target_tok=tc, accept_len=ac, next_tok=nc,
                                           workspace=wsp["accept"]) for lg in lgc])
        acc_c5_us = time_graph(g, max(4, args.reps // 4)) * 1e3 / len(lgc)
        acc_main_us = main_kernel_us(lambda i: S.spec_accept(lgc[i % len(lgc)], drc, target_tok=tc,
                                                             accept_len=ac, next_tok=nc,
                                                             workspace=wsp["accept"]), 6)
        hsr_main_us = main_kernel_us(lambda i: S.spec_hsr_fuse(ec, hc, ws[i % R], y=yc,
                                                               workspace=wsp["hsr"]), 10)
        del lgc
        hsr_c5_flops = 2 * Mc * D * 2 * D
        vata_c5_bytes = 2 * Bc * Hkv * Lt * d * 2 + Bc * Lt * 4 + 2 * Bc * gamma * Hq * d * 2
        acc_c5_bytes = Bc * n * V * 2
        c5 = {"workload": "batched-draft-64x5", "hsr_us": round(hsr_c5_us, 2),
              "hsr_tflops": round(hsr_c5_flops / (hsr_c5_us * 1e-6) / 1e12, 1),
              "hsr_mfma_frac": round(hsr_c5_flops / (hsr_c5_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS,
                                     4),
              "vendor_gemm_us": round(vendor_c5_us, 2),
              "vata_us": round(vata_c5_us, 2),
              "vata_gbs": round(vata_c5_bytes / (vata_c5_us * 1e-6) / 1e9, 1),
              "accept_us": round(acc_c5_us, 2),
              "accept_gbs": round(acc_c5_bytes / (acc_c5_us * 1e-6) / 1e9, 1),
              # main kernels: the GEMM (no split-K reduce), the split pass of
              # the text-anchored attention (its K/V/Q reads), the logits scan
              "roofline": roofline("c5_hsr_gemm", "mfma", hsr_c5_flops, hsr_main_us),
              "vata_roofline": roofline("c5_vata_split", "hbm",
                                        2 * Bc * Hkv * Lt * d * 2 + Bc * Lt * 4 +
                                        Bc * gamma * Hq * d * 2, vata_main_us),
              "accept_roofline": roofline("c5_accept_scan", "hbm", acc_c5_bytes, acc_main_us)}

    # ---- the draft step as the video grows: text-anchored attention (one
    # row, 512 text positions in the same layout) and the draft step (HSR row
    # + VATA) at 500, 5,000 and 25,000 visual tokens, against dense one-row
    # decoding over the whole cache, the cost the text anchoring avoids.
    # Enough cache copies rotate that 520 MB stream per pass over them.
    sweep = None
    if only in (None, "lvis"):
        sweep = []
        call_hsr(0, 0)          # the draft query below is this HSR row
        torch.cuda.synchronize()
        for lv in (500, 5000, 25000):
            Lw = lv + 512
            copy_bytes = 2 * Hkv * Lw * d * 2
            Rw = max(R, -(-520_000_000 // copy_bytes))
            lw_len = torch.full((1,), Lw, dtype=torch.int32, device=dev)
            kvw = [S.KVCache(torch.randn(1, Hkv, Lw, d, device=dev).mul_(0.5).to(torch.bfloat16),
                             torch.randn(1, Hkv, Lw, d, device=dev).mul_(0.5).to(torch.bfloat16),
                             lw_len) for _ in range(Rw)]
            tiw = torch.tensor(W.c2_text_layout(lv, 512)[None, :], dtype=torch.int32,
                               device=dev)
            tlw = torch.full((1,), 512, dtype=torch.int32, device=dev)
            ow = torch.empty((1, 1, Hq, d), dtype=torch.bfloat16, device=dev)
            lw = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)
            ws_w = {k_: S.Workspace(dev) for k_ in ("vata", "dense")}

            def vata_w(j):
                S.spec_vata_attn(kvw[j], y_hsr[:1].view(1, 1, Hq, d), tiw, tlw, scale=scale,
                                 out=ow, lse=lw, workspace=ws_w["vata"])

            def dense_w(j):
                S.spec_verify_attn(kvw[j], q_last, scale=scale, out=ow, lse=lw,
                                   workspace=ws_w["dense"])
            for j in range(Rw):
                vata_w(j), dense_w(j)
            torch.cuda.synchronize()
            t_v = time_graph(capture(lambda: [vata_w(j) for j in range(Rw)]), 4) * 1e3 / Rw
            t_s = time_graph(capture(lambda: [(call_hsr(j % R, 0), vata_w(j))
                                              for j in range(Rw)]), 4) * 1e3 / Rw
            t_d = time_graph(capture(lambda: [dense_w(j) for j in range(Rw)]), 4) * 1e3 / Rw
            sweep.append({"visual_tokens": lv, "kv_len": Lw, "copies": Rw,
                          "vata_us": round(t_v, 3), "draft_step_us": round(t_s, 3),
                          "draft_steps_per_s": round(1e6 / t_s, 1),
                          "dense_decode_us": round(t_d, 3)})
            del kvw

    # ---- Sparse-to-Dense at the same shape: the prefill selection of one
    # layer (512 text queries x 28 heads over 25,512 positions, K = 2048) and
    # the sparse draft step over the kept lists plus 64 decoded positions.
    std = None
    if only in (None, "std"):
        cs = W.c2_std(0)
        kv_s = S.KVCache(to_dev(cs.k), to_dev(cs.v), kv_len)
        qt = to_dev(cs.q_text)
        ti_s = torch.tensor(cs.text_idx, dtype=torch.int32, device=dev)
        tl_s = torch.tensor(cs.text_len, dtype=torch.int32, device=dev)
        ws_std = S.Workspace(dev)
        ws_sp = S.Workspace(dev)
        o_sp = torch.empty((B, 1, Hq, d), dtype=torch.bfloat16, device=dev)
        l_sp = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
        tail = 64
        t0_s = torch.full((B,), L - tail, dtype=torch.int32, device=dev)

        def select_and_sparse(kk):
            """Prefill selection with K = kk, then the sparse draft step over
            the kept lists plus the last `tail` positions; returns the two
            times (us), the kept positions per KV head and the step's bytes."""
            sel_s = torch.empty((B, Hkv, kk), dtype=torch.int32, device=dev)
            keep_s = torch.empty((B, Hkv, kk + cs.t_max), dtype=torch.int32, device=dev)
            klen_s = torch.empty((B, Hkv), dtype=torch.int32, device=dev)

            def call_select():
                S.spec_std_select(kv_s, qt, ti_s, tl_s, kk, scale=scale, sel_idx=sel_s,
                                  keep_idx=keep_s, keep_len=klen_s, workspace=ws_std)
            call_select()
            torch.cuda.synchronize()
            sel_t = time_graph(capture(call_select), max(4, args.reps // 4)) * 1e3
            if kk == cs.top_k:
                pass_us[0] = main_kernel_us(lambda i: call_select(), 4)
            keep_tail = keep_s.clone()
            # the kept positions at or past the tail start are the tail's own
            keep_tail[keep_tail >= L - tail] = -1
            klen_tail = (keep_tail >= 0).sum(dim=2).to(torch.int32)
            keep_tail = torch.sort(torch.where(keep_tail < 0, torch.full_like(keep_tail, 1 << 30),
                                               keep_tail), dim=2).values
            keep_tail = torch.where(keep_tail == (1 << 30), torch.full_like(keep_tail, -1),
                                    keep_tail).contiguous()

            def call_sparse(r):
                S.spec_sparse_attn(kvs[r], q_last, keep_tail, klen_tail, tail_start=t0_s,
                                   tail_max=tail, scale=scale, out=o_sp, lse=l_sp,
                                   workspace=ws_sp)
            for r in range(R):
                call_sparse(r)
            torch.cuda.synchronize()
            sp_t = time_graph(capture(lambda: [call_sparse(r) for r in range(R)]),
                              args.reps) * 1e3 / R
            kept_ = int(klen_tail.sum().item()) + Hkv * tail
            bytes_ = 2 * kept_ * d * 2 + kept_ * 4 + 2 * Hq * d * 2 + Hq * 4
            return sel_t, sp_t, kept_, bytes_

        pass_us = [None]
        per_k = {kk: select_and_sparse(kk) for kk in (512, 1024, 2048, 4096)}
        select_us, sparse_us, kept, sparse_bytes = per_k[cs.top_k]
        # work of the selection: both passes form every visible score
        pos = cs.text_idx[0, :cs.text_len[0]].astype(np.int64)
        visible = int((pos + 1).sum()) * Hq          # (row, key) pairs over all heads
        sel_flops = 2 * 2 * d * visible
        # dense verification at gamma + 1 rows (and plain one-token decode)
        ver_us = {}
        for nr in (1, 4, 6, 9):
            qn = torch.randn((B, nr, Hq, d), device=dev).to(torch.bfloat16)
            on = torch.empty((B, nr, Hq, d), dtype=torch.bfloat16, device=dev)
            ln = torch.empty((B, nr, Hq), dtype=torch.float32, device=dev)
            for r in range(R):
                S.spec_verify_attn(kvs[r], qn, scale=scale, out=on, lse=ln, workspace=wsp["verify"])
            torch.cuda.synchronize()
            g = capture(lambda: [S.spec_verify_attn(kvs[r], qn, scale=scale, out=on, lse=ln,
                                                    workspace=wsp["verify"]) for r in range(R)])
            ver_us[nr] = time_graph(g, args.reps) * 1e3 / R
        kvb = 2 * L * Hkv * d * 2
        model = [io_model(al, gm, sparse_us, ver_us[gm + 1], ver_us[1], sparse_bytes,
                          kvb + 2 * (gm + 1) * Hq * d * 2, kvb + 2 * Hq * d * 2)
                 for gm in (3, 5, 8) for al in (0.5, 0.7, 0.9)]
        # the same model as the retained fraction K/L changes: measured
        # selection and sparse-step times per K, the per-token attention time
        # at gamma = 5, and the acceptance rate at which a round breaks even
        # with plain decoding (time, and KV bytes read)
        kl_rows = []
        for kk, (st_, sp_, kept_, by_) in per_k.items():
            be_t = {str(gm): break_even_alpha(gm, sp_, ver_us[gm + 1], ver_us[1])
                    for gm in (3, 5, 8)}
            be_b = {str(gm): break_even_alpha(gm, by_, kvb + 2 * (gm + 1) * Hq * d * 2,
                                              kvb + 2 * Hq * d * 2) for gm in (3, 5, 8)}
            kl_rows.append({
                "top_k": kk, "kept_per_head": round(kept_ / Hkv, 1),
                "kept_fraction": round(kept_ / (Hkv * L), 4),
                "select_us": round(st_, 2), "sparse_us": round(sp_, 3),
                "sparse_bytes": by_,
                "break_even_alpha_time": be_t, "break_even_alpha_bytes": be_b,
                "gamma5": [io_model(al, 5, sp_, ver_us[6], ver_us[1], by_,
                                    kvb + 2 * 6 * Hq * d * 2, kvb + 2 * Hq * d * 2)
                           for al in (0.5, 0.7, 0.9)]})
        std = {"workload": "std-prefill-select-25k", "select_us": round(select_us, 2),
               "select_tflops": round(sel_flops / (select_us * 1e-6) / 1e12, 1),
               "select_mfma_frac": round(sel_flops / (select_us * 1e-6) / 1e12 /
                                         MFMA_BF16_PEAK_TFS, 4),
               "select_gexp_per_s": round(2 * visible / (select_us * 1e-6) / 1e9, 1),
               "sparse_us": round(sparse_us, 3),
               "sparse_gbs": round(sparse_bytes / (sparse_us * 1e-6) / 1e9, 1),
               "sparse_steps_per_s": round(1e6 / sparse_us, 1),
               "kept_per_head": round(kept / Hkv, 1),
               "verify_us_by_rows": {str(k): round(v, 2) for k, v in ver_us.items()},
               "io_model": {"assumption": "each draft token accepted independently with "
                                          "probability alpha; attention of one layer only",
                            "rows": model},
               "io_model_by_top_k": kl_rows}
        # main kernel: the first of the two score passes (each forms every
        # visible score once: 2 d flops per (row, key) pair and head)
        std["roofline"] = roofline("std_score_pass", "mfma", sel_flops // 2, pass_us[0])
        if not args.no_cpu_baseline and only is None:
            # the oracle on one of the four KV heads (about 2 s), scaled to the layer
            import oracle
            g1 = 2
            k1 = cs.k.values[:, g1:g1 + 1]
            q1 = cs.q_text.values[:, :, 7 * g1:7 * g1 + 7]
            t0 = time.perf_counter()
            oracle.std_prefill_select(q1, k1, cs.kv_len, cs.text_idx, cs.text_len, 1, cs.top_k,
                                      scale)
            one = time.perf_counter() - t0
            std["cpu_baseline"] = {"value": round(one * Hkv * 1e6, 0), "unit": "us per layer",
                                   "kind": "oracle",
                                   "sample": "one of 4 KV heads (512 text rows x 7 heads x "
                                             "25,512 positions, fp64 numpy), times 4"}
        del kv_s

    # ---- the same verification kernel on a batch large enough to stream:
    # 16 sequences x 32,768 positions (1.07 GB of KV), two rotated copies.
    # Device-side normals of the workload's shapes; context for the
    # fixed-cost analysis of the 52 MB call above.
    vb16 = None
    if only in (None, "verify_b16"):
        Bb, Lb = 16, 32768
        kvb = [S.KVCache(torch.randn(Bb, Hkv, Lb, d, device=dev).mul_(0.5).to(torch.bfloat16),
                         torch.randn(Bb, Hkv, Lb, d, device=dev).mul_(0.5).to(torch.bfloat16),
                         torch.full((Bb,), Lb, dtype=torch.int32, device=dev)) for _ in range(2)]
        qb = torch.randn(Bb, n, Hq, d, device=dev).to(torch.bfloat16)
        ob = torch.empty((Bb, n, Hq, d), dtype=torch.bfloat16, device=dev)
        lb = torch.empty((Bb, n, Hq), dtype=torch.float32, device=dev)
        for kv in kvb:
            S.spec_verify_attn(kv, qb, scale=scale, out=ob, lse=lb, workspace=wsp["verify"])
        torch.cuda.synchronize()
        g = capture(lambda: [S.spec_verify_attn(kv, qb, scale=scale, out=ob, lse=lb,
                                                workspace=wsp["verify"]) for kv in kvb])
        vb_us = time_graph(g, max(4, args.reps // 4)) * 1e3 / len(kvb)
        vb_main_us = main_kernel_us(lambda i: S.spec_verify_attn(kvb[i % 2], qb, scale=scale, out=ob,
                                                                 lse=lb, workspace=wsp["verify"]), 6)
        vb_bytes = 2 * Bb * Hkv * Lb * d * 2 + 2 * Bb * n * Hq * d * 2 + Bb * n * Hq * 4
        vb_gbs = vb_bytes / (vb_us * 1e-6) / 1e9
        vb16 = {"workload": "verify-16x32768", "us": round(vb_us, 1), "gbs": round(vb_gbs, 1),
                "frac": round(vb_gbs / HBM_PEAK_GBS, 4),
                "roofline": roofline("b16_verify_split", "hbm",
                                     2 * Bb * Hkv * Lb * d * 2 + Bb * n * Hq * d * 2, vb_main_us)}
        del kvb

    # ---- ragged paged batch (16 sequences, 16-token pages in a random pool
    # order, L_b = Lvis_b + Ltxt_b, n_b = gamma_b + 1 rows padded to 8): verify
    # and text-anchored attention per sequence, and the same batch in a
    # contiguous cache.  One copy of the pool (565 MB) already exceeds the
    # 256 MiB cache twice over.  K/V/Q are drawn on the device (same shapes
    # and scales as the parity cases, which use the host generator).
    c3 = None
    if only in (None, "c3"):
        lay = W.c3_layout(0)
        B3, n3, ps = len(lay.L), 8, 16
        L3 = torch.tensor(lay.L, dtype=torch.int32, device=dev)
        ql3 = torch.tensor(lay.gamma + 1, dtype=torch.int32, device=dev)
        pt3 = torch.tensor(lay.page_table, dtype=torch.int32, device=dev)
        kp = torch.randn(lay.pages, Hkv, ps, d, device=dev).mul_(0.5).to(torch.bfloat16)
        vp = torch.randn(lay.pages, Hkv, ps, d, device=dev).mul_(0.5).to(torch.bfloat16)
        kv3 = S.KVCache(kp, vp, L3, page_table=pt3, page_size=ps, max_len=int(lay.L.max()))
        q3 = torch.randn(B3, n3, Hq, d, device=dev).to(torch.bfloat16)
        o3 = torch.empty((B3, n3, Hq, d), dtype=torch.bfloat16, device=dev)
        l3 = torch.empty((B3, n3, Hq), dtype=torch.float32, device=dev)
        tmax3 = int(lay.ltxt.max())
        ti3 = np.zeros((B3, tmax3), np.int32)
        for b_ in range(B3):
            ti3[b_, :lay.ltxt[b_]] = np.arange(lay.lvis[b_], lay.L[b_], dtype=np.int32)
        ti3 = torch.tensor(ti3, device=dev)
        tl3 = torch.tensor(lay.ltxt, dtype=torch.int32, device=dev)
        ws3 = {k_: S.Workspace(dev) for k_ in ("verify", "vata")}

        def c3_verify(kv):
            S.spec_verify_attn(kv, q3, q_len=ql3, scale=scale, out=o3, lse=l3,
                               workspace=ws3["verify"])

        def c3_vata(kv):
            S.spec_vata_attn(kv, q3, ti3, tl3, q_len=ql3, scale=scale, out=o3, lse=l3,
                             workspace=ws3["vata"])

        reps3 = max(4, args.reps // 4)
        c3_verify(kv3), c3_vata(kv3)
        torch.cuda.synchronize()
        # four calls to a graph, so that the graph's own launch is not on the
        # clock of one call (the 565 MB pool is twice the 256 MiB MALL, so a
        # call still streams it from HBM)
        t_ver = time_graph(capture(lambda: [c3_verify(kv3) for _ in range(4)]), reps3) * 1e3 / 4
        t_vat = time_graph(capture(lambda: [c3_vata(kv3) for _ in range(4)]), reps3) * 1e3 / 4
        ver3_main_us = main_kernel_us(lambda i: c3_verify(kv3), 4)
        del kp, vp, kv3
        mx = int(lay.L.max())
        kc = torch.randn(B3, Hkv, mx, d, device=dev).mul_(0.5).to(torch.bfloat16)
        vc = torch.randn(B3, Hkv, mx, d, device=dev).mul_(0.5).to(torch.bfloat16)
        kvc3 = S.KVCache(kc, vc, L3)
        c3_verify(kvc3)
        torch.cuda.synchronize()
        t_verc = time_graph(capture(lambda: [c3_verify(kvc3) for _ in range(4)]), reps3) * 1e3 / 4
        del kc, vc, kvc3
        nq3 = int((lay.gamma + 1).sum())
        ver3_bytes = 2 * int(lay.L.sum()) * Hkv * d * 2 + 2 * nq3 * Hq * d * 2 + nq3 * Hq * 4
        vat3_bytes = 2 * int(lay.ltxt.sum()) * Hkv * d * 2 + int(lay.ltxt.sum()) * 4 + \
            2 * nq3 * Hq * d * 2 + nq3 * Hq * 4
        gbs = lambda by, us: round(by / (us * 1e-6) / 1e9, 1)
        c3 = {"workload": "ragged-paged-16", "kv_tokens": int(lay.L.sum()),
              "verify_paged_us": round(t_ver, 1), "verify_paged_gbs": gbs(ver3_bytes, t_ver),
              "verify_paged_frac": round(ver3_bytes / (t_ver * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "verify_contiguous_us": round(t_verc, 1),
              "verify_contiguous_gbs": gbs(ver3_bytes, t_verc),
              "vata_paged_us": round(t_vat, 1), "vata_paged_gbs": gbs(vat3_bytes, t_vat),
              # main kernel: the paged split pass (K/V of every position, the
              # valid query rows, the page table)
              "roofline": roofline("c3_verify_paged_split", "hbm",
                                   2 * int(lay.L.sum()) * Hkv * d * 2 + nq3 * Hq * d * 2 +
                                   4 * int(((lay.L + ps - 1) // ps).sum()), ver3_main_us)}

    # ---- top-K draft and dense verification, 4 sequences of 32,768 keys
    # (28,672 visual + 4,096 text), K = 2048: the per-step top-K (score all
    # keys, select, attend) against the dense verification of gamma + 1 rows.
    c4 = None
    if only in (None, "c4"):
        B4, L4, K4 = 4, 32768, 2048
        kv4 = [S.KVCache(torch.randn(B4, Hkv, L4, d, device=dev).mul_(0.5).to(torch.bfloat16),
                         torch.randn(B4, Hkv, L4, d, device=dev).mul_(0.5).to(torch.bfloat16),
                         torch.full((B4,), L4, dtype=torch.int32, device=dev)) for _ in range(2)]
        q4 = torch.randn(B4, n, Hq, d, device=dev).to(torch.bfloat16)
        q4l = q4[:, -1:].contiguous()
        o4 = torch.empty((B4, n, Hq, d), dtype=torch.bfloat16, device=dev)
        l4 = torch.empty((B4, n, Hq), dtype=torch.float32, device=dev)
        s4 = torch.empty((B4, Hkv, K4), dtype=torch.int32, device=dev)
        o4k = torch.empty((B4, 1, Hq, d), dtype=torch.bfloat16, device=dev)
        l4k = torch.empty((B4, 1, Hq), dtype=torch.float32, device=dev)
        ws4 = {k_: S.Workspace(dev) for k_ in ("verify", "topk")}
        f_ver = lambda: [S.spec_verify_attn(kv, q4, scale=scale, out=o4, lse=l4,
                                            workspace=ws4["verify"]) for kv in kv4]
        f_top = lambda: [S.spec_topk_attn(kv, q4l, K4, scale=scale, sel_idx=s4, out=o4k, lse=l4k,
                                          workspace=ws4["topk"]) for kv in kv4]
        f_ver(), f_top()
        torch.cuda.synchronize()
        reps4 = max(4, args.reps // 4)
        t4v = time_graph(capture(f_ver), reps4) * 1e3 / len(kv4)
        t4k = time_graph(capture(f_top), reps4) * 1e3 / len(kv4)
        v4_main_us = main_kernel_us(lambda i: S.spec_verify_attn(kv4[i % 2], q4, scale=scale, out=o4,
                                                                 lse=l4, workspace=ws4["verify"]), 6)
        k4_main_us = main_kernel_us(lambda i: S.spec_topk_attn(kv4[i % 2], q4l, K4, scale=scale,
                                                               sel_idx=s4, out=o4k, lse=l4k,
                                                               workspace=ws4["topk"]), 6)
        del kv4
        v4_bytes = 2 * B4 * Hkv * L4 * d * 2 + 2 * B4 * n * Hq * d * 2 + B4 * n * Hq * 4
        k4_bytes = B4 * Hkv * L4 * d * 2 + 2 * B4 * Hkv * K4 * d * 2 + B4 * Hkv * K4 * 4 + \
            2 * B4 * Hq * d * 2
        c4 = {"workload": "topk-4x32768", "verify_us": round(t4v, 1),
              "verify_gbs": round(v4_bytes / (t4v * 1e-6) / 1e9, 1),
              "verify_frac": round(v4_bytes / (t4v * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "topk_us": round(t4k, 1), "topk_gbs": round(k4_bytes / (t4k * 1e-6) / 1e9, 1),
              "topk_to_dense_bytes": round(k4_bytes / v4_bytes, 3),
              # main kernels: the score pass of the top-K call (every key row
              # and the query heads) and the split pass of the verification
              "roofline": roofline("c4_topk_score", "hbm",
                                   B4 * Hkv * L4 * d * 2 + B4 * Hq * d * 2, k4_main_us),
              "verify_roofline": roofline("c4_verify_split", "hbm",
                                          2 * B4 * Hkv * L4 * d * 2 + B4 * n * Hq * d * 2,
                                          v4_main_us)}

    # ---- plain streaming at the sizes above: the library's read probe (a
    # bare read: 16-byte loads, eight in flight per thread, 1024 workgroups)
    # and, for context, the vendor's device copy (reads and writes every
    # byte), each over enough rotated copies that 520 MB or more stream per
    # pass.  The probe's time for a 52 MB verification call's bytes bounds
    # what any kernel can reach at that size.
    ceiling = None
    if only in (None, "ceiling"):
        ceiling = []
        sink = torch.empty(S.SPEC_READ_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
        for nbytes in (52_335_264, 268_435_456, 1_073_741_824):
            cn = max(2, -(-520_000_000 // nbytes))
            xs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(cn)]
            ys = [torch.empty_like(xs[0]) for _ in range(cn)]
            for j in range(cn):
                S.read_probe(xs[j], sink)
                ys[j].copy_(xs[j])
            torch.cuda.synchronize()
            t_rd = time_graph(capture(lambda: [S.read_probe(x_, sink) for x_ in xs]), 6) * 1e3 / cn
            t_cpy = time_graph(capture(lambda: [y_.copy_(x_) for x_, y_ in zip(xs, ys)]),
                               6) * 1e3 / cn
            ceiling.append({"bytes": nbytes, "copies": cn,
                            "read_us": round(t_rd, 2),
                            "read_gbs": round(nbytes / (t_rd * 1e-6) / 1e9, 1),
                            "copy_us": round(t_cpy, 2),
                            "copy_moved_gbs": round(2 * nbytes / (t_cpy * 1e-6) / 1e9, 1)})
            del xs, ys

    # ---- algorithmic bytes (per call)
    kv_bytes = 2 * L * Hkv * d * 2
    verify_bytes = kv_bytes + 2 * (n * Hq * d * 2) + n * Hq * 4
    vata_bytes = 2 * int(attn.text_len[0]) * Hkv * d * 2 + int(attn.text_len[0]) * 4 + \
        2 * Hq * d * 2 + Hq * 4
    hsr_bytes = D * 2 * D * 2 + 2 * D * 2 + D * 2
    hsr_flops = 2 * 1 * D * 2 * D
    topk_bytes = L * Hkv * d * 2 + 2 * top_k * Hkv * d * 2 + Hq * d * 4 + Hkv * top_k * 4
    accept_bytes = n * V * 2 + gamma * 4 + (n + 2) * 4

    # ---- parity of the timed outputs: every (sequence, KV head) unit of the
    # verification call against the oracle, with the tests' bf16 bounds
    import oracle
    torch.cuda.synchronize()
    call_verify(0)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attention(attn.q.values, attn.k.values, attn.v.values, attn.kv_len,
                                     attn.q_len, Hkv, scale)
    o = o_ver.float().cpu().numpy()
    lo = l_ver.cpu().numpy()
    err = float(np.abs(o - ro).max())
    G = Hq // Hkv
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        eg = float(np.abs(o[:, :, hs] - ro[:, :, hs]).max())
        if eg > 2e-2 or eg > 1e-2 * float(np.abs(ro[:, :, hs]).max()) + 1e-7 or \
                float(np.abs(lo[:, :, hs] - rl[:, :, hs]).max()) > 1e-3:
            print(f"bench: verification output of KV head {g} differs from the oracle "
                  f"(max abs err {eg})", file=sys.stderr)
            sys.exit(1)

    # ---- CPU baseline: the oracle as it stands, on the host cores.  The
    # call's (sequence, KV head) units run on a thread pool as wide as the
    # CPUs this process may use, with BLAS pinned to one thread per worker
    # (numpy releases the GIL inside its kernels).
    cpu = None
    if not args.no_cpu_baseline and only is None:
        cpu = cpu_verify_baseline(oracle, attn, Hkv, scale, verify_bytes, args.cpu_seconds)

    verify_us = parts.get("verify_us")
    value = verify_bytes / (verify_us * 1e-6) / 1e9 if verify_us else None
    roof = None
    if verify_us:
        # the call's dominant kernel: the split pass (the K/V rows and the
        # query block it must read; the partials it writes for the merge are
        # this implementation's traffic, not the method's)
        split_us = main_kernel_us(lambda i: call_verify(i % R), 4 * R)
        roof = roofline("c2_verify_split", "hbm", kv_bytes + n * Hq * d * 2, split_us)
    draft_us = parts.get("draft_step_us")
    result = {
        "metric": "verify-attn HBM GB/s (% peak) + draft steps/s at 25k visual tokens, 1 GPU",
        "value": round(value, 1) if value else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4) if ms_per_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sparrow-25k-visual-step", "batch": 1, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "kv_len": L, "visual_tokens": 25000,
                   "text_tokens": int(attn.text_len[0]), "gamma": gamma, "top_k": top_k,
                   "hidden": D, "vocab": V, "rotate": R},
        "pct_peak": round(100 * value / HBM_PEAK_GBS, 2) if value else None,
        "draft_steps_per_s": round(1e6 / draft_us, 1) if draft_us else None,
        "vata_steps_per_s": round(1e6 / parts["vata_us"], 1) if "vata_us" in parts else None,
        "per_call_us": {k[:-3]: round(v, 3) for k, v in parts.items()},
        "per_call_gbs": {k: round(b / (parts[k + "_us"] * 1e-6) / 1e9, 1)
                         for k, b in (("verify", verify_bytes), ("vata", vata_bytes),
                                      ("hsr", hsr_bytes), ("topk", topk_bytes),
                                      ("accept", accept_bytes)) if k + "_us" in parts},
        "hsr_tflops": round(hsr_flops / (parts["hsr_us"] * 1e-6) / 1e12, 2)
        if "hsr_us" in parts else None,
        "batched_draft": c5,
        "draft_by_visual_tokens": sweep,
        "std": std,
        "verify_batch16": vb16,
        "ragged_paged": c3,
        "topk_batch4": c4,
        "read_ceiling": ceiling,
        "verify_max_abs_err_vs_oracle": err,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
