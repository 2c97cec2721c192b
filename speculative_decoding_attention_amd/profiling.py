"""Counter evidence for the benched kernels: rocprofv3 runs over bench.py
sections, and their summaries under profiles/.

    python -m speculative_decoding_attention_amd.profiling collect OUT [PASS ...]
    python -m speculative_decoding_attention_amd.profiling summarize OUT

(PASS: run only the passes whose names start with one of these, e.g.
``trace`` or ``FETCH_SIZE``, so that the collection can be split into
several shorter runs.)

``collect`` (on a GPU host) runs, from the repository root, one rocprofv3
process per pass, each under its own time limit, and stops at the first
failure:

* a kernel trace of every section (``--kernel-trace --stats``);
* FETCH_SIZE, then WRITE_SIZE, each in a run of its own, for the sections
  whose main kernels are HBM-bound;
* the derived MfmaUtil counter for the sections whose main kernels are
  matrix-core work;
* both byte counters over a plain 256 MiB device copy, which converts the
  counters to bytes (the copy reads and writes exactly 256 MiB).

``summarize`` reads the CSV files back and writes profiles/traffic.json,
profiles/traffic.md and one kernel-duration table per section.  For every
configuration the main kernel is the kernel of the given name whose mean
duration in that section's trace is largest; its counters are then taken
from the dispatches with the same name and grid (the slow mode only, when
two calls of a section share both).  traffic.json carries the
hash of the kernel sources, and bench.py reports ``traffic`` only while the
sources still hash the same.

rocprofv3 runs as a child process of this script; this process never
touches the GPU.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "speculative_decoding_attention_amd", "csrc")
# every source that shapes a kernel or its launch: counters taken before a
# change to any of them no longer describe the library
KERNEL_SOURCES = ["api.hip", "attention.hip", "topk.hip", "hsr.hip", "accept.hip", "std.hip",
                  "stream.hip", "common.h", "internal.h"]

# the bench's own rotation (enough input copies that every pass streams from
# HBM, not from the 256 MiB MALL), fewer replays
BENCH_ARGS = ["--no-cpu-baseline", "--steps", "2", "--warmup", "1", "--reps", "4"]
TRACE_SECTIONS = ["step", "verify", "c3", "c4", "c5", "std", "verify_b16", "ceiling"]
BYTE_SECTIONS = ["verify", "c3", "c4", "c5", "std", "verify_b16"]
MFMA_SECTIONS = ["c5", "std"]
COPY_CMD = ("import torch; x = torch.ones(128 * 1024 * 1024, dtype=torch.bfloat16, device='cuda'); "
            "y = torch.empty_like(x); [y.copy_(x) for _ in range(3)]; torch.cuda.synchronize(); "
            "print('copied 256 MiB three times')")
COPY_BYTES = 256 * 1024 * 1024

PIPE = "attn_bf16_pipe_kernel<"
# configuration -> (bench section, name test of its main kernel, bound)
MAIN_KERNELS = {
    "c2_verify_split": ("verify", lambda k: PIPE in k and "false>" in k, "hbm"),
    "c3_verify_paged_split": ("c3", lambda k: PIPE in k and "true>" in k, "hbm"),
    "c4_verify_split": ("c4", lambda k: PIPE in k and "false>" in k, "hbm"),
    "c4_topk_score": ("c4", lambda k: "topk_score_ring_kernel<" in k, "hbm"),
    "c5_hsr_gemm": ("c5", lambda k: "hsr_mfma_kernel<" in k, "mfma"),
    "c5_vata_split": ("c5", lambda k: PIPE in k and "true>" in k, "hbm"),
    "c5_accept_scan": ("c5", lambda k: "accept_scan_kernel<" in k, "hbm"),
    "b16_verify_split": ("verify_b16", lambda k: PIPE in k and "false>" in k, "hbm"),
    "std_score_pass": ("std", lambda k: "std_mfma_kernel<128, 0" in k, "mfma"),
}


def source_hash() -> str:
    """The hash bench.py compares against (the same files in the same order)."""
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------- collect ----

def _commands(out: str):
    bench = os.path.join(ROOT, "bench.py")
    for sec in TRACE_SECTIONS:
        yield (f"trace_{sec}", 240, ["rocprofv3", "--kernel-trace", "--stats", "--output-format",
                                     "csv", "-d", os.path.join(out, f"trace_{sec}"), "-o", "t",
                                     "--", sys.executable, bench, "--only", sec, *BENCH_ARGS])
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        yield (f"{ctr}_copy", 90, ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d",
                                   os.path.join(out, f"{ctr}_copy"), "-o", "p", "--",
                                   sys.executable, "-c", COPY_CMD])
        for sec in BYTE_SECTIONS:
            yield (f"{ctr}_{sec}", 240, ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d",
                                         os.path.join(out, f"{ctr}_{sec}"), "-o", "p", "--",
                                         sys.executable, bench, "--only", sec, *BENCH_ARGS])
    for sec in MFMA_SECTIONS:
        yield (f"MfmaUtil_{sec}", 240, ["rocprofv3", "--pmc", "MfmaUtil", "--output-format", "csv",
                                        "-d", os.path.join(out, f"MfmaUtil_{sec}"), "-o", "p", "--",
                                        sys.executable, bench, "--only", sec, *BENCH_ARGS])


def collect(out: str, only=()) -> int:
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name, limit, cmd in _commands(out):
        if only and not any(name.startswith(o) for o in only):
            continue
        print(f"[profiling] {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"{name}.log"), "w") as log:
            r = subprocess.run(["timeout", "-s", "KILL", str(limit), *cmd], cwd="/tmp", env=env,
                               stdout=log, stderr=subprocess.STDOUT)
        print(f"[profiling] {name}: exit {r.returncode}", flush=True)
        if r.returncode != 0:
            return r.returncode
    return 0


# ----------------------------------------------------------- summarize ----

def _rows(path_glob: str):
    for p in sorted(glob.glob(path_glob, recursive=True)):
        with open(p) as f:
            yield from csv.DictReader(f)


def _short(name: str) -> str:
    n = name.replace("spec::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0] if n.startswith("void ") or "<" in n else n[:90]


def _durations(out: str, sec: str):
    """{(kernel, grid): [duration us, in dispatch order]} of one section's trace."""
    d = defaultdict(list)
    rows = sorted(_rows(os.path.join(out, f"trace_{sec}", "**", "*kernel_trace.csv")),
                  key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        d[(r["Kernel_Name"], grid)].append((int(r["End_Timestamp"]) -
                                            int(r["Start_Timestamp"])) / 1000.0)
    return d


def _mode_labels(durs, gap: float = 2.0):
    """Mode of each dispatch of one (kernel, grid) group, durations given in
    dispatch order.  Two calls of a section can launch the same kernel with
    the same grid (the paged verification and the paged text-anchored
    attention of the ragged batch, the read probe at three sizes).  The
    dispatches are cut into runs wherever one takes over `gap` times as long
    as the one before it, or under 1/gap of it; runs whose medians are
    within `gap` of each other form one mode.  Returns (labels, modes),
    label 0 the fastest mode."""
    runs = []
    for i, t in enumerate(durs):
        if runs and max(t, durs[i - 1]) <= gap * min(t, durs[i - 1]):
            runs[-1].append(i)
        else:
            runs.append([i])
    med = [statistics.median(durs[j] for j in r) for r in runs]
    order = sorted(range(len(runs)), key=lambda k: med[k])
    labels, mode = [0] * len(durs), 0
    for pos, k in enumerate(order):
        if pos > 0 and med[k] > gap * med[order[pos - 1]]:
            mode += 1
        for j in runs[k]:
            labels[j] = mode
    return labels, mode + 1


def _slowest(durs):
    """The durations of the slowest mode (all of them when there is one)."""
    labels, n = _mode_labels(durs)
    return [t for t, m in zip(durs, labels) if m == n - 1]


def _counter(out: str, run: str, name: str, grid: int, counter: str):
    """Mean of one counter over the slowest mode of a kernel's dispatches."""
    rows = sorted((r for r in _rows(os.path.join(out, run, "**", "*counter_collection.csv"))
                   if r["Kernel_Name"] == name and int(r.get("Grid_Size") or 0) == grid and
                   r["Counter_Name"] == counter), key=lambda r: int(r["Start_Timestamp"]))
    if not rows:
        return None
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in rows]
    labels, n = _mode_labels(durs)
    return statistics.mean(float(r["Counter_Value"]) for r, m in zip(rows, labels) if m == n - 1)


def summarize(out: str, dest: str = PROFILES) -> dict:
    out = os.path.abspath(out)
    fetch_copy = _counter(out, "FETCH_SIZE_copy", _copy_name(out, "FETCH_SIZE_copy"),
                          _copy_grid(out, "FETCH_SIZE_copy"), "FETCH_SIZE")
    write_copy = _counter(out, "WRITE_SIZE_copy", _copy_name(out, "WRITE_SIZE_copy"),
                          _copy_grid(out, "WRITE_SIZE_copy"), "WRITE_SIZE")
    fscale = COPY_BYTES / (fetch_copy * 1024.0)
    wscale = COPY_BYTES / (write_copy * 1024.0)
    kernels, traces = {}, {}
    for key, (sec, test, bound) in MAIN_KERNELS.items():
        if sec not in traces:
            traces[sec] = _durations(out, sec)
        cands = [(statistics.mean(_slowest(v)), k) for k, v in traces[sec].items() if test(k[0])]
        if not cands:
            continue
        _, (name, grid) = max(cands)
        dur = _slowest(traces[sec][(name, grid)])
        e = {"section": sec, "kernel": _short(name), "grid": grid, "bound": bound,
             "dispatches": len(dur), "mean_us": round(statistics.mean(dur), 3),
             "median_us": round(statistics.median(dur), 3)}
        f = _counter(out, f"FETCH_SIZE_{sec}", name, grid, "FETCH_SIZE")
        w = _counter(out, f"WRITE_SIZE_{sec}", name, grid, "WRITE_SIZE")
        if f is not None and w is not None:
            e.update({"fetch_kib": round(f, 1), "write_kib": round(w, 1),
                      "fetch_bytes": int(f * 1024 * fscale), "write_bytes": int(w * 1024 * wscale)})
            e["bytes"] = e["fetch_bytes"] + e["write_bytes"]
        if bound == "mfma":
            m = _counter(out, f"MfmaUtil_{sec}", name, grid, "MfmaUtil")
            if m is not None:
                e["mfma_util_pct"] = round(m, 1)
        kernels[key] = e
    doc = {"source_hash": source_hash(), "fetch_scale": round(fscale, 4),
           "write_scale": round(wscale, 4), "copy_fetch_kib": fetch_copy,
           "copy_write_kib": write_copy, "bench_args": BENCH_ARGS, "kernels": kernels}
    os.makedirs(dest, exist_ok=True)
    with open(os.path.join(dest, "traffic.json"), "w") as f:
        json.dump(doc, f, indent=1)
    _write_traffic_md(doc, dest)
    for sec in TRACE_SECTIONS:
        d = traces.get(sec) or _durations(out, sec)
        if d:
            _write_trace_md(sec, d, dest)
    return doc


def _copy_name(out, run):
    for r in _rows(os.path.join(out, run, "**", "*counter_collection.csv")):
        if "copyBuffer" in r["Kernel_Name"]:
            return r["Kernel_Name"]
    raise RuntimeError(f"no copy kernel in {run}")


def _copy_grid(out, run):
    grids = defaultdict(int)
    for r in _rows(os.path.join(out, run, "**", "*counter_collection.csv")):
        if "copyBuffer" in r["Kernel_Name"]:
            grids[int(r.get("Grid_Size") or 0)] += 1
    return max(grids, key=grids.get)


def _bench_cmd(sec: str) -> str:
    return f"python3 bench.py --only {sec} {' '.join(BENCH_ARGS)}"


def _write_traffic_md(doc: dict, dest: str) -> None:
    lines = [
        "# HBM traffic and matrix-core use of each configuration's main kernel",
        "",
        "Made by `python -m speculative_decoding_attention_amd.profiling collect OUT` on one "
        "MI355X, then `... profiling summarize OUT`.  Each pass is its own rocprofv3 run "
        "(from /tmp, TMPDIR=/tmp), one counter per run:",
        "",
        "```",
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/FETCH_SIZE_<section> -o p -- "
        "python3 bench.py --only <section> " + " ".join(BENCH_ARGS),
        "rocprofv3 --pmc WRITE_SIZE ... (the same, WRITE_SIZE)",
        "rocprofv3 --pmc MfmaUtil ... (sections c5 and std)",
        "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) ... -- python3 -c \"<256 MiB torch copy, "
        "three times>\"",
        "```",
        "",
        f"Calibration: the 256 MiB device copy reads FETCH_SIZE = {doc['copy_fetch_kib']:.1f} KiB "
        f"and WRITE_SIZE = {doc['copy_write_kib']:.1f} KiB per dispatch for 262144 KiB moved each "
        f"way, so fetch counts are scaled by {doc['fetch_scale']} and write counts by "
        f"{doc['write_scale']}.",
        "",
        "Main kernel of a configuration: the kernel of that name with the largest mean duration in "
        "the section's kernel trace; counters are the mean over its dispatches with the same "
        "grid (when one section launches the same kernel and grid for two calls of very "
        "different length, only the slow call's dispatches count).  Durations here are from the kernel trace (profiling adds little to a kernel's "
        "own duration; bench.py measures the same kernels live with the library's event hook).",
        "",
        "| configuration | kernel (grid) | mean us | fetched bytes | written bytes | traffic "
        "bytes | MFMA busy |",
        "|---|---|---|---|---|---|---|",
    ]
    for key, e in doc["kernels"].items():
        lines.append(f"| {key} | `{e['kernel']}` ({e['grid']}) | {e['mean_us']} | "
                     f"{e.get('fetch_bytes', '')} | {e.get('write_bytes', '')} | "
                     f"{e.get('bytes', '')} | "
                     f"{str(e['mfma_util_pct']) + ' %' if 'mfma_util_pct' in e else ''} |")
    lines += ["", f"Kernel source hash: {doc['source_hash']} (bench.py reports `traffic` only "
              "while the sources hash the same).", ""]
    with open(os.path.join(dest, "traffic.md"), "w") as f:
        f.write("\n".join(lines))


def _write_trace_md(sec: str, d: dict, dest: str) -> None:
    lines = [f"# Kernel durations, bench.py section `{sec}`", "",
             "Command (repository root; rocprofv3 from /tmp with TMPDIR=/tmp):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace_{sec} -o t -- "
             + _bench_cmd(sec), "```", "",
             "Per kernel and grid size (threads); durations in microseconds.  The counts include "
             "the eager warm-up calls before graph capture.  A kernel launched with the same "
             "grid by two calls of very different length is split into duration modes (runs of "
             "dispatches cut where one takes over twice or under half as long as the one before; "
             "runs with medians within a factor of two form a mode).", "",
             "| kernel | grid | dispatches | mean | median | min | max |",
             "|---|---|---|---|---|---|---|"]
    rows = sorted(d.items(), key=lambda kv: -sum(kv[1]))
    for (name, grid), v in rows[:24]:
        labels, n = _mode_labels(v)
        modes = [[t for t, lab in zip(v, labels) if lab == i] for i in range(n)]
        for i, m in enumerate(modes):
            tag = f" (mode {i + 1} of {n})" if n > 1 else ""
            lines.append(f"| `{_short(name)}`{tag} | {grid} | {len(m)} | {statistics.mean(m):.2f} | "
                         f"{statistics.median(m):.2f} | {min(m):.2f} | {max(m):.2f} |")
    lines.append("")
    with open(os.path.join(dest, f"kernels_{sec}.md"), "w") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("collect", "summarize"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "collect":
        sys.exit(collect(sys.argv[2], tuple(sys.argv[3:])))
    doc = summarize(sys.argv[2])
    print(json.dumps(doc["kernels"], indent=1))
