"""Host logic of the counter summaries: the main kernel of a configuration
is the slowest kernel of its name in the section's trace, and counter
values become bytes through the copy calibration."""
import csv
import json
import os

from speculative_decoding_attention_amd import profiling as P

TRACE_COLS = ["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_summary_picks_the_slowest_named_kernel_and_scales_counters(tmp_path):
    out = str(tmp_path / "raw")
    split = "void spec::(anonymous namespace)::attn_bf16_pipe_kernel<3, false>(spec::AttnArgs)"
    small = "void spec::(anonymous namespace)::attn_bf16_pipe_kernel<1, false>(spec::AttnArgs)"
    merge = "void spec::(anonymous namespace)::attn_merge_kernel<128>(spec::AttnArgs)"
    _write(f"{out}/trace_verify/x/t_kernel_trace.csv", TRACE_COLS, [
        (split, 126976, 0, 15000), (split, 126976, 0, 17000),     # 15 and 17 us
        (small, 4096, 0, 9000), (merge, 172032, 0, 4000)])
    copy = "__amd_rocclr_copyBuffer"
    _write(f"{out}/FETCH_SIZE_copy/x/p_counter_collection.csv", PMC_COLS,
           [(copy, 131072, "FETCH_SIZE", 131072.0, 0, 9000)] * 3)   # half the bytes counted
    _write(f"{out}/WRITE_SIZE_copy/x/p_counter_collection.csv", PMC_COLS,
           [(copy, 131072, "WRITE_SIZE", 262144.0, 0, 9000)] * 3)
    _write(f"{out}/FETCH_SIZE_verify/x/p_counter_collection.csv", PMC_COLS, [
        (split, 126976, "FETCH_SIZE", 25000.0, 0, 15000), (split, 126976, "FETCH_SIZE", 27000.0, 0, 16000),
        (small, 4096, "FETCH_SIZE", 999.0, 0, 9000)])
    _write(f"{out}/WRITE_SIZE_verify/x/p_counter_collection.csv", PMC_COLS, [
        (split, 126976, "WRITE_SIZE", 5000.0, 0, 15000)])
    dest = str(tmp_path / "profiles")
    doc = P.summarize(out, dest)
    e = doc["kernels"]["c2_verify_split"]
    assert e["grid"] == 126976 and e["dispatches"] == 2 and e["mean_us"] == 16.0
    assert doc["fetch_scale"] == 2.0 and doc["write_scale"] == 1.0
    assert e["fetch_bytes"] == 26000 * 1024 * 2 and e["write_bytes"] == 5000 * 1024
    assert e["bytes"] == e["fetch_bytes"] + e["write_bytes"]
    assert set(doc["kernels"]) == {"c2_verify_split"}          # no other section traced
    on_disk = json.load(open(os.path.join(dest, "traffic.json")))
    assert on_disk["source_hash"] == P.source_hash()
    assert os.path.exists(os.path.join(dest, "traffic.md"))
    assert os.path.exists(os.path.join(dest, "kernels_verify.md"))


def test_a_kernel_shared_by_two_calls_counts_the_slow_one(tmp_path):
    """The paged verification and the paged text-anchored attention launch
    the same kernel with the same grid; the main kernel is the slow call."""
    out = str(tmp_path / "raw")
    k = "void spec::(anonymous namespace)::attn_bf16_pipe_kernel<4, true>(spec::AttnArgs)"
    _write(f"{out}/trace_c3/x/t_kernel_trace.csv", TRACE_COLS,
           [(k, 131072, 0, 130000), (k, 131072, 0, 14000), (k, 131072, 0, 136000),
            (k, 131072, 0, 13000)])
    copy = "__amd_rocclr_copyBuffer"
    for ctr, v in (("FETCH_SIZE", 262144.0), ("WRITE_SIZE", 262144.0)):
        _write(f"{out}/{ctr}_copy/x/p_counter_collection.csv", PMC_COLS,
               [(copy, 131072, ctr, v, 0, 1000)])
    cols = PMC_COLS
    _write(f"{out}/FETCH_SIZE_c3/x/p_counter_collection.csv", cols,
           [(k, 131072, "FETCH_SIZE", 550000.0, 0, 140000), (k, 131072, "FETCH_SIZE", 9000.0, 0, 15000)])
    _write(f"{out}/WRITE_SIZE_c3/x/p_counter_collection.csv", cols,
           [(k, 131072, "WRITE_SIZE", 12000.0, 0, 140000), (k, 131072, "WRITE_SIZE", 900.0, 0, 15000)])
    e = P.summarize(out, str(tmp_path / "profiles"))["kernels"]["c3_verify_paged_split"]
    assert e["dispatches"] == 2 and e["mean_us"] == 133.0
    assert e["fetch_bytes"] == 550000 * 1024 and e["write_bytes"] == 12000 * 1024
