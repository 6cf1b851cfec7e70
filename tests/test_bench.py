"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte and flop counts
the roofline divides by, and the profile summaries' counter scaling."""
import csv
import json
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_algorithmic_counts_by_hand():
    # request 0: prefix 70, two kept tokens; request 1: nothing kept (moves nothing)
    st = types.SimpleNamespace(prefix_len=np.array([70, 5]), blk=32, Hkv=2, d=64, Hq=4, S=64)
    by, fl = bench.attn_algorithmic(st, np.array([2, 0]))
    kv = (70 + 32) * 2 * 64 * 2 * 2          # prefix + block K and V, bf16
    qo = 2 * 4 * 64 * 2 * 2                  # kept queries and outputs
    lse = 2 * 4 * 4
    table = 4 * 2 + 8                        # two page ids, prefix length and offset
    assert by == kv + qo + lse + table
    assert fl == 4 * 2 * 4 * (70 + 32) * 64


def test_score_algorithmic_counts_by_hand():
    st = types.SimpleNamespace(B=3, blk=16, Hq=4, Hkv=2, d=64, score_dtype="bf16")
    by, fl = bench.score_algorithmic(st)
    assert by == 2 * 3 * 16 * (4 + 2) * 64 * 2 + 4 * 3 * 16
    assert fl == 2 * 2 * 3 * 16 * 16 * 4 * 64
    st.score_dtype = "f32"
    assert bench.score_algorithmic(st)[0] == 2 * 3 * 16 * (4 + 2) * 64 * 4 + 4 * 3 * 16


def _write_pmc(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows):
            w.writerow([i, name, counter, value])


def test_profile_summary_scales_counters_by_the_copy(tmp_path, monkeypatch):
    out = tmp_path / "out"
    attn = ("void focus::(anonymous namespace)::attn_kernel<128, 1, 2, true, false, true>"
            "(focus::Params, int const*)")
    copy = "__amd_rocclr_copyBuffer(void*)"
    w = out / "sdar_b256_blk32"
    # the copy of 1 GiB reads as half its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    _write_pmc(out / "calib" / "fetch", "FETCH_SIZE", [(copy, 524288.0), (copy, 12.0)])
    _write_pmc(out / "calib" / "write", "WRITE_SIZE", [(copy, 1048576.0)])
    _write_pmc(w / "fetch", "FETCH_SIZE", [(attn, 1000.0), (attn, 3000.0), (attn, 2000.0)])
    _write_pmc(w / "write", "WRITE_SIZE", [(attn, 10.0)])
    # MFMA: busy cycles over (active cycles of one XCD x 1024 SIMDs); bf16 work in 512-flop units
    os.makedirs(w / "mfma")
    with open(w / "mfma" / "run_counter_collection.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writerow([0, attn, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000 * 0.25])
        wr.writerow([0, attn, "GRBM_GUI_ACTIVE", 8 * 1000])     # summed over the 8 XCDs
        wr.writerow([0, attn, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0e6])
    os.makedirs(w / "trace")
    with open(w / "trace" / "run_kernel_stats.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        wr.writerow([attn, 3, 150000, 140000, 160000, 80.0])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h")
    bench.summarize_profiles(str(out), "sdar_b256_blk32")
    rec = json.load(open(tmp_path / "profiles" / "attn_traffic_sdar_b256_blk32.json"))
    assert rec["kernel"] == "attn_kernel<128, 1, 2, true, false, true>"
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert rec["hbm_read_bytes"] == 2000 * 1024 * 2
    assert rec["hbm_write_bytes"] == 10 * 1024
    assert abs(rec["mfma_busy_frac"] - 0.25) < 1e-9
    assert rec["mfma_bf16_flops_per_launch"] == 2.0e6 * 512
    assert rec["trace_avg_us"] == 150.0
    table = open(tmp_path / "profiles" / "kernels_sdar_b256_blk32.txt").read()
    assert "attn_kernel<128, 1, 2, true, false, true>" in table and "150.00" in table


def test_focused_attention_instantiation_per_recipe():
    from workloads import BY_NAME
    # the focused step reads its queries in place (the last template argument)
    one_wave = {"sdar_b256_blk32": "attn_kernel<128, 1, 2, true, false, true>",
                "sdar_b32_blk32": "attn_kernel<128, 2, 2, true, false, true>",
                "longctx_b64_blk32": "attn_kernel<128, 1, 2, true, false, true>",
                "tiny_b2_blk16": "attn_kernel<64, 1, 2, true, false, true>"}
    # the adaptive recipes' launch bound is 16 kept tokens x 4 query heads = 64 rows: shared
    shared = {"sweep_b128_blk64": "attn_kernel<128, 1, 3, true, true, true>",
              "sweep_b128_blk16": "attn_kernel<128, 1, 3, true, true, true>"}
    for name, want in {**one_wave, **shared}.items():
        assert bench.focused_attn_kernel(BY_NAME[name]) == want, name


def test_host_cpu_description():
    cpu = bench.host_cpu()
    assert cpu["logical_cpus"] >= 1 and 1 <= cpu["physical_cores"] <= cpu["logical_cpus"]
    assert 1 <= cpu["workers"] <= cpu["logical_cpus"] and cpu["model"]


def test_counter_traffic_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    with open(tmp_path / "profiles" / "attn_traffic_w.json", "w") as fh:
        json.dump({"kernel_source_hash": "abc", "hbm_bytes_per_launch": 123}, fh)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.counter_traffic("w") == 123
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.counter_traffic("w") is None
    assert bench.counter_traffic("other") is None
