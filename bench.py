"""Throughput of the focused block-diffusion step on one MI355X.

A step is one pass of the whole hot path over one batch: importance scoring (layer 1 minus
layer 0), budgeted top-k selection, compaction + gather of the hidden states and of the
attention queries, and ragged paged attention over each request's paged prefix plus block KV.
Inputs are seeded synthetic tensors already resident in HBM.  One JSON line is printed.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_algorithmic(st, kept):
    """Bytes and flops the attention must move/do: per request with k_r > 0, its whole prefix
    plus block K and V once, its queries, outputs, LSE, page-table entries and two ints."""
    P = st.prefix_len.astype(np.int64)
    k = kept.astype(np.int64)
    act = k > 0
    kv = ((P + st.blk) * st.Hkv * st.d * 2 * 2)[act].sum()
    qo = (k * st.Hq * st.d * 2 * 2).sum()
    ls = (k * st.Hq * 4).sum()
    tab = (4 * ((P + st.S - 1) // st.S))[act].sum() + 8 * act.sum()
    flops = (4 * k * st.Hq * (P + st.blk) * st.d).sum()
    return int(kv + qo + ls + tab), int(flops)


def score_algorithmic(st):
    es = 4 if st.score_dtype == "f32" else 2
    by = 2 * st.B * st.blk * (st.Hq + st.Hkv) * st.d * es + 4 * st.B * st.blk
    fl = 2 * 2 * st.B * st.blk * st.blk * st.Hq * st.d
    return by, fl


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("attn.hip", "device_common.h"):
        with open(os.path.join(ROOT, "decodability_aware_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"attn_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(recipe, budget_s):
    """The fp64 oracle timed on a bounded sample of the same workload (batches of 16 requests
    drawn from the same distributions, new seeds each batch, until about budget_s seconds of
    oracle time), scaled to focused tokens per second."""
    import oracle
    from workloads import make_step
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    Bs = 16
    total_t, total_tok, reqs = 0.0, 0, 0
    seed = recipe.seed
    while total_t < budget_s:
        st = make_step(recipe.scaled(B=Bs), seed=seed)
        t0 = time.perf_counter()
        res = oracle.step(st)
        total_t += time.perf_counter() - t0
        total_tok += int(res["offsets"][-1])
        reqs += Bs
        seed += 1
    return {"value": total_tok / total_t, "unit": "focused tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reqs} requests of {recipe.name} in batches of {Bs} (seeds {recipe.seed}.."
                      f"{seed - 1}), full step score+select+compact+attend in fp64, "
                      f"{total_t:.1f} s of oracle time"}


# ------------------------------------------------------------------------------------------
# profile summaries (run on the CSV output of the rocprofv3 commands listed in PROFILE_CMDS)
# ------------------------------------------------------------------------------------------
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof -o trace "
             "-- python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline",
    "step_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc/step_fetch "
                  "-o run -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
    "step_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc/step_write "
                  "-o run -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc/copy_fetch "
                  "-o run -- python3 bench.py --calibrate",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc/copy_write "
                  "-o run -- python3 bench.py --calibrate",
}


def _find(root, pattern):
    import glob
    hits = sorted(glob.glob(os.path.join(root, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"{pattern} under {root}")
    return hits[0]


def _short(name):
    import re
    m = re.search(r"::(\w+)(<[^(]*>)?\(", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    m = re.search(r"\w+", name)
    return m.group(0) if m else name[:60]


def _counter_per_dispatch(root, counter):
    """{kernel short name: [value per dispatch]} from a rocprofv3 --pmc CSV."""
    import csv
    vals = {}
    with open(_find(root, "*counter_collection.csv")) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(_short(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    return vals


def summarize_profiles(out_root, workload):
    """Writes profiles/kernels_<workload>.txt (kernel-trace statistics) and
    profiles/attn_traffic_<workload>.{json,txt} (HBM bytes per attention launch from FETCH_SIZE /
    WRITE_SIZE, each scaled by what the counter reads for a 1 GiB device copy)."""
    import csv
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    rows = list(csv.DictReader(open(_find(os.path.join(out_root, "prof"), "*kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics, workload {workload}",
             f"# command: {PROFILE_CMDS['trace']}",
             f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{_short(r['Name'])[:72]:72s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    with open(os.path.join(prof, f"kernels_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    pmc = os.path.join(out_root, "pmc")
    med = lambda v: sorted(v)[len(v) // 2]
    gib = float(1 << 30)
    cf = _counter_per_dispatch(os.path.join(pmc, "copy_fetch"), "FETCH_SIZE")
    cw = _counter_per_dispatch(os.path.join(pmc, "copy_write"), "WRITE_SIZE")
    # the calibration copy is the one dispatch whose byte counts are near 1 GiB
    copy_f = max(max(v) for v in cf.values()) * 1024.0
    copy_w = max(max(v) for v in cw.values()) * 1024.0
    f_fac, w_fac = gib / copy_f, gib / copy_w
    sf = _counter_per_dispatch(os.path.join(pmc, "step_fetch"), "FETCH_SIZE")
    sw = _counter_per_dispatch(os.path.join(pmc, "step_write"), "WRITE_SIZE")
    key = next(k for k in sf if k.startswith("attn_kernel"))
    fetch = med(sf[key]) * 1024.0 * f_fac
    write = med(sw[key]) * 1024.0 * w_fac
    rec = {"workload": workload, "kernel": key, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": med(sf[key]), "write_kib_per_dispatch": med(sw[key]),
           "fetch_scale": f_fac, "write_scale": w_fac,
           "hbm_bytes_per_launch": int(round(fetch + write)),
           "hbm_read_bytes": int(round(fetch)), "hbm_write_bytes": int(round(write)),
           "commands": [PROFILE_CMDS[k] for k in ("step_fetch", "step_write", "copy_fetch",
                                                  "copy_write")]}
    with open(os.path.join(prof, f"attn_traffic_{workload}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    txt = [f"# HBM traffic of {key}, workload {workload}",
           *[f"# command: {c}" for c in rec["commands"]],
           f"copy calibration: 1 GiB copy reads as FETCH_SIZE {copy_f / 1024:.0f} KiB "
           f"(scale {f_fac:.3f}), WRITE_SIZE {copy_w / 1024:.0f} KiB (scale {w_fac:.3f})",
           f"attention per launch: FETCH_SIZE {med(sf[key]):.0f} KiB -> {fetch / 1e6:.1f} MB read; "
           f"WRITE_SIZE {med(sw[key]):.0f} KiB -> {write / 1e6:.1f} MB written; "
           f"total {(fetch + write) / 1e6:.1f} MB"]
    with open(os.path.join(prof, f"attn_traffic_{workload}.txt"), "w") as fh:
        fh.write("\n".join(txt) + "\n")
    print("\n".join(lines + txt))


def full_block_pass(inp, st, args, stream):
    """The unfocused baseline on the same kernels (every block token a query), timed like the
    focused step: its attention launch by HIP events, the step by graph replays."""
    import torch
    from decodability_aware_token_amd import FullBlockStep
    fb = FullBlockStep(inp)
    for _ in range(args.warmup):
        fb.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fb.run()
    e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = e0.elapsed_time(e1) / args.steps
    kept = np.full(st.B, st.blk)
    nbytes, flops = attn_algorithmic(st, kept)
    rows = st.B * st.blk
    log(f"[bench] full-block step: attention over {rows} rows {attn_ms * 1000:.1f} us, "
        f"{nbytes / (attn_ms * 1e-3) / 1e9:.0f} GB/s, {flops / (attn_ms * 1e-3) / 1e12:.1f} TFLOP/s")
    return {"rows": rows, "attn_us": round(attn_ms * 1000, 2),
            "block_tokens_per_s": rows / (attn_ms * 1e-3),
            "attn_algorithmic_bytes": nbytes, "attn_flops": flops,
            "attn_hbm_frac": round(nbytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "attn_mfma_frac": round(flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def full_domain_pass(inp, t, st, args, stream):
    """Importance over the full attention domain: the score kernel with each block query's
    prefix+block log-sum-exp given (its own roofline), and the two layers' attentions that
    produce those LSEs here (in a model they come with layers 0 and 1)."""
    import torch
    from decodability_aware_token_amd import FullDomainScore
    fd = FullDomainScore(inp, t["k_cache0"], t["k_blk0"])
    for _ in range(args.warmup):
        fd.run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(args.steps):
        fd.layer_lse()
    ev[1].record(stream)
    for _ in range(args.steps):
        fd.score()
    ev[2].record(stream)
    torch.cuda.synchronize()
    lse_ms = ev[0].elapsed_time(ev[1]) / args.steps
    sc_ms = ev[1].elapsed_time(ev[2]) / args.steps
    sb, sf = score_algorithmic(st)
    sb += 2 * st.B * st.blk * st.Hq * 4  # the two LSE arrays
    log(f"[bench] full-domain score: {sc_ms * 1000:.1f} us ({sb / (sc_ms * 1e-3) / 1e9:.0f} GB/s); "
        f"the two layers' LSE attentions {lse_ms * 1000:.1f} us")
    return {"score_lse_us": round(sc_ms * 1000, 2), "score_lse_algorithmic_bytes": sb,
            "score_lse_hbm_frac": round(sb / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "layer_lse_attention_us": round(lse_ms * 1000, 2)}


def kv_pass(fs, inp, st, args, stream):
    """Intra-block KV write-back of the kept rows (fresh K/V stand-ins: the gathered Q rows'
    first Hkv heads) and the commit of every request's block into its paged prefix, each timed
    by HIP events; the commit runs on a copy of the caches extended by free pages."""
    import torch
    from decodability_aware_token_amd import binding as F
    dev = inp.q_att.device
    T = int(fs.offsets[-1])
    rows = fs.q_rows[:, : st.Hkv].contiguous()        # [cap, Hkv, d] bf16
    kb, vb = inp.k_blk.clone(), inp.v_blk.clone()
    S = st.S
    extra = st.B * (-(-st.blk // S) + 1)
    kc = torch.cat([inp.k_cache, torch.zeros((extra,) + tuple(inp.k_cache.shape[1:]),
                                             dtype=inp.k_cache.dtype, device=dev)])
    vc = torch.cat([inp.v_cache, torch.zeros((extra,) + tuple(inp.v_cache.shape[1:]),
                                             dtype=inp.v_cache.dtype, device=dev)])
    cols = int((st.prefix_len.max() + st.blk + S - 1) // S)
    pt = torch.full((st.B, max(cols, inp.page_table.shape[1])), -1, dtype=torch.int32, device=dev)
    pt[:, : inp.page_table.shape[1]] = inp.page_table
    free = torch.arange(inp.k_cache.shape[0], inp.k_cache.shape[0] + extra, dtype=torch.int32,
                        device=dev)
    commit = torch.ones(st.B, dtype=torch.uint8, device=dev)
    pl_out = torch.empty_like(inp.prefix_len)
    fc_in = torch.tensor([extra], dtype=torch.int32, device=dev)
    fc_out = torch.empty_like(fc_in)
    status = torch.empty_like(fc_in)
    wb = lambda: F.kv_writeback(rows, rows, fs.offsets, fs.kept_pos, kb, vb)
    cm = lambda: F.block_commit(commit, kb, vb, kc, vc, pt, inp.prefix_len, pl_out, free, fc_in,
                                fc_out, status)
    for _ in range(args.warmup):
        wb()
        cm()
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(args.steps):
        wb()
    ev[1].record(stream)
    for _ in range(args.steps):
        cm()
    ev[2].record(stream)
    torch.cuda.synchronize()
    wb_ms = ev[0].elapsed_time(ev[1]) / args.steps
    cm_ms = ev[1].elapsed_time(ev[2]) / args.steps
    wb_bytes = 2 * 2 * T * st.Hkv * st.d * 2 + 4 * (T + st.B + 1)
    cm_bytes = 2 * 2 * st.B * st.blk * st.Hkv * st.d * 2 + 16 * st.B
    log(f"[bench] kv write-back {wb_ms * 1000:.1f} us ({wb_bytes / (wb_ms * 1e-3) / 1e9:.0f} GB/s)"
        f"; block commit {cm_ms * 1000:.1f} us ({cm_bytes / (cm_ms * 1e-3) / 1e9:.0f} GB/s)")
    return {"writeback_us": round(wb_ms * 1000, 2), "writeback_bytes": wb_bytes,
            "commit_us": round(cm_ms * 1000, 2), "commit_bytes": cm_bytes,
            "commit_hbm_frac": round(cm_bytes / (cm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sdar_b256_blk32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-domain", action="store_true",
                    help="skip the full-domain importance measurement")
    ap.add_argument("--no-full-block", action="store_true",
                    help="skip the unfocused (every block token kept) comparison step")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager launches instead of HIP graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--summarize-profiles", metavar="OUT_ROOT",
                    help="write the profiles/ summaries from the CSV output of the rocprofv3 "
                         "commands in PROFILE_CMDS (OUT_ROOT is the folder that holds their -d output)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known bytes) 5 times, "
                         "to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the step would shard "
              "by request, each GPU running the whole step on its share).", file=sys.stderr)
        sys.exit(2)

    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    import torch
    if args.calibrate:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "ms": ms, "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}))
        return
    from decodability_aware_token_amd import FocusStep, StepInputs
    from workloads import BY_NAME, make_step
    from workloads.torch_io import upload

    recipe = BY_NAME[args.workload]
    log(f"[bench] generating {recipe.name}")
    st = make_step(recipe, layer0_prefix=not args.no_full_domain)
    dev = torch.device("cuda:0")
    t = upload(st, dev)
    inp = StepInputs(**{k: t[k] for k in ("q0", "k0", "q1", "k1", "masked", "budget", "adaptive",
                                           "max_kept", "q_att", "k_cache", "v_cache",
                                           "page_table", "prefix_len", "k_blk", "v_blk",
                                           "sm_scale", "hidden")})
    fs = FocusStep(inp)
    stream = torch.cuda.current_stream(dev)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        fs.run()
    torch.cuda.synchronize()

    # Pass 1 (eager, per-stage HIP events on the launch stream): the stage breakdown and the
    # attention kernel's launch duration for the roofline.
    stages = fs.front_stages + ("attend",)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    log(f"[bench] eager pass: {args.steps} steps with per-stage events")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, name in enumerate(stages):
            getattr(fs, name)()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    per_stage = np.zeros(len(stages))
    step_ms = np.zeros(args.steps)
    for i in range(args.steps):
        for j in range(len(stages)):
            per_stage[j] += ev[i][j].elapsed_time(ev[i][j + 1])
        step_ms[i] = ev[i][0].elapsed_time(ev[i][-1])
    per_stage /= args.steps
    eager_ms = eager_wall * 1000.0 / args.steps

    # Pass 2 (the measured step): the whole step (score partials, reduction + selection +
    # compaction of the hidden states and queries, attention) captured once in a HIP graph, W
    # untimed replays, then exactly K replays between device synchronisations.
    ms_per_step = eager_ms
    mode = "eager"
    if not args.no_graph:
        fs.capture()
        for _ in range(args.warmup):
            fs.replay()
        log(f"[bench] graph pass: {args.steps} replays")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fs.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1000.0 / args.steps
        mode = "hip graph"

    offsets = fs.offsets.cpu().numpy()
    kept = np.diff(offsets)
    T = int(offsets[-1])
    attn_bytes, attn_flops = attn_algorithmic(st, kept)
    attn_ms = per_stage[stages.index("attend")]
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    sb, sf = score_algorithmic(st)
    for j, name in enumerate(stages):
        log(f"[bench] {name:15s} {per_stage[j] * 1000:9.1f} us")
    log(f"[bench] eager step (events) {step_ms.mean() * 1000:.1f} us median "
        f"{np.median(step_ms) * 1000:.1f} us; eager wall {eager_ms * 1000:.1f} us; "
        f"{mode} wall {ms_per_step * 1000:.1f} us; T={T}")
    log(f"[bench] attention {attn_bytes / 1e6:.1f} MB algorithmic -> {achieved:.0f} GB/s "
        f"({achieved / PEAK_HBM_GBS * 100:.1f}% of HBM), "
        f"{attn_flops / (attn_ms * 1e-3) / 1e12:.2f} TFLOP/s")
    sc_ms = per_stage[0]
    log(f"[bench] {stages[0]}: score inputs {sb / 1e6:.1f} MB -> "
        f"{sb / (sc_ms * 1e-3) / 1e9:.0f} GB/s, {sf / (sc_ms * 1e-3) / 1e12:.2f} TFLOP/s")

    full = None
    if not args.no_full_block:
        full = full_block_pass(inp, st, args, stream)
    fdom = None
    if not args.no_full_domain:
        fdom = full_domain_pass(inp, t, st, args, stream)
    kvres = kv_pass(fs, inp, st, args, stream)

    res = {
        "metric": "focused block-tokens/s per diffusion step",
        "value": T / (ms_per_step * 1e-3),
        "unit": "focused tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no weights or datasets)",
        "config": {
            "workload": recipe.name, "global_batch": st.B, "block": st.blk, "Hq": st.Hq,
            "Hkv": st.Hkv, "head_dim": st.d, "page": st.S,
            "prefix": f"{recipe.prefix}", "budget": f"{recipe.budget}",
            "hidden": recipe.hidden, "kept_tokens": T, "block_tokens": st.B * st.blk,
            "block_tokens_per_s": st.B * st.blk / (ms_per_step * 1e-3),
            "stage_us": {n: round(per_stage[j] * 1000, 2) for j, n in enumerate(stages)},
            "step_launch": mode, "eager_ms_per_step": round(eager_ms, 5),
            "full_block_step": full,
            "full_domain_score": fdom,
            "kv_cache": kvres,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "ragged paged attention (focus_ragged_paged_attn)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": counter_traffic(recipe.name),
            "algorithmic_bytes_per_launch": attn_bytes,
            "avg_launch_us": round(attn_ms * 1000, 2),
            "mfma_util": round(attn_flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
        },
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        res["cpu_baseline"] = cpu_baseline(recipe, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
