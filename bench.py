"""Throughput of the focused block-diffusion step on one MI355X.

A step is one pass of the whole hot path over one batch: importance scoring (layer 1 minus
layer 0), budgeted top-k selection, compaction + gather of the hidden states, and ragged paged
attention of the kept tokens (their queries read in place at the kept positions) over each
request's paged prefix plus block KV.
Inputs are seeded synthetic tensors already resident in HBM.  One JSON line is printed.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-graph]
                    [--no-flush] [--only-step]

Each timed step is preceded by a cache flush (a 1 GiB read, outside the timed events), so no
input of the step is served from the 256 MB Infinity Cache or the L2s.
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


def code_only(text):
    """Source text without its comments and blank space: what a comment edit leaves unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the attention kernel's code (comments and spacing excluded)."""
    h = hashlib.sha256()
    for f in ("attn.hip", "device_common.h"):
        with open(os.path.join(ROOT, "decodability_aware_token_amd", "csrc", f)) as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_record(workload):
    """The committed rocprofv3 counter record of the focused step's attention (HBM bytes per
    launch, MFMA busy fraction), if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"attn_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec


def counter_traffic(workload):
    """HBM bytes per attention launch from the counter record (None if absent or stale)."""
    rec = counter_record(workload)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def host_cpu():
    """CPU model, logical CPUs this process may run on, physical cores among them, and the
    worker count the oracle's pool uses (capped by OMP_NUM_THREADS where the host sets it)."""
    model = "unknown"
    phys = set()
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else \
        list(range(os.cpu_count() or 1))
    try:
        proc, core, pkg = None, None, None
        with open("/proc/cpuinfo") as fh:
            for line in fh.read().splitlines() + [""]:
                if line.startswith("model name") and model == "unknown":
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("processor"):
                    proc = int(line.split(":")[1])
                elif line.startswith("physical id"):
                    pkg = line.split(":")[1].strip()
                elif line.startswith("core id"):
                    core = line.split(":")[1].strip()
                elif not line.strip() and proc is not None:
                    if proc in allowed:
                        phys.add((pkg, core))
                    proc, core, pkg = None, None, None
    except OSError:  # pragma: no cover
        pass
    logical = len(allowed)
    physical = len(phys) if phys else logical
    workers = logical
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        workers = max(1, min(workers, int(os.environ["OMP_NUM_THREADS"])))
    return {"model": model, "logical_cpus": logical, "physical_cores": physical,
            "workers": workers}


def _oracle_batch(name, B, seed, threads):
    """One oracle step on a batch of the recipe: (focused tokens, seconds)."""
    from threadpoolctl import threadpool_limits
    import oracle
    from workloads import BY_NAME, make_step
    st = make_step(BY_NAME[name].scaled(B=B), seed=seed)
    with threadpool_limits(threads):
        t0 = time.perf_counter()
        res = oracle.step(st)
        dt = time.perf_counter() - t0
    return int(res["offsets"][-1]), dt


def oracle_worker(name, B, seed, stride, seconds):
    """A pool worker (a child process of its own, importing no GPU library): single-threaded
    oracle steps on batches seed, seed + stride, ... until `seconds` of oracle time; prints one
    JSON line with its totals."""
    tok, t, n = 0, 0.0, 0
    while t < seconds:
        k, dt = _oracle_batch(name, B, seed + n * stride, 1)
        tok, t, n = tok + k, t + dt, n + 1
    print(json.dumps({"tokens": tok, "seconds": t, "batches": n}), flush=True)


def cpu_baseline(recipe, budget_s):
    """The fp64 oracle as it stands, timed on the host's cores on bounded samples of the
    workload (batches of 16 requests drawn from the same recipe with new seeds), scaled to
    focused tokens per second:
      * pool: one single-threaded oracle process per worker, all running at once, each for
        about budget_s seconds of oracle time (the reported value: the sum of the workers'
        rates, each its tokens over its own oracle time -- input generation is not timed);
      * threaded: one process with the BLAS library's threads, about budget_s / 3 seconds;
      * single_core: the tiny and the 32-request recipes' whole steps on one thread."""
    import subprocess
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle
    from workloads import BY_NAME, make_step
    cpu = host_cpu()
    Bs = 16
    n = cpu["workers"]
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    t0 = time.perf_counter()
    procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--oracle-worker",
                               recipe.name, str(Bs), str(recipe.seed + 1 + i), str(n),
                               str(budget_s)], stdout=subprocess.PIPE, text=True, env=env)
             for i in range(n)]
    rows = []
    for p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"oracle worker failed ({p.returncode})")
        rows.append(json.loads(out.strip().splitlines()[-1]))
    wall = time.perf_counter() - t0
    rate = sum(r["tokens"] / r["seconds"] for r in rows)
    batches = sum(r["batches"] for r in rows)
    busy = sum(r["seconds"] for r in rows)
    # threaded: the BLAS library's own threads in one process
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    th_t, th_tok, th_seed = 0.0, 0, recipe.seed + 1 + n * max(r["batches"] for r in rows)
    while th_t < budget_s / 3:
        k, dt = _oracle_batch(recipe.name, Bs, th_seed, None)
        th_t, th_tok, th_seed = th_t + dt, th_tok + k, th_seed + 1
    # single core: whole steps of the small recipes
    single = {}
    for name in ("tiny_b2_blk16", "sdar_b32_blk32"):
        st = make_step(BY_NAME[name])
        with threadpool_limits(1):
            t1 = time.perf_counter()
            res = oracle.step(st)
            dt = time.perf_counter() - t1
        single[name] = {"focused_tokens": int(res["offsets"][-1]), "seconds": round(dt, 4),
                        "focused_tokens_per_s": round(int(res["offsets"][-1]) / dt, 1)}
    return {"value": rate, "unit": "focused tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{batches} batches of {Bs} requests of {recipe.name} (new seeds from "
                      f"{recipe.seed + 1}), full step score+select+compact+attend in fp64, "
                      f"{n} single-threaded oracle processes at once, {busy:.1f} s of oracle "
                      f"time in {wall:.1f} s wall",
            "cpu_model": cpu["model"], "logical_cpus": cpu["logical_cpus"],
            "physical_cores": cpu["physical_cores"],
            "threaded": {"value": th_tok / th_t, "blas_threads": int(threads),
                         "seconds": round(th_t, 1)},
            "single_core": single}


# ------------------------------------------------------------------------------------------
# profile summaries (from the CSV output of the rocprofv3 commands of profile_commands())
# ------------------------------------------------------------------------------------------
SIMD_NUM = 256 * 4   # MI355X: 256 compute units of 4 SIMDs (MFMA-busy normalisation)
NUM_XCC = 8          # MI355X: 8 accelerator complex dies, each with its own GRBM counter
PROF_OUT = "gpurun_out/prof"


def _bench_cmd(workload, steps, warmup, only_step):
    cmd = (f"python3 bench.py --workload {workload} --steps {steps} --warmup {warmup} "
           "--no-cpu-baseline")
    return cmd + (" --only-step" if only_step else "")


def profile_commands(workload, out=PROF_OUT):
    """The rocprofv3 runs behind the profiles/ summaries of one workload, in order.  Counter
    runs (one per counter group) time the focused step only; the copy calibration is shared."""
    w = f"{out}/{workload}"
    cmds = {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {w}/trace -o run -- "
                 + _bench_cmd(workload, 20, 5, True),
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {w}/fetch -o run -- "
                 + _bench_cmd(workload, 5, 2, True),
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {w}/write -o run -- "
                 + _bench_cmd(workload, 5, 2, True),
        "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                f"GRBM_GUI_ACTIVE --output-format csv -d {w}/mfma -o run -- "
                + _bench_cmd(workload, 5, 2, True),
        "trace_all": f"rocprofv3 --kernel-trace --stats --output-format csv -d {w}/trace_all "
                     "-o run -- " + _bench_cmd(workload, 10, 3, False),
    }
    return cmds


def calibration_commands(out=PROF_OUT):
    return {
        "copy_fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/calib/fetch -o run "
                      "-- python3 bench.py --calibrate",
        "copy_write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/calib/write -o run "
                      "-- python3 bench.py --calibrate",
    }


def _find(root, pattern):
    import glob
    hits = sorted(glob.glob(os.path.join(root, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"{pattern} under {root}")
    return hits[0]


def _short(name):
    """A kernel's name without return type, namespaces and parameter list: the identifier (and
    template arguments) before the first parenthesis outside template brackets."""
    name = name.replace("(anonymous namespace)", "anon")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    head = name[:cut].strip()
    if head.startswith("void "):
        head = head[5:]
    depth, start = 0, 0
    for i, ch in enumerate(head):      # last "::" outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and head[i:i + 2] == "::":
            start = i + 2
    return head[start:] or name[:60]


def _counters_per_dispatch(root):
    """{kernel short name: {counter: [value per dispatch]}} from a rocprofv3 --pmc CSV."""
    import csv
    vals = {}
    with open(_find(root, "*counter_collection.csv")) as fh:
        for row in csv.DictReader(fh):
            d = vals.setdefault(_short(row["Kernel_Name"]), {})
            d.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return vals


FRONT_KERNELS = ("score_partial_kernel", "score_reduce_kernel", "select_compact_kernel",
                 "select_kernel", "compact_kernel", "compact_scan_kernel")


def focused_attn_kernel(recipe):
    """Name of the attention instantiation the focused step of a recipe launches, as the launch
    plan chooses it: <d, query tiles per wave, tiles in flight, output, shared tiles, queries
    read in place>.  Items of 33..128 rows share each tile among a workgroup's four waves (16
    rows per wave up to 64, 32 rows above); the others run one wave per item."""
    rows = recipe.max_kept() * recipe.G
    if 32 < rows <= 128:
        qt = 1 if rows <= 64 else 2
        return f"attn_kernel<{recipe.d}, {qt}, 3, true, true, true>"
    qt = 1 if rows <= 16 else (2 if rows <= 32 else 4)
    return f"attn_kernel<{recipe.d}, {qt}, 2, true, false, true>"


def _kernel_table(csv_path, title, command):
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics, {title}", f"# command: {command}",
             f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{_short(r['Name'])[:72]:72s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    return lines, {_short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in rows}


def summarize_profiles(out_root, workload):
    """Writes, from the output of profile_commands(workload) and calibration_commands():
      * profiles/kernels_<workload>.txt: kernel statistics of the focused step (and, when run,
        of every pass of the bench);
      * profiles/attn_traffic_<workload>.{json,txt}: HBM bytes per launch of the focused step's
        attention from FETCH_SIZE / WRITE_SIZE (median over dispatches), each scaled by what the
        counter reads for a 1 GiB device copy, and its MFMA busy fraction
        SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs) with the bf16 MFMA work
        SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 flops."""
    from workloads import BY_NAME
    recipe = BY_NAME[workload]
    cmds = profile_commands(workload)
    cal = calibration_commands()
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    w = os.path.join(out_root, workload)
    lines, avg = _kernel_table(_find(os.path.join(w, "trace"), "*kernel_stats.csv"),
                               f"focused step only, workload {workload}", cmds["trace"])
    if os.path.isdir(os.path.join(w, "trace_all")):
        more, _ = _kernel_table(_find(os.path.join(w, "trace_all"), "*kernel_stats.csv"),
                                f"every pass of the bench, workload {workload}",
                                cmds["trace_all"])
        lines += [""] + more
    with open(os.path.join(prof, f"kernels_{workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    med = lambda v: sorted(v)[len(v) // 2]
    gib = float(1 << 30)
    cf = _counters_per_dispatch(os.path.join(out_root, "calib", "fetch"))
    cw = _counters_per_dispatch(os.path.join(out_root, "calib", "write"))
    # the calibration copy is the one dispatch whose byte counts are near 1 GiB
    copy_f = max(max(d["FETCH_SIZE"]) for d in cf.values() if "FETCH_SIZE" in d) * 1024.0
    copy_w = max(max(d["WRITE_SIZE"]) for d in cw.values() if "WRITE_SIZE" in d) * 1024.0
    f_fac, w_fac = gib / copy_f, gib / copy_w
    key = focused_attn_kernel(recipe)
    sf = _counters_per_dispatch(os.path.join(w, "fetch"))[key]["FETCH_SIZE"]
    sw = _counters_per_dispatch(os.path.join(w, "write"))[key]["WRITE_SIZE"]
    fetch = med(sf) * 1024.0 * f_fac
    write = med(sw) * 1024.0 * w_fac
    rec = {"workload": workload, "kernel": key, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": med(sf), "write_kib_per_dispatch": med(sw),
           "fetch_scale": f_fac, "write_scale": w_fac,
           "hbm_bytes_per_launch": int(round(fetch + write)),
           "hbm_read_bytes": int(round(fetch)), "hbm_write_bytes": int(round(write)),
           "trace_avg_us": avg.get(key),
           "commands": [cmds["fetch"], cmds["write"], cal["copy_fetch"], cal["copy_write"]]}
    mdir = os.path.join(w, "mfma")
    txt_mfma = []
    if os.path.isdir(mdir):
        m = _counters_per_dispatch(mdir)[key]
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (each counts the kernel's cycles);
        # SQ_VALU_MFMA_BUSY_CYCLES over all 1024 SIMDs
        busy = [b / (g / NUM_XCC * SIMD_NUM) for b, g in zip(m["SQ_VALU_MFMA_BUSY_CYCLES"],
                                                               m["GRBM_GUI_ACTIVE"])]
        flops = med(m["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512.0
        rec.update({"mfma_busy_frac": round(med(busy), 5), "mfma_bf16_flops_per_launch": flops})
        rec["commands"].append(cmds["mfma"])
        txt_mfma = [f"# command: {cmds['mfma']}",
                    f"MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {NUM_XCC} XCDs x "
                    f"{SIMD_NUM} SIMDs)):"
                    f" {med(busy) * 100:.2f}% (median of {len(busy)} dispatches); bf16 MFMA work "
                    f"SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = {flops / 1e9:.2f} GFLOP per launch"]
    with open(os.path.join(prof, f"attn_traffic_{workload}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    txt = [f"# HBM traffic and MFMA use of {key}, workload {workload} (focused step)",
           *[f"# command: {c}" for c in rec["commands"][:4]],
           f"copy calibration: 1 GiB copy reads as FETCH_SIZE {copy_f / 1024:.0f} KiB "
           f"(scale {f_fac:.3f}), WRITE_SIZE {copy_w / 1024:.0f} KiB (scale {w_fac:.3f})",
           f"attention per launch: FETCH_SIZE {med(sf):.0f} KiB -> {fetch / 1e6:.1f} MB read; "
           f"WRITE_SIZE {med(sw):.0f} KiB -> {write / 1e6:.1f} MB written; "
           f"total {(fetch + write) / 1e6:.1f} MB", *txt_mfma]
    if avg.get(key):
        txt.append(f"kernel-trace average duration {avg[key]:.2f} us")
    with open(os.path.join(prof, f"attn_traffic_{workload}.txt"), "w") as fh:
        fh.write("\n".join(txt) + "\n")
    # the front end's kernels from the same counter runs (every kernel of the step is counted)
    allf = _counters_per_dispatch(os.path.join(w, "fetch"))
    allw = _counters_per_dispatch(os.path.join(w, "write"))
    front = [f"# HBM traffic of the front-end kernels, workload {workload} (focused step; the "
             "same counter runs, scaled by the copy calibration)",
             *[f"# command: {c}" for c in rec["commands"][:4]],
             f"{'kernel':56s} {'read MB':>9s} {'written MB':>11s} {'trace avg us':>13s}"]
    for name in sorted(allf):
        if not name.startswith(FRONT_KERNELS):
            continue
        r_mb = med(allf[name]["FETCH_SIZE"]) * 1024.0 * f_fac / 1e6
        w_mb = med(allw.get(name, {}).get("WRITE_SIZE", [0.0])) * 1024.0 * w_fac / 1e6
        front.append(f"{name[:56]:56s} {r_mb:9.2f} {w_mb:11.2f} {avg.get(name, float('nan')):13.2f}")
    with open(os.path.join(prof, f"front_traffic_{workload}.txt"), "w") as fh:
        fh.write("\n".join(front) + "\n")
    print("\n".join(lines + txt + front))


class Flush:
    """Evicts the step's data from the caches (L2 and the 256 MB Infinity Cache) by reading a
    1 GiB buffer: clean lines, so no write-back lands in the next timed region."""

    def __init__(self, device, enabled=True):
        import torch
        self.enabled = enabled
        if enabled:
            self.buf = torch.ones(1 << 28, dtype=torch.float32, device=device)
            self.out = torch.empty((), dtype=torch.float32, device=device)

    def __call__(self):
        if self.enabled:
            import torch
            torch.sum(self.buf, dim=0, out=self.out)


def front_end_batch(args):
    """The front end alone at batch args.front_end_batch with the workload's shapes: layer-0/1
    Q/K and hidden states drawn on the device from a seeded generator, each position masked
    with probability 0.8, the budget ceil(0.125 * masked count) (the headline's rule); the
    hidden states are gathered (the attention reads its queries in place).  Prints one JSON
    line: mean us per call (caches flushed before each) and the score inputs' bytes."""
    import torch
    from decodability_aware_token_amd import binding as F
    from workloads import BY_NAME
    rc = BY_NAME[args.workload]
    B, blk, Hq, Hkv, d = args.front_end_batch, rc.blk, rc.Hq, rc.Hkv, rc.d
    W = rc.hidden or Hq * d
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(rc.seed)
    draw = lambda *shape: (torch.randn(*shape, device=dev, generator=g) * 0.5).to(torch.bfloat16)
    q0, q1 = draw(B, blk, Hq, d), draw(B, blk, Hq, d)
    k0, k1 = draw(B, blk, Hkv, d), draw(B, blk, Hkv, d)
    masked = (torch.rand(B, blk, device=dev, generator=g) < 0.8).to(torch.uint8)
    budget = torch.ceil(0.125 * masked.sum(1).float()).to(torch.int32)
    sets = [draw(B, blk, W)]
    cap = B * blk
    outs = dict(delta=torch.empty(B, blk, device=dev),
                keep=torch.empty(B, blk, dtype=torch.uint8, device=dev),
                kept_count=torch.empty(B, dtype=torch.int32, device=dev),
                offsets=torch.empty(B + 1, dtype=torch.int32, device=dev),
                kept_pos=torch.empty(cap, dtype=torch.int32, device=dev),
                gathered=[torch.empty((cap,) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
                          for x in sets])
    ws = torch.zeros(F.lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d),
                     dtype=torch.uint8, device=dev)
    max_kept = -(-blk // 8)
    fn = lambda: F.score_select_compact(q0, k0, q1, k1, d ** -0.5, masked, budget, sets, cap,
                                        max_kept=max_kept, workspace=ws, **outs)
    for _ in range(args.warmup):
        fn()
    ms = timed(fn, args.steps, Flush(dev, enabled=not args.no_flush),
               torch.cuda.current_stream(dev))
    print(json.dumps({"front_end_batch": B, "workload_shapes": rc.name, "us": round(ms * 1e3, 2),
                      "kept_tokens": int(outs["offsets"][-1]),
                      "score_input_bytes": 2 * B * blk * (Hq + Hkv) * d * 2}))


def timed(fn, steps, flush, stream):
    """Mean ms of fn() over `steps` calls, each bracketed by HIP events on `stream` with a cache
    flush before it (outside the events)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        flush()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))


def full_block_pass(inp, st, args, stream, flush):
    """The unfocused baseline on the same kernels (every block token a query): its attention
    launch timed by HIP events, caches flushed before each."""
    import torch
    from decodability_aware_token_amd import FullBlockStep
    fb = FullBlockStep(inp)
    for _ in range(args.warmup):
        fb.run()
    attn_ms = timed(fb.run, args.steps, flush, stream)
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


def full_domain_pass(inp, t, st, args, stream, flush):
    """Importance over the full attention domain: the score kernel with each block query's
    prefix+block log-sum-exp given (its own roofline), and the two layers' attentions that
    produce those LSEs here (in a model they come with layers 0 and 1)."""
    import torch
    from decodability_aware_token_amd import FullDomainScore
    fd = FullDomainScore(inp, t["k_cache0"], t["k_blk0"])
    for _ in range(args.warmup):
        fd.run()
    lse_ms = timed(fd.layer_lse, args.steps, flush, stream)
    sc_ms = timed(fd.score, args.steps, flush, stream)
    sb, sf = score_algorithmic(st)
    sb += 2 * st.B * st.blk * st.Hq * 4  # the two LSE arrays
    log(f"[bench] full-domain score: {sc_ms * 1000:.1f} us ({sb / (sc_ms * 1e-3) / 1e9:.0f} GB/s); "
        f"the two layers' LSE attentions {lse_ms * 1000:.1f} us")
    return {"score_lse_us": round(sc_ms * 1000, 2), "score_lse_algorithmic_bytes": sb,
            "score_lse_hbm_frac": round(sb / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "layer_lse_attention_us": round(lse_ms * 1000, 2)}


def kv_pass(fs, inp, st, args, stream, flush):
    """Intra-block KV write-back of the kept rows (fresh K/V stand-ins: the first Hkv heads of
    the block's query rows) and the commit of every request's block into its paged prefix, each
    timed by HIP events; the commit runs on a copy of the caches extended by free pages."""
    import torch
    from decodability_aware_token_amd import binding as F
    dev = inp.q_att.device
    T = int(fs.offsets[-1])
    rows = inp.q_att.reshape(-1, st.Hq, st.d)[: fs.cap, : st.Hkv].contiguous()  # [cap, Hkv, d]
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
    wb_ms = timed(wb, args.steps, flush, stream)
    cm_ms = timed(cm, args.steps, flush, stream)
    wb_bytes = 2 * 2 * T * st.Hkv * st.d * 2 + 4 * (T + st.B + 1)
    cm_bytes = 2 * 2 * st.B * st.blk * st.Hkv * st.d * 2 + 16 * st.B
    log(f"[bench] kv write-back {wb_ms * 1000:.1f} us ({wb_bytes / (wb_ms * 1e-3) / 1e9:.0f} GB/s)"
        f"; block commit {cm_ms * 1000:.1f} us ({cm_bytes / (cm_ms * 1e-3) / 1e9:.0f} GB/s)")
    # conversion of the whole prefix cache from plain head-major rows [pages, Hkv, S, d]
    pages, Hkv, D8 = inp.k_cache.shape[0], inp.k_cache.shape[1], inp.k_cache.shape[2]
    k_plain = inp.k_cache.permute(0, 1, 3, 2, 4).reshape(pages, Hkv, S, 8 * D8).contiguous()
    v_plain = inp.v_cache.permute(0, 1, 2, 4, 3).reshape(pages, Hkv, S, 8 * D8).contiguous()
    k_out, v_out = torch.empty_like(inp.k_cache), torch.empty_like(inp.v_cache)
    pk = lambda: F.kv_pack(k_plain, v_plain, k_out=k_out, v_out=v_out)
    pk()
    torch.cuda.synchronize()
    assert torch.equal(k_out.view(torch.int16), inp.k_cache.view(torch.int16))
    assert torch.equal(v_out.view(torch.int16), inp.v_cache.view(torch.int16))
    pk_ms = timed(pk, args.steps, flush, stream)
    pk_bytes = 4 * inp.k_cache.numel() * 2
    log(f"[bench] kv pack of the prefix cache {pk_bytes / 1e6:.0f} MB moved in {pk_ms * 1000:.1f} "
        f"us ({pk_bytes / (pk_ms * 1e-3) / 1e9:.0f} GB/s)")
    del k_plain, v_plain, k_out, v_out
    return {"writeback_us": round(wb_ms * 1000, 2), "writeback_bytes": wb_bytes,
            "commit_us": round(cm_ms * 1000, 2), "commit_bytes": cm_bytes,
            "commit_hbm_frac": round(cm_bytes / (cm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "pack_us": round(pk_ms * 1000, 2), "pack_bytes": pk_bytes,
            "pack_hbm_frac": round(pk_bytes / (pk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sdar_b256_blk32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batch", type=int, default=0,
                    help="run the workload's recipe at this batch size instead (a batch-scaling "
                         "point, named <workload>_b<B>; no counter record applies to it)")
    ap.add_argument("--no-full-domain", action="store_true",
                    help="skip the full-domain importance measurement")
    ap.add_argument("--no-full-block", action="store_true",
                    help="skip the unfocused (every block token kept) comparison step")
    ap.add_argument("--only-step", action="store_true",
                    help="time the focused step only (no full-block, full-domain or KV passes)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP graph replays reported beside the measured step")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not flush the caches before each timed step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--summarize-profiles", metavar="OUT_ROOT",
                    help="write the profiles/ summaries of --workload from the CSV output of the "
                         "rocprofv3 commands that --profile-commands prints (OUT_ROOT holds their "
                         "-d folders)")
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the rocprofv3 commands behind the profiles/ summaries of "
                         "--workload (the copy calibration first)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known bytes) 5 times, "
                         "to scale HBM byte counters")
    ap.add_argument("--front-end-batch", type=int, metavar="B",
                    help="only time the front end (score + select + compact of the hidden states "
                         "and queries) at batch B with --workload's shapes, on seeded synthetic "
                         "device tensors (no attention inputs are generated)")
    ap.add_argument("--oracle-worker", nargs=5, metavar=("RECIPE", "B", "SEED", "STRIDE", "S"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.oracle_worker:
        name, B, seed, stride, secs = args.oracle_worker
        oracle_worker(name, int(B), int(seed), int(stride), float(secs))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the step would shard "
              "by request, each GPU running the whole step on its share).", file=sys.stderr)
        sys.exit(2)
    if args.profile_commands:
        for c in list(calibration_commands().values()) + \
                list(profile_commands(args.workload).values()):
            print(c)
        return
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
    if args.front_end_batch:
        front_end_batch(args)
        return
    from decodability_aware_token_amd import FocusStep, StepInputs
    from workloads import BY_NAME, make_step
    from workloads.torch_io import upload

    recipe = BY_NAME[args.workload]
    if args.batch:  # the workload's recipe at another batch size (same seed and distributions)
        recipe = recipe.scaled(B=args.batch, name=f"{recipe.name}_b{args.batch}")
    only = args.only_step
    log(f"[bench] generating {recipe.name}")
    st = make_step(recipe, layer0_prefix=not (args.no_full_domain or only))
    dev = torch.device("cuda:0")
    t = upload(st, dev)
    inp = StepInputs(**{k: t[k] for k in ("q0", "k0", "q1", "k1", "masked", "budget", "adaptive",
                                           "max_kept", "q_att", "k_cache", "v_cache",
                                           "page_table", "prefix_len", "k_blk", "v_blk",
                                           "sm_scale", "hidden")})
    fs = FocusStep(inp)
    stream = torch.cuda.current_stream(dev)
    flush = Flush(dev, enabled=not args.no_flush)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        fs.run()
    torch.cuda.synchronize()

    # Pass 1 (eager, per-stage HIP events on the launch stream, caches flushed before each
    # step): the stage breakdown.
    stages = fs.front_stages + ("attend",)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    log(f"[bench] eager pass: {args.steps} steps with per-stage events")
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush()
        ev[i][0].record(stream)
        for j, name in enumerate(stages):
            getattr(fs, name)()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    per_stage = np.zeros(len(stages))
    step_ms = np.zeros(args.steps)
    for i in range(args.steps):
        for j in range(len(stages)):
            per_stage[j] += ev[i][j].elapsed_time(ev[i][j + 1])
        step_ms[i] = ev[i][0].elapsed_time(ev[i][-1])
    per_stage /= args.steps
    eager_ms = float(step_ms.mean())

    # Pass 2 (the measured step): the whole step (score partials, reduction + selection +
    # compaction of the hidden states and queries, attention) launched eagerly, with no host
    # synchronisation inside it, exactly K times, each bracketed by one pair of HIP events with
    # the caches flushed before it (outside the events): ms_per_step is their mean.  The kernels
    # of a step are enqueued while the flush still runs, so no launch gap of the host shows.
    log(f"[bench] measured pass: {args.steps} eager steps")
    ms_per_step = timed(fs.run, args.steps, flush, stream)
    mode = "eager"
    # The attention kernel's launch duration for the roofline: K launches on the last step's
    # compacted queries and offsets, each bracketed by HIP events on the launch stream with the
    # caches flushed before it (an event recorded between the front end and the attention, as
    # in pass 1, adds its own wait to the attention's interval).
    log(f"[bench] attention pass: {args.steps} launches")
    attn_ms = timed(fs.attend, args.steps, flush, stream)
    # Pass 3: the same step captured once in a HIP graph, replayed K times the same way, and
    # back to back without flushes: reported beside the measured step.
    graph_ms = b2b_ms = None
    if not args.no_graph:
        fs.capture()
        for _ in range(args.warmup):
            fs.replay()
        log(f"[bench] graph pass: {args.steps} replays")
        graph_ms = timed(fs.replay, args.steps, flush, stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fs.replay()
        torch.cuda.synchronize()
        b2b_ms = (time.perf_counter() - t0) * 1000.0 / args.steps

    offsets = fs.offsets.cpu().numpy()
    kept = np.diff(offsets)
    T = int(offsets[-1])
    attn_bytes, attn_flops = attn_algorithmic(st, kept)
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    sb, sf = score_algorithmic(st)
    for j, name in enumerate(stages):
        log(f"[bench] {name:20s} {per_stage[j] * 1000:9.1f} us")
    log(f"[bench] step (eager, flushed) {ms_per_step * 1000:.1f} us; with per-stage events "
        f"{eager_ms * 1000:.1f} us" + (f"; graph replays (flushed) {graph_ms * 1000:.1f} us, back "
                                       f"to back {b2b_ms * 1000:.1f} us" if graph_ms else "")
        + f"; T={T}")
    log(f"[bench] attention {attn_bytes / 1e6:.1f} MB algorithmic -> {achieved:.0f} GB/s "
        f"({achieved / PEAK_HBM_GBS * 100:.1f}% of HBM), "
        f"{attn_flops / (attn_ms * 1e-3) / 1e12:.2f} TFLOP/s")
    sc_ms = per_stage[0]
    log(f"[bench] {stages[0]}: score inputs {sb / 1e6:.1f} MB -> "
        f"{sb / (sc_ms * 1e-3) / 1e9:.0f} GB/s, {sf / (sc_ms * 1e-3) / 1e12:.2f} TFLOP/s")

    full = fdom = kvres = None
    if not (args.no_full_block or only):
        full = full_block_pass(inp, st, args, stream, flush)
    if not (args.no_full_domain or only):
        fdom = full_domain_pass(inp, t, st, args, stream, flush)
    if not only:
        kvres = kv_pass(fs, inp, st, args, stream, flush)

    counters = counter_record(recipe.name)
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
            "step_launch": mode, "cache_flush": "1 GiB read before each timed step"
            if flush.enabled else "none",
            "per_stage_events_ms_per_step": round(eager_ms, 5),
            "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
            "graph_back_to_back_ms_per_step": None if b2b_ms is None else round(b2b_ms, 5),
            "full_block_step": full,
            "full_domain_score": fdom,
            "kv_cache": kvres,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "ragged paged attention, queries read in place (focus_ragged_paged_attn_pos)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if counters is None else counters.get("hbm_bytes_per_launch"),
            "algorithmic_bytes_per_launch": attn_bytes,
            "avg_launch_us": round(attn_ms * 1000, 2),
            "mfma_util": round(attn_flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
            "mfma_busy_counter": None if counters is None else counters.get("mfma_busy_frac"),
        },
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s of oracle work per worker)")
        res["cpu_baseline"] = cpu_baseline(recipe, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
