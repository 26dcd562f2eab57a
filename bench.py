"""Benchmark of the shared-prefix GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fanout]

A step is one forward of the whole path (plan reuse, attention kernels, LSE
merge) over one batch of synthetic input already resident in HBM. The
headline workload is the 8-agent fan-out (8 sub-agents x 20 new tokens over
a 32768-token shared prefix, 512 private tokens each in 16-token pages,
Llama3-70B heads: H_q 64, H_kv 8, d 128, bf16). Input copies are rotated so
the K/V working set is at least twice the 256 MB last-level cache and every
step reads its K/V from HBM.

Before each timed region the forward runs untimed until the GPU has been
busy for CLOCK_WARMUP_S (the clocks leave their low-power state only under
sustained load); the timed region is exactly K forwards.

Prints ONE JSON line: throughput (TFLOP/s on the algorithmic FLOP count),
effective KV GB/s, the roofline of the dominant kernel (timed with HIP
events recorded by the library on the forward's stream), the fp64 CPU oracle
timed on a bounded sample on this host, and secondary lines for the other
workloads (decode, prefill, mixed, joins, K/V append).

Other modes: --sweep-splits W times a workload over a range of shard counts
(GPU); --kernel-summary, --counter-summary, --trace-summary and
--traffic-summary turn rocprofv3 output into the tables under profiles/ (no
GPU needed).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + KV GB/s (% of MI355X roofline), 8-agent fan-out GQA"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 matrix/vector (published)
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E (published)
LLC_BYTES = 256 << 20           # Infinity Cache
CLOCK_WARMUP_S = 0.3            # untimed sustained load before each timed region

WORKLOADS = {"fanout": "fanout_8x20_32k", "decode": "decode_8k", "prefill": "prefill_32k",
             "mixed": "mixed_32dec_64x4", "tiny": "tiny_fp32_fanout", "join400": "join_400_32k",
             "join8000": "join_8000_32k"}
# The attention kernels and the planner that lays out their work: HBM traffic
# depends on both (shard counts, M-tiles, chains, XCD placement).
KERNEL_SOURCES = ["gqa_attention_agentic_amd/csrc/attention.hip", "gqa_attention_agentic_amd/csrc/plan.cpp",
                  "gqa_attention_agentic_amd/csrc/plan_types.h"]
APPEND_SOURCES = ["gqa_attention_agentic_amd/csrc/append.hip"]


def kernel_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def clone_inputs(inp, n):
    from workload.generate import Inputs
    out = [inp]
    for _ in range(n - 1):
        out.append(Inputs(inp.q.clone(), inp.k_shared.clone(), inp.v_shared.clone(), inp.k_pages.clone(),
                          inp.v_pages.clone(), inp.page_table.clone(), inp.group_shared_start,
                          inp.group_shared_len, inp.branch_group, inp.branch_q_len,
                          inp.branch_private_len))
    return out


class Prepared:
    """A workload's inputs on the device: enough rotated copies that the K/V
    working set is at least twice the Infinity Cache (a rotation just above
    its size still hits in it for a good part), so every step reads its K/V
    from HBM."""

    def __init__(self, name, log):
        import torch

        from workload import generate, get_workload

        self.w = w = get_workload(name) if isinstance(name, str) else name
        t0 = time.time()
        base = generate(w, "cuda")
        n_copies = max(1, min(16, -(-2 * LLC_BYTES // max(1, w.kv_bytes()))))
        if w.kv_bytes() > 4 * LLC_BYTES:
            n_copies = 1
        self.copies = clone_inputs(base, n_copies)
        self.out = torch.empty_like(base.q)
        self.lse = torch.empty(base.q.shape[0], w.num_q_heads, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] {w.name}: inputs ready ({n_copies} copies, {time.time() - t0:.1f}s)")

    def close(self):
        import torch
        del self.copies, self.out, self.lse
        torch.cuda.empty_cache()


def time_forwards(p: Prepared, steps: int, warmup: int, log, splits="config"):
    """Times `steps` forwards of a prepared workload; returns the result dict.
    splits: "config" uses the workload's own split list (None: heuristic);
    a list overrides it (one entry per unit, 0 = heuristic)."""
    import torch

    import gqa_attention_agentic_amd as G

    w, copies = p.w, p.copies
    n_copies = len(copies)
    split_list = w.splits if isinstance(splits, str) else splits
    h = G.GqaAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.dtype)
    stream = torch.cuda.current_stream()

    def step(i):
        h.forward_inputs(copies[i % n_copies], w.causal, splits=split_list, out=p.out, lse=p.lse,
                         stream=stream.cuda_stream)

    # Every input copy is used once before timing, so no timed step pays a
    # first touch (page-table walks) of a copy. The warm-up then goes on
    # until the GPU has been kept busy for CLOCK_WARMUP_S: it leaves its
    # low-power clocks only after some tens of milliseconds of sustained load
    # (measured on MI355X: the fan-out's attention launch takes ~220 us in
    # the first ~10 ms of load and ~183 us after ~50 ms).
    warmup = max(warmup, n_copies)
    t0 = time.perf_counter()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    per_step = max(1e-6, (time.perf_counter() - t0) / warmup)
    batch = max(1, int(0.02 / per_step))   # ~20 ms of work between host checks
    while time.perf_counter() - t0 < CLOCK_WARMUP_S:
        for _ in range(batch):
            step(warmup)
            warmup += 1
        torch.cuda.synchronize()
    # Wall clock over exactly `steps` forwards with no per-kernel events: the
    # library's timing events cost ~9 us at every kernel boundary (measured
    # in rocprofv3 traces: back-to-back kernels without them).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = start.elapsed_time(end) / steps
    # Kernel durations over `steps` more forwards, from the HIP events each
    # launch records around its own kernel on the stream it runs on; the
    # medians over those forwards of the attention time, the merge time and
    # their sum per forward.
    h.enable_timing(True)
    for i in range(steps):
        step(warmup + steps + i)
    torch.cuda.synchronize()
    per = h.kernel_times_list()
    h.enable_timing(False)
    attn_ms = statistics.median(a for a, _ in per)
    merge_ms = statistics.median(m for _, m in per)
    kernel_ms = statistics.median(a + m for a, m in per)
    stats = h.plan_stats()
    flops, kv_bytes = w.flops(), w.kv_bytes()
    res = {
        "workload": w.name,
        "description": w.description,
        "flops": flops,
        "kv_bytes": kv_bytes,
        "io_bytes": w.io_bytes(),
        "ms_per_step": wall_ms,
        "attn_kernel_ms": attn_ms,
        "merge_kernel_ms": merge_ms,
        "kernel_ms": kernel_ms,
        "kernel_ms_mean": sum(a + m for a, m in per) / len(per),
        "timed_forwards": len(per),
        "tflops": flops / (wall_ms * 1e-3) / 1e12,
        "kv_gbps": kv_bytes / (wall_ms * 1e-3) / 1e9,
        "attn_kernel_tflops": flops / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None,
        "plan": stats,
        "splits": h.plan_splits()[:8],
        "input_copies": n_copies,
        "warmup_steps": warmup,
        "dtype": w.dtype,
    }
    log(f"[bench] {w.name}: {wall_ms:.4f} ms/step, attention {attn_ms:.4f} ms, merge {merge_ms:.4f} ms (medians), "
        f"{res['tflops']:.1f} TFLOP/s, KV {res['kv_gbps']:.0f} GB/s")
    h.close()
    return res


def run_workload(name: str, steps: int, warmup: int, log, splits="config"):
    """Times `steps` forwards of the named workload; returns (workload, result dict)."""
    p = Prepared(name, log)
    res = time_forwards(p, steps, warmup, log, splits=splits)
    p.close()
    return p.w, res


def run_append(steps: int, warmup: int, log):
    """Times the paged K/V append of a full-text join's 8000 new rows (AHBM
    Agentic Runtime Architecture, §5.5) into one branch's private pages:
    HBM-bound, each row's K and V read once and written once. Input copies
    rotate over more than twice the Infinity Cache."""
    import torch

    import gqa_attention_agentic_amd as G
    from workload import get_workload

    w = get_workload("join_8000_32k")
    rows, H_kv, d, ps = 8000, w.num_kv_heads, w.head_dim, w.page_size
    n_pages = -(-rows // ps)
    row_bytes = 2 * H_kv * d * 2                 # K and V, bf16
    moved = 2 * rows * row_bytes                 # read + written
    n_copies = max(1, min(16, -(-2 * LLC_BYTES // (moved))))
    g = torch.Generator(device="cuda").manual_seed(8)
    sets = []
    for _ in range(n_copies):
        kn = torch.randn(rows, H_kv, d, generator=g, device="cuda").to(torch.bfloat16)
        vn = torch.randn(rows, H_kv, d, generator=g, device="cuda").to(torch.bfloat16)
        kp = torch.empty(n_pages, H_kv, ps, d, dtype=torch.bfloat16, device="cuda")
        vp = torch.empty_like(kp)
        table = torch.randperm(n_pages, generator=g, device="cuda").to(torch.int32).view(1, -1).contiguous()
        sets.append((kn, vn, kp, vp, table))
    h = G.GqaAttention(w.num_q_heads, H_kv, d, ps, w.dtype)
    stream = torch.cuda.current_stream()

    def step(i):
        kn, vn, kp, vp, table = sets[i % n_copies]
        h.append_kv(kn, vn, kp, vp, table, [0], [rows], stream=stream.cuda_stream)

    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < max(warmup, n_copies) or time.perf_counter() - t0 < CLOCK_WARMUP_S:
        for _ in range(64):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    h.enable_timing(True)
    for i in range(steps):
        step(steps + i)
    torch.cuda.synchronize()
    kms, n = h.append_times()
    h.enable_timing(False)
    kms /= max(1, n)
    gbps = moved / (kms * 1e-3) / 1e9
    log(f"[bench] append 8000 rows: {ms * 1e3:.1f} us/call wall, kernel {kms * 1e3:.1f} us, {gbps:.0f} GB/s")
    # HBM bytes of the append kernel from the counter runs that profiled it
    # (a decode run with the append leg), while its source is unchanged.
    traffic = None
    path = os.path.join(ROOT, "profiles", "traffic_decode_8k.json")
    if os.path.exists(path):
        with open(path) as f:
            t = json.load(f)
        a = t.get("per_kernel", {}).get("append_kv_rows")
        if a and t.get("append_kernel_hash") == kernel_hash(APPEND_SOURCES):
            traffic = a["fetch_bytes"] + a["write_bytes"]
    return {"workload": "append_kv: 8000 rows (join input) into 16-token pages", "ms_per_step": ms,
            "kernel_ms": kms, "bytes_per_call": moved, "input_copies": n_copies,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": gbps / PEAK_HBM_GBPS, "traffic": traffic}}


def roofline_of(w, res, traffic, achievable=None):
    """Roofline of the attention path from its kernel time T: the median over
    the timed forwards of attention + merge kernel time per forward (HIP
    events recorded by each launch). frac_attention uses the attention
    launch alone; frac_of_achievable divides by the probe-measured ceiling
    of the same kind, when there is one."""
    t = res["kernel_ms"] * 1e-3
    ta = res["attn_kernel_ms"] * 1e-3
    peak_mfma = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    intensity = w.flops() / (w.kv_bytes() + w.io_bytes())
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if intensity >= ridge:
        work, unit, peak, scale, ach_key = w.flops(), "TFLOP/s", peak_mfma, 1e12, "mfma_bf16_tflops"
        bound = "mfma"
    else:
        work, unit, peak, scale, ach_key = w.kv_bytes() + w.io_bytes(), "GB/s", PEAK_HBM_GBPS, 1e9, "hbm_read_gbps"
        bound = "hbm"
    achieved = work / t / scale
    out = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
           "frac_attention": work / ta / scale / peak, "traffic": traffic,
           "time_basis": f"median over {res['timed_forwards']} forwards of attention + merge kernel time"}
    if achievable and achievable.get(ach_key) and (bound == "hbm" or w.dtype == "bf16"):
        out["achievable"] = achievable[ach_key]
        out["frac_of_achievable"] = achieved / achievable[ach_key]
    return out


def measure_peaks(log):
    """Achievable ceilings on this GPU (include/gqa_probe.h), after a warm-up
    that brings the clocks up: the bf16 MFMA rate of four independent
    v_mfma_f32_32x32x16_bf16 chains per wave (1 and 2 waves per SIMD, the
    better one), and a plain streaming read of 33,554,432 bytes (the 8k
    decode's K/V) rotated over 16 copies and of 1 GiB over 2 copies (each
    set at least twice the Infinity Cache)."""
    import torch

    import gqa_attention_agentic_amd as G

    G.probe_mfma_bf16(2, 2048, 400)   # warm-up, ~0.1 s of MFMA load
    mfma = {wps: G.probe_mfma_bf16(wps, 2048, 50) for wps in (1, 2)}
    out = {"mfma_bf16_tflops": max(t for t, _ in mfma.values()),
           "mfma_bf16_tflops_by_waves_per_simd": {str(k): v[0] for k, v in mfma.items()}}
    small = 33554432
    buf = torch.empty(16 * small, dtype=torch.uint8, device="cuda").fill_(1)
    G.probe_read(buf, small, 16, 200)
    out["hbm_read_gbps"], out["hbm_read_us_33MB"] = G.probe_read(buf, small, 16, 64)
    del buf
    big = 1 << 30
    buf = torch.empty(2 * big, dtype=torch.uint8, device="cuda").fill_(1)
    out["hbm_read_gbps_1GiB"], out["hbm_read_us_1GiB"] = G.probe_read(buf, big, 2, 16)
    del buf
    torch.cuda.empty_cache()
    out["note"] = ("medians of probe launches timed with HIP events; published peaks: 2500 TFLOP/s bf16, "
                   "8000 GB/s HBM")
    log(f"[bench] achievable: MFMA bf16 {out['mfma_bf16_tflops']:.0f} TFLOP/s, read 33.5 MB "
        f"{out['hbm_read_gbps']:.0f} GB/s ({out['hbm_read_us_33MB']:.2f} us), read 1 GiB "
        f"{out['hbm_read_gbps_1GiB']:.0f} GB/s")
    return out


def traffic_for(w):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(name: str, budget_s: float, log):
    """The fp64 oracle on this host's cores over whole branches of the same
    workload until about budget_s seconds of CPU work (input generation and
    copies excluded)."""
    import torch

    import oracle
    from workload import cpu_subset, generate, get_workload

    w = get_workload(name)
    torch.set_num_threads(os.cpu_count() or 1)
    inp = generate(w, "cpu")
    done_flops, spent, branches = 0, 0.0, []
    qb = [0]
    for b in w.branches:
        qb.append(qb[-1] + b.q_len)
    order = sorted(range(len(w.branches)), key=lambda b: -w.branches[b].q_len)
    for b in order:
        if spent >= budget_s:
            break
        br = w.branches[b]
        if br.q_len == 0:
            continue
        sub, _ = cpu_subset(inp, [b])
        t0 = time.perf_counter()
        if br.q_len > 1024:   # long prefill: a bounded row sample across the whole sequence
            toks = list(range(0, br.q_len, max(1, br.q_len // 48)))
            oracle.attention(sub, w.num_kv_heads, w.page_size, w.causal, tokens=toks)
            C = w.context_len(br)
            pairs = sum((C - br.q_len + t + 1) if w.causal else C for t in toks)
        else:
            oracle.attention(sub, w.num_kv_heads, w.page_size, w.causal)
            C = w.context_len(br)
            pairs = sum((C - br.q_len + t + 1) if w.causal else C for t in range(br.q_len))
        spent += time.perf_counter() - t0
        done_flops += 4 * w.head_dim * w.num_q_heads * pairs
        branches.append(b)
    value = done_flops / spent / 1e12
    sample = (f"{len(branches)} of {len(w.branches)} branches of {w.name} "
              f"({done_flops / 1e9:.1f} GFLOP, all {w.num_q_heads} heads, fp64, {spent:.1f}s)")
    log(f"[bench] cpu oracle: {value * 1e3:.2f} GFLOP/s on {sample}")
    return {"value": value, "unit": "TFLOP/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": sample, "cpu": cpu_model(), "os_cpu_count": os.cpu_count(), "seconds": spent}


# Split counts swept for the first unit (the group's shared prefix) of each
# workload; the other units keep the library's heuristic (0).
SWEEPS = {"decode": [1, 2, 4, 8, 16, 24, 32, 48, 64, 128],
          "fanout": [1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16],
          "prefill": [1, 2, 4, 8, 16],
          "join400": [1, 2, 4, 6, 7, 8, 12, 16]}


def sweep_splits(name: str, steps: int, warmup: int, log, out_path: str):
    """Times the workload at each swept split count of its shared prefix and
    with every unit left to the heuristic; prints a table and writes the
    points (with the number of forwards each issued, for grouping a kernel
    trace of the same run) to out_path."""
    p = Prepared(WORKLOADS[name], log)
    n_units = len(p.w.groups) + len(p.w.branches)
    points = [("heuristic", [0] * n_units)] + [(str(k), [k] + [0] * (n_units - 1)) for k in SWEEPS[name]]
    if p.w.splits is not None:
        points.insert(1, ("workload's own", list(p.w.splits)))
    rows = []
    for label, sp in points:
        r = time_forwards(p, steps, warmup, log, splits=sp)
        rows.append({"label": label, "splits_override": sp, "chosen": r["splits"][:2],
                     "forwards": r["warmup_steps"] + 2 * steps, "timed": steps,
                     "attn_us": r["attn_kernel_ms"] * 1e3, "merge_us": r["merge_kernel_ms"] * 1e3,
                     "wall_us": r["ms_per_step"] * 1e3, "plan": r["plan"]})
    p.close()
    print(f"split sweep of {p.w.name} ({p.w.description}); kernel times from the library's HIP events, "
          f"mean over {steps} timed forwards")
    print("| point | splits (prefix, first suffix) | items wide / narrow | merge launch | attention us | merge us | wall us |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        pl = r["plan"]
        print(f"| {r['label']} | {r['chosen'][0]}, {r['chosen'][1]} | {pl['n_items_wide']} / {pl['n_items_narrow']} | "
              f"{pl['merge_launch']} | {r['attn_us']:.1f} | {r['merge_us']:.1f} | {r['wall_us']:.1f} |")
    with open(out_path, "w") as f:
        json.dump({"workload": p.w.name, "points": rows}, f, indent=1)


def read_kernel_trace(csv_path: str):
    """(kernel name, start ns, end ns) of every dispatch in a rocprofv3
    kernel-trace CSV, in start order."""
    import csv

    out = []
    with open(csv_path) as f:
        for rec in csv.DictReader(f):
            out.append((rec.get("Kernel_Name", ""), int(rec["Start_Timestamp"]), int(rec["End_Timestamp"])))
    out.sort(key=lambda x: x[1])
    return out


def kernel_summary(csv_path: str, last: int):
    """Per-kernel durations of a bench run's kernel trace: all calls, and the
    last `last` calls (the timed steps of a single-workload run)."""
    import statistics

    by = {}
    for name, s, e in read_kernel_trace(csv_path):
        if "gqa::" not in name:
            continue   # the library's kernels only (input generation and copies are left out)
        name = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0].replace("gqa::", "")
        by.setdefault(name, []).append((e - s) / 1e3)
    print(f"| kernel | calls | average us (all calls) | average us (last {last} calls) | median us (last {last}) | min us |")
    print("|---|---|---|---|---|---|")
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        tail = d[-last:]
        print(f"| {name} | {len(d)} | {sum(d) / len(d):.2f} | {sum(tail) / len(tail):.2f} | "
              f"{statistics.median(tail):.2f} | {min(d):.2f} |")


def counter_summary(csv_path: str, last: int):
    """Per-kernel means of a rocprofv3 --pmc CSV (one row per dispatch and
    counter) over each kernel's last `last` dispatches, with the dispatch
    duration and each counter's rate per nanosecond of it."""
    import csv

    rows = {}
    with open(csv_path) as f:
        for rec in csv.DictReader(f):
            key = (rec["Kernel_Name"], int(rec["Dispatch_Id"]))
            d = rows.setdefault(key, {"dur": int(rec["End_Timestamp"]) - int(rec["Start_Timestamp"])})
            d[rec["Counter_Name"]] = d.get(rec["Counter_Name"], 0.0) + float(rec["Counter_Value"])
    by = {}
    for (name, disp), d in sorted(rows.items(), key=lambda kv: kv[0][1]):
        by.setdefault(name, []).append(d)
    for name, ds in by.items():
        tail = ds[-last:]
        cols = sorted(k for k in tail[0] if k != "dur")
        dur = sum(d["dur"] for d in tail) / len(tail)
        print(f"{name}: {len(ds)} dispatches, mean over the last {len(tail)}: duration {dur / 1e3:.2f} us")
        for c in cols:
            v = sum(d.get(c, 0.0) for d in tail) / len(tail)
            print(f"  {c} = {v:.6g} ({v / dur:.4g} per ns)")


def traffic_summary(fetch_csv: str, write_csv: str, workload: str, last: int, cmd_fetch: str, cmd_write: str):
    """HBM bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) of `bench.py --copy-calibration 1024`:
    each counter is scaled by 2^30 bytes over what it read for the largest
    plain device copy (2^30 bytes) of the same run, then averaged over each
    attention / merge kernel's last `last` dispatches. Writes
    profiles/traffic_<workload>.json."""
    import csv

    from workload import get_workload

    def read(path, counter):
        per = {}
        with open(path) as f:
            for rec in csv.DictReader(f):
                if rec["Counter_Name"] != counter:
                    continue
                key = (int(rec["Dispatch_Id"]), rec["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(rec["Counter_Value"])
        rows = [(d, n, v) for (d, n), v in sorted(per.items())]
        copy = max(v for _, n, v in rows if "gqa::" not in n)
        scale = (1 << 30) / (copy * 1024.0)
        by = {}
        for _, n, v in rows:
            if "gqa::" in n:
                by.setdefault(n, []).append(v)
        return scale, {n: sum(v[-last:]) / len(v[-last:]) * 1024.0 * scale for n, v in by.items()}

    fs, fetch = read(fetch_csv, "FETCH_SIZE")
    ws, write = read(write_csv, "WRITE_SIZE")
    short = lambda n: n.replace("(anonymous namespace)::", "").split("(")[0].split("::")[-1]
    per_kernel = {short(n): {"fetch_bytes": round(fetch[n]), "write_bytes": round(write.get(n, 0.0))} for n in fetch}
    # the kernels the roofline's time covers: the attention launches and the merge
    attn = [k for k in per_kernel if k.startswith("attn_") or k.startswith("lse_merge")]
    w = get_workload(WORKLOADS[workload])
    out = {"workload": w.name, "kernel_hash": kernel_hash(),
           "hbm_bytes_per_launch": sum(per_kernel[k]["fetch_bytes"] + per_kernel[k]["write_bytes"] for k in attn),
           "per_kernel": per_kernel, "fetch_scale": fs, "write_scale": ws,
           "calibration": f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by 2^30 bytes / the counter read "
                          f"for a device copy of 2^30 bytes in the same run (fetch x{fs:.4f}, write x{ws:.4f})",
           "algorithmic_bytes": w.kv_bytes() + w.io_bytes(),
           "command_fetch": cmd_fetch, "command_write": cmd_write}
    if "append_kv_rows" in per_kernel:
        out["append_kernel_hash"] = kernel_hash(APPEND_SOURCES)
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    for k, v in per_kernel.items():
        print(f"| {k} | {v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} |")
    print(f"wrote {path}")


def read_once_variants():
    """Fan-out variants over the 32768-token shared prefix (20 new tokens and
    512 private tokens per agent, 16-token pages, H_kv 8, d 128, bf16): the
    agent count at G = 8, then the query heads per KV head at 8 agents. The
    prefix is stored once; every variant should fetch about its unique bytes."""
    from workload.configs import Branch, Group, Workload

    out = []
    for n in (1, 2, 4, 8):
        out.append((f"{n} agents, G 8", Workload(
            name=f"fanout_{n}x20_32k", dtype="bf16", num_q_heads=64, num_kv_heads=8, head_dim=128,
            page_size=16, groups=[Group(32768)], branches=[Branch(0, 20, 512) for _ in range(n)],
            causal=True, seed=3, description=f"{n} agents x 20 tokens over a 32768-token prefix")))
    for g in (1, 2, 4):
        out.append((f"8 agents, G {g}", Workload(
            name=f"fanout_8x20_32k_g{g}", dtype="bf16", num_q_heads=8 * g, num_kv_heads=8, head_dim=128,
            page_size=16, groups=[Group(32768)], branches=[Branch(0, 20, 512) for _ in range(8)],
            causal=True, seed=3, description=f"8 agents x 20 tokens, G {g}")))
    return out


def sweep_read_once(steps: int, warmup: int, log, out_path: str):
    """Times each read-once variant (run it under rocprofv3 --pmc FETCH_SIZE
    with --copy-calibration); writes the points with their forward counts
    and unique bytes to out_path for --pmc-sweep-summary."""
    rows = []
    for label, w in read_once_variants():
        p = Prepared(w, log)
        r = time_forwards(p, steps, warmup, log, splits=None)
        p.close()
        rows.append({"label": label, "workload": w.name, "forwards": r["warmup_steps"] + 2 * steps, "timed": steps,
                     "unique_bytes": w.kv_bytes() + w.io_bytes(), "kv_bytes": w.kv_bytes(),
                     "attn_us": r["attn_kernel_ms"] * 1e3, "plan": r["plan"]})
        print(f"{label}: attention {r['attn_kernel_ms'] * 1e3:.1f} us, unique bytes {rows[-1]['unique_bytes']:,}",
              flush=True)
    with open(out_path, "w") as f:
        json.dump({"points": rows}, f, indent=1)


def pmc_sweep_summary(sweep_path: str, csv_path: str, counter: str = "FETCH_SIZE"):
    """Per-point HBM bytes of the attention launches of a read-once sweep run
    under rocprofv3 --pmc: attention dispatches in dispatch order are
    assigned to the points by their forward counts (a side-by-side forward
    has two), each point averages its timed forwards, and KiB are scaled by
    the largest plain device copy (2^30 bytes) of the run."""
    import csv

    with open(sweep_path) as f:
        sweep = json.load(f)
    per = {}
    with open(csv_path) as f:
        for rec in csv.DictReader(f):
            if rec["Counter_Name"] != counter:
                continue
            key = (int(rec["Dispatch_Id"]), rec["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(rec["Counter_Value"])
    rows = sorted(per.items())
    copy = max(v for (_, n), v in rows if "gqa::" not in n)
    scale = (1 << 30) / (copy * 1024.0)
    attn = [v * 1024.0 * scale for (_, n), v in rows if "attn_" in n]
    i = 0
    print(f"| point | unique bytes (K/V once + Q, O, LSE) | {counter} of the attention launch, bytes | ratio |")
    print("|---|---|---|---|")
    for r in sweep["points"]:
        pl = r["plan"]
        per_fwd = int(pl["n_items_wide"] > 0) + int(pl["n_items_narrow"] > 0)
        n = r["forwards"] * per_fwd
        a = attn[i:i + n]
        i += n
        tail = [sum(a[k:k + per_fwd]) for k in range(0, len(a), per_fwd)][-r["timed"]:]
        b = sum(tail) / max(1, len(tail))
        print(f"| {r['label']} | {r['unique_bytes']:,} | {b:,.0f} | {b / r['unique_bytes']:.3f} |")
    if i != len(attn):
        print(f"(dispatch count mismatch: {i} of {len(attn)})")
    print(f"(counter scale x{scale:.4f} from the largest plain copy)")


def trace_summary(sweep_path: str, csv_path: str):
    """Per-point kernel durations from a rocprofv3 kernel-trace CSV of a
    sweep run: dispatches of the attention and merge kernels, in start order,
    are assigned to the sweep points by the number of forwards each point
    issued; each point's average covers its timed forwards only."""
    with open(sweep_path) as f:
        sweep = json.load(f)
    attn, merge = [], []
    for name, s, e in read_kernel_trace(csv_path):
        if "attn_" in name:
            attn.append((s, e))
        elif "lse_merge" in name:
            merge.append((s, e))
    ia = im = 0
    print(f"| point | attention launches | attention us (rocprofv3, timed forwards) | merge us | library events: attention / merge us |")
    print("|---|---|---|---|---|")
    for r in sweep["points"]:
        pl = r["plan"]
        per_fwd = int(pl["n_items_wide"] > 0) + int(pl["n_items_narrow"] > 0)
        n = r["forwards"]
        a = attn[ia:ia + per_fwd * n]
        ia += per_fwd * n
        spans = [max(e for _, e in a[k:k + per_fwd]) - min(s for s, _ in a[k:k + per_fwd])
                 for k in range(0, len(a), per_fwd)][-r["timed"]:]
        m_us = 0.0
        if pl["merge_launch"]:
            m = merge[im:im + n]
            im += n
            m_us = sum(e - s for s, e in m[-r["timed"]:]) / max(1, r["timed"]) / 1e3
        a_us = sum(spans) / max(1, len(spans)) / 1e3
        print(f"| {r['label']} ({r['chosen'][0]}) | {per_fwd} x {n} | {a_us:.1f} | {m_us:.1f} | "
              f"{r['attn_us']:.1f} / {r['merge_us']:.1f} |")
    if ia != len(attn) or im != len(merge):
        print(f"(dispatch count mismatch: attention {ia} of {len(attn)}, merge {im} of {len(merge)})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fanout", choices=sorted(WORKLOADS))
    ap.add_argument("--others", default="decode,decode_heuristic,prefill,mixed,join400,join8000,append",
                    help="comma list of secondary workloads ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 plain device copies of MIB MiB each, so that byte counters read "
                         "under a profiler can be scaled by a copy of known size")
    ap.add_argument("--sweep-splits", choices=sorted(SWEEPS), default=None,
                    help="time the workload over a range of split counts instead of the bench line")
    ap.add_argument("--sweep-out", default="sweep.json")
    ap.add_argument("--trace-summary", nargs=2, metavar=("SWEEP_JSON", "KERNEL_TRACE_CSV"), default=None,
                    help="print per-point rocprofv3 kernel durations of a sweep run (no GPU needed)")
    ap.add_argument("--kernel-summary", metavar="KERNEL_TRACE_CSV", default=None,
                    help="print per-kernel rocprofv3 durations of a bench run, the last --steps calls "
                         "apart (no GPU needed)")
    ap.add_argument("--counter-summary", metavar="PMC_CSV", default=None,
                    help="print per-kernel means of a rocprofv3 --pmc run over the last --steps dispatches "
                         "(no GPU needed)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CMD_FETCH", "CMD_WRITE"),
                    default=None, help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs "
                                       "of --workload (no GPU needed)")
    ap.add_argument("--read-once-sweep", action="store_true",
                    help="run the fan-out at 1/2/4/8 agents and G 1/2/4/8 (for a --pmc FETCH_SIZE run)")
    ap.add_argument("--probe-peaks", action="store_true",
                    help="only measure the achievable MFMA and HBM read ceilings (include/gqa_probe.h)")
    ap.add_argument("--no-probes", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--pmc-sweep-summary", nargs=2, metavar=("SWEEP_JSON", "PMC_CSV"), default=None,
                    help="per-point HBM bytes of a --read-once-sweep run under --pmc (no GPU needed)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.kernel_summary:
        kernel_summary(args.kernel_summary, args.steps)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.steps)
        return
    if args.pmc_sweep_summary:
        pmc_sweep_summary(*args.pmc_sweep_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary[:2], args.workload, args.steps, *args.traffic_summary[2:])
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    log = lambda m: print(m, file=sys.stderr, flush=True)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gqa_attention_agentic_amd as G
    G.load()
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration: 3 device copies of {n} bytes")
        del src, dst

    if args.probe_peaks:
        print(json.dumps(measure_peaks(log)), flush=True)
        return
    if args.read_once_sweep:
        os.makedirs(os.path.dirname(os.path.abspath(args.sweep_out)), exist_ok=True)
        sweep_read_once(args.steps, args.warmup, log, args.sweep_out)
        return
    if args.sweep_splits:
        os.makedirs(os.path.dirname(os.path.abspath(args.sweep_out)), exist_ok=True)
        sweep_splits(args.sweep_splits, args.steps, args.warmup, log, args.sweep_out)
        return
    achievable = None if args.no_probes else measure_peaks(log)
    w, res = run_workload(WORKLOADS[args.workload], args.steps, args.warmup, log)
    traffic = traffic_for(w)
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        if name == "append":
            others[name] = run_append(args.steps, 2, log)
            continue
        if name == "decode_heuristic":
            # The 8k decode with every shard count left to the library (the
            # workload as specified pins 32 shards).
            wo, ro = run_workload(WORKLOADS["decode"], args.steps, 2, log, splits=None)
            ro["roofline"] = roofline_of(wo, ro, None, achievable)
            ro["note"] = "decode_8k with the library's own shard choice instead of the pinned 32"
            others[name] = ro
            continue
        # Long workloads get fewer timed steps, so the default run stays short.
        long_wl = name in ("prefill", "mixed", "join8000")
        wo, ro = run_workload(WORKLOADS[name], max(3, args.steps // 4) if long_wl else args.steps, 2, log)
        ro["roofline"] = roofline_of(wo, ro, traffic_for(wo), achievable)
        others[name] = ro
    line = {
        "metric": METRIC,
        "value": res["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic N(0,1), seeded; shapes of the Llama3-70B attention layer",
        "config": {"workload": w.name, "agents": len(w.branches), "new_tokens_per_agent": w.branches[0].q_len,
                   "shared_prefix": w.groups[0].shared_len, "private_suffix": w.branches[0].private_len,
                   "page_size": w.page_size, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "causal": w.causal, "parallelism": "single GPU"},
        "kv_gbps": res["kv_gbps"],
        "kv_frac_of_hbm_peak": res["kv_gbps"] / PEAK_HBM_GBPS,
        "attn_kernel_ms": res["attn_kernel_ms"],
        "merge_kernel_ms": res["merge_kernel_ms"],
        "kernel_ms": res["kernel_ms"],
        "roofline": roofline_of(w, res, traffic, achievable),
        "achievable_peak": achievable,
        "kernel_source_hash": kernel_hash(),
        "plan": res["plan"],
        "splits": res["splits"],
        "input_copies": res["input_copies"],
        "warmup_steps": res["warmup_steps"],
        "clock_warmup_s": CLOCK_WARMUP_S,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w.name, args.cpu_budget, log)
    line["others"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
