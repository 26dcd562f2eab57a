"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline
bound of each workload, and the readers that turn rocprofv3 CSV output into
the tables under profiles/ -- dispatches grouped by kernel and by sweep
point, counters averaged over the last dispatches, HBM bytes scaled by the
calibration copy."""

import csv
import io
import json
import os
import subprocess
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workload import get_workload  # noqa: E402

ATTN = "void gqa::(anonymous namespace)::attn_wide_dma<128>(gqa::AttnArgs)"
MERGE = "void gqa::(anonymous namespace)::lse_merge<unsigned short, 128, 8>(gqa::AttnArgs)"
COPY = "void at::native::elementwise_kernel<copy>(int)"


def _trace_csv(path, dispatches):
    """dispatches: (name, start_ns, end_ns) in any order."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, (n, s, e) in enumerate(dispatches):
            w.writerow(["KERNEL_DISPATCH", i + 1, n, s, e])


def _pmc_csv(path, rows):
    """rows: (dispatch id, kernel name, counter, value, start, end)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for r in rows:
            w.writerow(list(r))


def _out(fn, *a):
    buf = io.StringIO()
    with redirect_stdout(buf):
        fn(*a)
    return buf.getvalue()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,bound", [("decode_8k", "hbm"), ("mixed_32dec_64x4", "hbm"),
                                        ("fanout_8x20_32k", "mfma"), ("prefill_32k", "mfma"),
                                        ("join_400_32k", "mfma"), ("tiny_fp32_fanout", "hbm")])
def test_roofline_bound_follows_the_ridge(name, bound):
    """The bound is the roofline side of the workload's algorithmic
    intensity (FLOP per unique byte) against the ridge of its dtype's peak;
    achieved and frac are algorithmic work over T = attention + merge kernel
    time per forward, frac_attention over the attention launch alone, and
    frac_of_achievable over the probe-measured ceiling of the same kind."""
    w = get_workload(name)
    res = {"attn_kernel_ms": 0.4, "kernel_ms": 0.5, "timed_forwards": 50}
    ach = {"mfma_bf16_tflops": 2000.0, "hbm_read_gbps": 5000.0}
    r = bench.roofline_of(w, res, traffic=123, achievable=ach)
    assert r["bound"] == bound and r["traffic"] == 123
    if bound == "mfma":
        work, scale = w.flops(), 1e12
        assert r["peak"] == (bench.PEAK_BF16_TFLOPS if w.dtype == "bf16" else bench.PEAK_FP32_TFLOPS)
    else:
        work, scale = w.kv_bytes() + w.io_bytes(), 1e9
        assert r["peak"] == bench.PEAK_HBM_GBPS
    assert r["achieved"] == pytest.approx(work / 0.5e-3 / scale)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["frac_attention"] == pytest.approx(work / 0.4e-3 / scale / r["peak"])
    if w.dtype == "bf16" or bound == "hbm":
        key = "mfma_bf16_tflops" if bound == "mfma" else "hbm_read_gbps"
        assert r["frac_of_achievable"] == pytest.approx(r["achieved"] / ach[key])
    else:
        assert "frac_of_achievable" not in r


def test_kernel_summary_separates_the_last_calls(tmp_path):
    # 5 attention calls of 10, 10, 10, 20, 30 us (the last two are "timed").
    d = [(ATTN, 1000 * k, 1000 * k + us * 1000) for k, us in enumerate([10, 10, 10, 20, 30])]
    d += [(MERGE, 100 + 1000 * k, 100 + 1000 * k + 2000) for k in range(5)]
    p = tmp_path / "t.csv"
    _trace_csv(p, d[::-1])   # order in the file must not matter
    out = _out(bench.kernel_summary, str(p), 2)
    row = [l for l in out.splitlines() if "attn_wide_dma" in l][0].split("|")
    assert row[2].strip() == "5"
    assert float(row[3]) == pytest.approx(16.0)          # all calls
    assert float(row[4]) == pytest.approx(25.0)          # last 2
    assert float(row[6]) == pytest.approx(10.0)          # min


def test_trace_summary_assigns_dispatches_to_sweep_points(tmp_path):
    """Point 1 issues 3 forwards (attention + merge each), point 2 issues 2
    forwards without a merge launch; each point averages its last `timed`."""
    sweep = {"workload": "x", "points": [
        {"label": "a", "chosen": [4, 1], "forwards": 3, "timed": 2, "attn_us": 0, "merge_us": 0,
         "plan": {"n_items_wide": 10, "n_items_narrow": 0, "merge_launch": 1}},
        {"label": "b", "chosen": [1, 1], "forwards": 2, "timed": 1, "attn_us": 0, "merge_us": 0,
         "plan": {"n_items_wide": 10, "n_items_narrow": 0, "merge_launch": 0}}]}
    t, d = 0, []
    for us in (50, 40, 60):            # point a
        d.append((ATTN, t, t + us * 1000))
        d.append((MERGE, t + us * 1000, t + us * 1000 + 5000))
        t += 100_000
    for us in (70, 80):                # point b
        d.append((ATTN, t, t + us * 1000))
        t += 100_000
    d.append((COPY, 5, 6))             # other kernels are ignored
    sp, cp = tmp_path / "s.json", tmp_path / "t.csv"
    sp.write_text(json.dumps(sweep))
    _trace_csv(cp, d)
    out = _out(bench.trace_summary, str(sp), str(cp))
    rows = [l.split("|") for l in out.splitlines() if l.startswith("| a") or l.startswith("| b")]
    assert float(rows[0][3]) == pytest.approx(50.0) and float(rows[0][4]) == pytest.approx(5.0)
    assert float(rows[1][3]) == pytest.approx(80.0) and float(rows[1][4]) == pytest.approx(0.0)
    assert "mismatch" not in out


def test_counter_summary_means_over_last_dispatches(tmp_path):
    rows = []
    for disp, v in ((1, 100.0), (2, 200.0), (3, 400.0)):
        # one counter reported per XCD-like instance: the reader sums them
        rows += [(disp, ATTN, "SQ_BUSY_CYCLES", v / 2, 0, 1000), (disp, ATTN, "SQ_BUSY_CYCLES", v / 2, 0, 1000)]
    p = tmp_path / "pmc.csv"
    _pmc_csv(p, rows)
    out = _out(bench.counter_summary, str(p), 2)
    assert "SQ_BUSY_CYCLES = 300" in out
    assert "duration 1.00 us" in out


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """A 2^30-byte device copy reads FETCH_SIZE = 2^19 KiB (half the bytes,
    as the counter does on this chip): the fetch scale is then 2, and the
    attention kernel's 1000 KiB become 2,048,000 bytes."""
    fetch = [(1, COPY, "FETCH_SIZE", float(1 << 19), 0, 1), (2, ATTN, "FETCH_SIZE", 1000.0, 0, 1),
             (3, ATTN, "FETCH_SIZE", 1000.0, 0, 1), (4, MERGE, "FETCH_SIZE", 50.0, 0, 1)]
    write = [(1, COPY, "WRITE_SIZE", float(1 << 20), 0, 1), (2, ATTN, "WRITE_SIZE", 10.0, 0, 1),
             (3, ATTN, "WRITE_SIZE", 30.0, 0, 1), (4, MERGE, "WRITE_SIZE", 5.0, 0, 1)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _pmc_csv(fp, fetch)
    _pmc_csv(wp, write)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    for name in bench.KERNEL_SOURCES + bench.APPEND_SOURCES:
        src = tmp_path / name
        src.parent.mkdir(parents=True, exist_ok=True)
        src.write_text("kernel source")
    _out(bench.traffic_summary, str(fp), str(wp), "fanout", 2, "cmd-f", "cmd-w")
    t = json.loads((tmp_path / "profiles" / "traffic_fanout_8x20_32k.json").read_text())
    k = t["per_kernel"]["attn_wide_dma<128>"]
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert k["fetch_bytes"] == 2_048_000 and k["write_bytes"] == 20 * 1024
    m = t["per_kernel"]["lse_merge<unsigned short, 128, 8>"]
    assert m["fetch_bytes"] == 102_400 and m["write_bytes"] == 5 * 1024
    # the roofline's time covers the attention launches and the merge, and so do its bytes
    assert t["hbm_bytes_per_launch"] == 2_048_000 + 20 * 1024 + 102_400 + 5 * 1024
    assert t["kernel_hash"] == bench.kernel_hash() and t["command_fetch"] == "cmd-f"
