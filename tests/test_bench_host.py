"""bench.py's host-side helpers, on synthetic profiler output (no GPU): the
traffic conversion (copy calibration, dispatch selection, the sources hash
that invalidates a record), the bench line's phase split of a kernel trace,
and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KERNEL = "fwd_kernel<128, 2, 8, 0, false, true>"


def _pmc_dir(tmp, name, counter, rows):
    """rows: (kernel name, grid, value) in dispatch order."""
    d = tmp / name
    d.mkdir()
    with open(d / "pmc_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, g, v) in enumerate(rows):
            w.writerow([i + 1, g, f"void ns::{k}(p)", counter, v])
    return str(d)


def test_parse_slice():
    assert bench._parse_slice("") == slice(None)
    assert bench._parse_slice(":24") == slice(None, 24)
    assert bench._parse_slice("-10:") == slice(-10, None)
    assert bench._parse_slice("3:-2") == slice(3, -2)


def test_traffic_from_scales_by_the_copy_and_picks_dispatches(tmp_path):
    copy = 512 << 20
    cf = _pmc_dir(tmp_path, "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512, copy / 1024 / 2)] * 3)
    cw = _pmc_dir(tmp_path, "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 512, copy / 1024)] * 3)
    # alternating step-1 (100 KiB) / step-4 (300 KiB) launches, then 5 launches
    # of a loop (1000 KiB) that the slice must leave out
    seq = [100, 300] * 4 + [1000] * 5
    kf = _pmc_dir(tmp_path, "kf", "FETCH_SIZE", [(KERNEL, 512, v) for v in seq])
    kw = _pmc_dir(tmp_path, "kw", "WRITE_SIZE", [(KERNEL, 512, v / 10) for v in seq])
    out = tmp_path / "rec.json"
    bench.traffic_from(cf, cw, kf, kw, KERNEL, 2, None, "w", str(out), ":8")
    rec = json.load(open(out))
    assert rec["dispatches"] == [4, 4]
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(100 * 1024 * 2.0)
    assert rec["write_bytes_per_launch"] == pytest.approx(10 * 1024)
    # a record counts only while the kernel sources hash the same
    assert bench.measured_traffic(str(out)) == int(100 * 1024 * 2.0 + 10 * 1024)
    rec["sources_sha256"] = "0" * 64
    json.dump(rec, open(out, "w"))
    assert bench.measured_traffic(str(out)) is None
    assert bench.measured_traffic(str(tmp_path / "absent.json")) is None


def test_traffic_from_refuses_mixed_dispatches(tmp_path):
    cf = _pmc_dir(tmp_path, "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512, 1.0)])
    cw = _pmc_dir(tmp_path, "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 512, 1.0)])
    kf = _pmc_dir(tmp_path, "kf", "FETCH_SIZE", [(KERNEL, 512, 1.0)] * 3)   # not whole pairs
    kw = _pmc_dir(tmp_path, "kw", "WRITE_SIZE", [(KERNEL, 512, 1.0)] * 3)
    with pytest.raises(SystemExit):
        bench.traffic_from(cf, cw, kf, kw, KERNEL, 2, None, "w", str(tmp_path / "r.json"))


def test_trace_summary_splits_phases_by_the_lines_counts(tmp_path, capsys):
    steps, warm, nc, ng = 4, 2, 3, 5
    loops = {"fwd_kernel step 1": {"settle_calls": 6, "warm": warm, "timed": steps},
             "mass_kernel step 2": {"settle_calls": 7, "warm": warm, "timed": steps},
             "fwd_kernel step 4": {"settle_calls": 5, "warm": warm, "timed": steps},
             "decode_kernel step 5": {"settle_calls": 9, "warm": warm, "timed": steps}}
    line = {"metric": "m", "steps": steps, "warmup": warm, "clock_warmup": {"eager_steps": nc, "graph_replays": ng},
            "ms_per_step": 0.5, "ms_per_step_eager": 0.6, "ops_ms": {}, "kernel_loops": loops,
            "kernels_ms": {"fwd_kernel step 1": 0.0111, "mass_kernel step 2": 0.0222,
                           "fwd_kernel step 4": 0.0333, "decode_kernel step 5": 0.0444}}
    (tmp_path / "b.log").write_text("noise\n" + json.dumps(line) + "\n")
    step_kernels = [k for _, k, per in bench.STEP_KERNELS for _ in range(per)]
    # launch order of one step: prefill, merge, mass, reduce, top-k, fuse, kv_len, prefill, merge, decode, merge
    order = [bench.STEP_KERNELS[i][1] for i in (0, 1, 2, 3, 4, 5, 6, 0, 1, 7, 8)]
    assert sorted(order) == sorted(step_kernels)
    rows, t = [], 0

    def emit(name, us):
        nonlocal t
        rows.append((len(rows) + 1, f"void ns::{name}(p)", t, t + int(us * 1000)))
        t += int(us * 1000) + 1

    total = nc + warm + steps + 1 + 3 + ng + warm + steps
    for k in range(total):
        eager = nc + warm <= k < nc + warm + steps
        graph = k >= total - steps
        for i, name in enumerate(order):
            emit(name, 100 + i + (1 if eager else 2 if graph else 0))
    for lname, kern, us, extra in (("fwd_kernel step 1", order[0], 11, [order[1]]),
                                   ("mass_kernel step 2", order[2], 22, [order[3], order[4]]),
                                   (None, None, 0, []),
                                   ("fwd_kernel step 4", order[0], 33, [order[1]]),
                                   ("decode_kernel step 5", order[9], 44, [order[10]])):
        if lname is None:   # one more eager step between the loops
            for name in order:
                emit(name, 7)
            continue
        lp = loops[lname]
        for j in range(lp["settle_calls"] + lp["warm"] + lp["timed"]):
            emit(kern, us if j >= lp["settle_calls"] + lp["warm"] else 3)
            for e in extra:
                emit(e, 1)
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
                    "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        for r in rows:
            w.writerow(list(r) + [512, 1, 1])
    bench.trace_summary(str(d), str(tmp_path / "b.log"))
    out = capsys.readouterr().out.splitlines()
    cells = {}
    for l in out:
        if l.startswith("| |"):
            parts = [c.strip() for c in l.strip("|").split("|")]
            cells.setdefault(parts[1], parts)   # the prefill kernel's rows come first
    first, second = cells["first launch of the step"], cells["second launch of the step"]
    # eager timed: 101 us (prefill index 0 + 1), graph timed 102 us; loops 11 and 33 us
    assert first[3] == f"{steps} / 101.0" and first[4] == f"{steps} / 102.0"
    assert first[5] == f"{steps} / 11.0" and first[6] == "11.1"
    assert second[3] == f"{steps} / 108.0" and second[5] == f"{steps} / 33.0"
    mass = [l for l in out if l.startswith("| `mass_kernel")][0]
    assert f"{steps} / 22.0" in mass and "22.2" in mass
    dec = [l for l in out if l.startswith("| `decode_kernel")][0]
    assert f"{steps} / 44.0" in dec and f"{steps} / 110.0" in dec


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
