#!/usr/bin/env python3
"""Throughput of the position-independent attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input (long-context
query-centric fusion shape: 1 request, 32 reused 1024-token spans at shuffled
logical offsets + 256 own query tokens = 33,024 KV slots, 32 q / 8 kv heads,
d = 128, theta 5e5):
  1. pic_attn_prefill   attention of the 256 queries with RoPE in-kernel, O + LSE
  2. qc_score_select    per-key softmax mass from the same scores, top 15% per span
  3. kv_fuse_scatter    4,928 recomputed K/V rows into request-private blocks
  4. pic_attn_prefill   attention over the fused cache
  5. pic_attn_decode    one generated token over the fused cache
(plus one small device copy that restores the un-fused pi / kv_len so that
every step starts from the same cache).

The step is captured once as a HIP graph and replayed once per timed step
(each replay first checked bit for bit against an eager step); --no-graph
times it eagerly.  Before any timing the step runs eagerly for
--clock-warmup-s seconds: the GPU's clock rises over the first tens of
milliseconds of sustained load, and the W warm-up steps alone may end before
it settles.  Per-op times come from an eager run with events between the calls.
The step's working set (~200 MB) stays in the 256 MB Infinity Cache from step
to step: the headline is a warm figure.

metric: attended KV tokens per second, where each attention-type call over a
request attends its kv_len minus masked slots (33,024 here) and the step makes
four such calls.  The roofline object is for the dominant op (step 1,
MFMA-bound: visible (query, key) pairs x Hq x 4d flops against the bf16 dense
peak), timed with HIP events on the launch stream around the whole
pic_attn_prefill call (its partials kernel and the split merge).

Other lines (each a single-op timing with HIP events on the launch stream):
  shared_serving      pic_attn_prefill at 16 requests x 8,320 slots that read one
                      pool of 64 spans at different offsets (MFMA roofline)
  selection_64q       qc_score_select with the first 64 query tokens over the
                      long-context cache (K only: the HBM-leaning selection)
  decode_heavy        pic_attn_decode, 64 requests x 16,385 slots, 64 q / 8 kv
                      heads: on 64 private pools of 16 spans (4 GiB, the HBM
                      roofline) and on 16 shared spans (64 MiB unique, which the
                      Infinity Cache holds: cache-resident), the latter also
                      cold (a 1 GiB write evicts the caches before each call)
  sparse_recompute, anchor_extraction, rotation_ablation, block_hashing
cpu_baseline: the double-precision CPU oracle on a sample of step 1's rows,
timed before the GPU is touched, on 1 core and as N processes over
(kv head, query token) shards, scaled by visible (row, key) pairs to the step.
measured_peaks: a streaming HBM read, a bf16 MFMA loop and a v_exp_f32 loop on
the same GPU (libpicpeaks.so); roofline fractions are given against both the
vendor and the measured peaks.

    python bench.py [--steps K] [--warmup W]

HBM traffic (roofline.traffic) comes from two rocprofv3 counter runs
(FETCH_SIZE, WRITE_SIZE) of this script, each scaled by what the same counter
reads for a plain device copy of known size (--calibrate-copy);
--traffic-from turns the four runs into a JSON record under profiles/ holding
a hash of the kernel sources: the field is null once those sources differ.
"""
import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attended KV tokens/s + % of HBM/MFMA roofline (GQA 32q/8kv, d=128)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic.json")
# counter-derived HBM bytes per launch of the other lines' kernels (same format)
TRAFFIC_RECORDS = {name: os.path.join(ROOT, "profiles", f"{name}_traffic.json")
                   for name in ("decode_private", "decode_shared", "decode_shared_cold", "mass_long_context",
                                "mass_selection_64q")}
TRAFFIC_KERNEL = "fwd_kernel<128, 2, 8, 0, false, true>"
# the files whose change invalidates a traffic measurement of a kernel
TRAFFIC_SOURCES = ["position_independent_attention_amd/csrc/attn_fwd.hip",
                   "position_independent_attention_amd/csrc/attn_decode.hip",
                   "position_independent_attention_amd/csrc/pic_internal.h",
                   "position_independent_attention_amd/csrc/api.cpp",
                   "position_independent_attention_amd/build.py"]
PEAKS_LIB = os.path.join(ROOT, "position_independent_attention_amd", "libpicpeaks.so")
COPY_BYTES = 512 << 20
ANCHOR_RATIO = 0.05   # anchor fraction per span (the pages say only "a small fraction")
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
MAX_CPU_WORKERS = 16  # the CPU share of one GPU on the GPU hosts
LINES = ["step", "select_lse_null", "llama_layer", "shared_serving", "selection_64q", "decode", "recompute", "anchor",
         "ablation", "hashing"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(w):
    """Number of visible (query token, key) pairs per q head over all requests."""
    tot = 0
    for r in range(w.batch):
        pi = w.kv_pos[r, :w.kv_len[r]]
        pi = np.sort(pi[pi >= 0])
        qp = w.q_pos[w.q_start[r]:w.q_start[r + 1]]
        tot += int(np.searchsorted(pi, qp, side="right").sum())
    return tot


def attended_tokens(w):
    return int(sum(int((w.kv_pos[r, :w.kv_len[r]] >= 0).sum()) for r in range(w.batch)))


def sources_hash():
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE):
    """Bytes per launch from a traffic record, or None if absent or taken from
    other kernel sources."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_hash():
        return None
    return int(t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES, 10 times (for the counter
    calibration run)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes": COPY_BYTES, "launches": 10}), flush=True)


def _parse_slice(text):
    """'a:b' -> slice(a, b) (either side may be empty or negative)."""
    if not text:
        return slice(None)
    a, _, b = text.partition(":")
    return slice(int(a) if a else None, int(b) if b else None)


def _pmc(d, counter, name_part, every=1, grid=None, part=None):
    """Mean counter value over the dispatches of kernels named like name_part
    (and with that grid size, if given), in dispatch order: `part` (a slice)
    of them first, then every n-th from the first.  With every > 1 the
    dispatches must all have one grid size and come in whole groups of
    `every`."""
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                g = r.get("Grid_Size", "")
                if grid is None or g == str(grid):
                    rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), g))
    rows = sorted(rows)[part if part is not None else slice(None)]
    if every > 1 and (len({g for _, _, g in rows}) > 1 or len(rows) % every):
        raise SystemExit(f"{d}: {len(rows)} dispatches of '{name_part}' with grids {sorted({g for _, _, g in rows})}; "
                         "profile one line alone (--only)")
    rows = rows[::every]
    if not rows:
        raise SystemExit(f"no {counter} rows for '{name_part}' under {d}")
    return float(np.mean([v for _, v, _ in rows])), len(rows)


def traffic_from(copy_fetch, copy_write, fetch, write, kernel, every, grid, workload, out, part_text=""):
    """Scale a kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the
    reading of the same counters for the calibration copy."""
    part = _parse_slice(part_text)
    cf, _ = _pmc(copy_fetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = _pmc(copy_write, "WRITE_SIZE", "copyBuffer")
    kf, nf = _pmc(fetch, "FETCH_SIZE", kernel, every=every, grid=grid, part=part)
    kw, nw = _pmc(write, "WRITE_SIZE", kernel, every=every, grid=grid, part=part)
    ff, fw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    rec = {"kernel": kernel, "grid": grid, "workload": workload, "sources_sha256": sources_hash(),
           "dispatch_slice": part_text or ":", "every": every,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES,
           "fetch_scale": ff, "write_scale": fw,
           "kernel_fetch_kib": kf, "kernel_write_kib": kw, "dispatches": [nf, nw],
           "fetch_bytes_per_launch": kf * 1024.0 * ff, "write_bytes_per_launch": kw * 1024.0 * fw}
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec), flush=True)


# the step's kernels in launch order: (role, name part, launches per step)
STEP_KERNELS = [("step 1 prefill + step 4 prefill over the fused cache", "fwd_kernel<128, 2, 8, 0, false, true>", 2),
                ("prefill split merge (steps 1 and 4)", "merge_kernel<128>", 2),
                ("step 2 mass pass", "mass_kernel<128, 4, 8, true>", 1),
                ("step 2 column reduction", "mass_reduce_kernel", 1),
                ("step 2 per-span top-k", "span_topk_kernel", 1),
                ("step 3 kv_fuse_scatter", "fuse_kernel<128>", 1),
                ("step 3 kv_len update", "fuse_len_kernel", 1),
                ("step 5 decode (1 request)", "decode_kernel<128>", 1),
                ("step 5 decode merge", "merge_many_kernel<128>", 1)]


def trace_summary(trace_dir, bench_json):
    """Per-kernel durations of the long-context step from a rocprofv3 kernel
    trace of a bench.py run, split by phase with the counts that the run's own
    JSON line records: the eager timed steps, the timed graph replays and the
    timed calls of each op's own loop (the loop whose library events give the
    line's kernels_ms)."""
    line = None
    for text in open(bench_json):
        text = text.strip()
        if text.startswith("{") and '"metric"' in text:
            line = json.loads(text)
    if line is None:
        raise SystemExit(f"no bench JSON line in {bench_json}")
    steps, warm = line["steps"], line["warmup"]
    n_clock = line["clock_warmup"]["eager_steps"]
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    disp = []
    for f in files:
        for r in csv.DictReader(open(f)):
            disp.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                         int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])))
    disp.sort()

    def launches(part, grid_of_first=False):
        ds = [d for d in disp if part in d[1]]
        if grid_of_first and ds:
            ds = [d for d in ds if d[3] == ds[0][3]]
        return np.array([d[2] for d in ds]) / 1e3

    # launches of each of the step's kernels, in order: clock warm-up, warm-up
    # and timed eager steps, the eager reference of the graph check, 3 checked
    # replays, clock warm-up replays, warm-up and timed replays; then the
    # kernel loops (settling, warm-up and timed calls of one op each; the
    # fused-cache loops come after one more eager step)
    eager0 = n_clock + warm
    graph0 = eager0 + steps + 1 + 3 + line["clock_warmup"]["graph_replays"] + warm
    step_end = graph0 + steps
    loops = line.get("kernel_loops", {})

    def loop_range(name, before):
        lp = loops.get(name)
        if not lp:
            return None
        a = before + lp["settle_calls"] + lp["warm"]
        return a, a + lp["timed"]

    L = {k: (v["settle_calls"] + v["warm"] + v["timed"]) for k, v in loops.items()}
    # dispatch index ranges of the timed loop calls, per kernel
    loop_ranges = {
        "fwd_kernel step 1": loop_range("fwd_kernel step 1", 2 * step_end),
        "mass_kernel step 2": loop_range("mass_kernel step 2", step_end),
        "fwd_kernel step 4": loop_range("fwd_kernel step 4", 2 * step_end + L.get("fwd_kernel step 1", 0) + 2)
        if loops else None,
        "decode_kernel step 5": loop_range("decode_kernel step 5", step_end + 1),
    }
    out = ["| kernel | role | per step | eager timed steps: n / avg us | timed graph replays: n / avg us | "
           "timed calls of its own loop: n / avg us | library events, same loop: avg us |",
           "|---|---|---|---|---|---|---|"]
    kms = line.get("kernels_ms", {})

    def cell(x):
        return f"{len(x)} / {x.mean():.1f}" if len(x) else "-"

    for role, part, per in STEP_KERNELS:
        us = launches(part, grid_of_first=part == "decode_kernel<128>")
        if not len(us):
            out.append(f"| `{part}` | {role} | {per} | 0 | | | |")
            continue
        eg = us[eager0 * per:(eager0 + steps) * per]
        gr = us[graph0 * per:(graph0 + steps) * per]
        if per == 2:
            out.append(f"| `{part}` | {role} | {per} | {cell(eg)} | {cell(gr)} | | |")
            for k, (name, lname) in enumerate((("first launch of the step", "fwd_kernel step 1"),
                                               ("second launch of the step", "fwd_kernel step 4"))):
                rg = loop_ranges.get(lname) if part.startswith("fwd_kernel") else None
                lp = us[rg[0]:rg[1]] if rg else np.array([])
                ev = f"{1e3 * kms[lname]:.1f}" if rg and lname in kms else ""
                out.append(f"| | {name} | 1 | {cell(eg[k::2])} | {cell(gr[k::2])} | {cell(lp) if rg else ''} | "
                           f"{ev} |")
        else:
            lname = {"mass_kernel<128, 4, 8, true>": "mass_kernel step 2",
                     "decode_kernel<128>": "decode_kernel step 5"}.get(part)
            rg = loop_ranges.get(lname) if lname else None
            lp = us[rg[0]:rg[1]] if rg else np.array([])
            ev = f"{1e3 * kms[lname]:.1f}" if lname in kms else "-"
            out.append(f"| `{part}` | {role} | {per} | {cell(eg)} | {cell(gr)} | {cell(lp) if rg else ''} | "
                       f"{ev if rg else ''} |")
    out.append("")
    out.append(f"bench line: ms_per_step {line.get('ms_per_step')} (graph), ms_per_step_eager "
               f"{line.get('ms_per_step_eager')}, ops_ms {json.dumps(line.get('ops_ms'))}; counts: clock warm-up "
               f"{n_clock} eager steps, {warm} warm-up + {steps} timed eager steps, 1 eager reference + 3 checked "
               f"replays, {line['clock_warmup']['graph_replays']} clock warm-up replays, {warm} warm-up + {steps} "
               f"timed replays; kernel loops {json.dumps(loops)}")
    print("\n".join(out), flush=True)


# ------------------------------------------------------------ CPU baseline

_CPU_W = None   # the workload the forked oracle workers read


def _oracle_rows(rows):
    import oracle
    t, h = rows
    oracle.attention(_CPU_W, (t, h))
    return len(t)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baselines(w, one_tokens, all_tokens, step_pairs, step_tokens):
    """The oracle as it stands, on step 1's first query tokens at the full
    context: one process on 1 core, then N processes over (kv head, token)
    shards.  Runs before the GPU is initialised, so the workers are plain
    forks of a CPU-only process."""
    import multiprocessing as mp
    import oracle
    global _CPU_W
    _CPU_W = w
    oracle.lib()
    G = w.num_q_heads // w.num_kv_heads
    pi = np.sort(w.kv_pos[0, :w.kv_len[0]][w.kv_pos[0, :w.kv_len[0]] >= 0])

    def pairs_of(nt):
        return int(np.searchsorted(pi, w.q_pos[:nt], side="right").sum()) * w.num_q_heads

    nt = min(one_tokens, w.total_q)
    ts = np.repeat(np.arange(nt), w.num_q_heads).astype(np.int32)
    hs = np.tile(np.arange(w.num_q_heads), nt).astype(np.int32)
    try:
        allowed = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(allowed)})
        pinned = True
    except (AttributeError, OSError):
        allowed, pinned = None, False
    c0 = time.perf_counter()
    oracle.attention(w, (ts, hs))
    one_s = time.perf_counter() - c0
    if pinned:
        os.sched_setaffinity(0, allowed)
    aff = len(allowed) if allowed else (os.cpu_count() or 1)
    n = max(1, min(os.cpu_count() or 1, aff, MAX_CPU_WORKERS))
    na = min(all_tokens, w.total_q)
    # shards: one kv head's q heads over a contiguous run of tokens
    shards = []
    per = max(1, (na * w.num_kv_heads + n - 1) // n)
    units = [(g, t) for g in range(w.num_kv_heads) for t in range(na)]
    for s in range(0, len(units), per):
        chunk = units[s:s + per]
        t = np.repeat([u[1] for u in chunk], G).astype(np.int32)
        h = np.concatenate([np.arange(u[0] * G, (u[0] + 1) * G) for u in chunk]).astype(np.int32)
        shards.append((t, h))
    ctx = mp.get_context("fork")
    with ctx.Pool(n) as pool:
        pool.map(_oracle_rows, [(np.zeros(1, np.int32), np.zeros(1, np.int32))] * n)   # workers up
        c0 = time.perf_counter()
        pool.map(_oracle_rows, shards, chunksize=1)
        all_s = time.perf_counter() - c0
    one_rate = step_tokens / (one_s * step_pairs / pairs_of(nt))
    all_rate = step_tokens / (all_s * step_pairs / pairs_of(na))
    return {
        "value": round(one_rate, 2), "unit": "attended KV tokens/s", "cores": 1, "kind": "oracle",
        "sample": f"oracle.attention on {nt} query tokens x {w.num_q_heads} heads of step 1 at the full "
                  f"33,024-slot context ({one_s:.1f} s, pinned to one core: {pinned}), scaled by visible "
                  "(row, key) pairs to the whole step",
        "all_cores": {"value": round(all_rate, 2), "unit": "attended KV tokens/s", "cores": n,
                      "processes": n, "os_cpu_count": os.cpu_count(), "affinity_cpus": aff,
                      "cpu_model": cpu_model(),
                      "sample": f"{na} query tokens x {w.num_q_heads} heads of step 1 in {len(shards)} "
                                f"(kv head, token) shards over {n} processes ({all_s:.2f} s wall), "
                                "scaled by visible (row, key) pairs"}}


# ------------------------------------------------------------------ peaks

def measure_peaks():
    if not os.path.exists(PEAKS_LIB):
        return None
    h = ctypes.CDLL(PEAKS_LIB)
    h.pic_peak_hbm_read.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    h.pic_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    h.pic_peak_exp2.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    v = ctypes.c_double(0)
    out = {}
    assert h.pic_peak_hbm_read(4 << 30, 5, ctypes.byref(v)) == 0
    out["hbm_read_gbs"] = round(v.value, 1)
    best = 0.0
    for shape, iters in ((16, 20000), (32, 10000)):
        assert h.pic_peak_mfma_bf16(shape, iters, ctypes.byref(v)) == 0
        out[f"mfma_bf16_{shape}x{shape}_tflops"] = round(v.value, 1)
        best = max(best, v.value)
    out["mfma_bf16_tflops"] = round(best, 1)
    assert h.pic_peak_exp2(5000, ctypes.byref(v)) == 0
    out["exp2_gexp_per_s"] = round(v.value, 1)
    out["what"] = ("streaming read of 4 GiB (16-byte loads), register-resident bf16 MFMA loops at 8 waves per "
                   "SIMD (best of 16x16x32 and 32x32x16), v_exp_f32 chains; measured on this GPU in this run")
    return out


def roof(bound, achieved, peak, unit, measured_peak=None, **extra):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4)}
    if measured_peak:
        r["measured_peak"] = measured_peak
        r["frac_of_measured"] = round(achieved / measured_peak, 4)
    r.update(extra)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--clock-warmup-s", type=float, default=1.0,
                    help="seconds of eager steps before any timing (the clock settles under load)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32)
    ap.add_argument("--cpu-all-tokens", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--only", default=",".join(LINES),
                    help="comma-separated lines to run: " + ", ".join(LINES))
    ap.add_argument("--no-graph", action="store_true", help="time the step eagerly, without a HIP graph")
    ap.add_argument("--decode-pools", default="private,shared",
                    help="decode lines to run: private (4 GiB pool), shared (64 MiB pool)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the device copy the traffic counters are scaled by")
    ap.add_argument("--traffic-from", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                    help="rocprofv3 --pmc output dirs -> a traffic record (see --traffic-*)")
    ap.add_argument("--traffic-kernel", default=TRAFFIC_KERNEL)
    ap.add_argument("--traffic-every", type=int, default=2,
                    help="take every n-th dispatch of the kernel (the step launches the prefill twice)")
    ap.add_argument("--traffic-grid", type=int, default=None)
    ap.add_argument("--traffic-workload", default="long_context_qc_fusion step 1 (pic_attn_prefill)")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE)
    ap.add_argument("--traffic-slice", default="",
                    help="python slice 'a:b' of the kernel's dispatches (in order) to average, before --traffic-every")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_OUTPUT"),
                    help="per-phase durations of the step's kernels from a kernel trace of a bench.py run "
                         "and that run's output")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from, args.traffic_kernel, args.traffic_every, args.traffic_grid,
                     args.traffic_workload, args.traffic_out, args.traffic_slice)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (requests and kv heads "
              "shard without exchange; a split KV range needs one exchange of partial O + LSE); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    only = set(x.strip() for x in args.only.split(",") if x.strip())
    bad = only - set(LINES)
    if bad:
        raise SystemExit(f"unknown --only lines {sorted(bad)}; choose from {LINES}")

    from position_independent_attention_amd import workloads as W

    t0 = time.time()
    w = W.long_context()
    log(f"workload built in {time.time() - t0:.1f}s: kv_len {w.max_kv_len}, q {w.total_q}")
    tokens = attended_tokens(w)
    step_tokens = 4 * tokens
    pairs = visible_pairs(w)
    cpu = None
    if not args.no_cpu_baseline and not args.calibrate_copy:
        step_pairs = 3 * pairs * w.num_q_heads + tokens * w.num_q_heads   # 3 prefill-shaped passes + decode
        cpu = cpu_baselines(w, args.cpu_sample_tokens, args.cpu_all_tokens, step_pairs, step_tokens)
        log("cpu baseline:", cpu["value"], "1 core;", cpu["all_cores"]["value"], cpu["all_cores"]["cores"], "cores")

    import torch
    from position_independent_attention_amd import pic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    peaks = None if args.no_peaks else measure_peaks()
    if peaks:
        log("measured peaks:", peaks)
    mp_tf = peaks["mfma_bf16_tflops"] if peaks else None
    mp_hbm = peaks["hbm_read_gbs"] if peaks else None

    def settle(fn, seconds):
        """Run fn back to back for `seconds` (the clock rises under load and
        drops when the GPU idles, e.g. between timed sections)."""
        c0, n = time.perf_counter(), 0
        while time.perf_counter() - c0 < seconds:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            n += 10
        return n

    def time_calls(fn, reps=10, warm=2, settle_s=0.3, kctx=None, info=None):
        """Mean ms per call over `reps` back-to-back calls; with kctx (the
        calls' context) also the mean ms of the call's main kernel, from the
        event pair the library has stamped with that kernel's start and end in
        the same timed loop.  info (a dict)
        receives the call counts: settling, warm-up, timed."""
        n_settle = settle(fn, settle_s)
        if info is not None:
            info.update(settle_calls=n_settle, warm=warm, timed=reps)
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if kctx is not None:
            pic.pic_timing_start(kctx, reps)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        call_ms = a.elapsed_time(b) / reps
        if kctx is None:
            return call_ms
        kms, _ = pic.pic_timing_stop(kctx, reps)
        assert len(kms) == reps, (len(kms), reps)
        return call_ms, float(np.mean(kms))

    def graph_ms(fn, outs, calls=20, reps=10):
        """GPU time per call with the host's launch work taken out: `calls`
        back-to-back calls fn(stream) captured as one HIP graph, replayed after
        0.3 s of settling and timed with events over `reps` replays.  None if
        any of three replays leaves outputs that differ bit for bit from an
        eager call's (with eager work and synchronisations in between)."""
        fn(stream)
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for _ in range(calls):
                fn(cs)
        for _ in range(3):
            for o in outs:
                o.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
                log("graph replay differed from the eager call: no graph timing")
                return None
        settle(g.replay, 0.3)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / (reps * calls)

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    ctx = pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position)
    sel_off = pic.pic_select_offsets(w.span_len, w.ratio)
    nsel = int(sel_off[-1])
    dc = pic.to_device(w, dev, sel_off=sel_off)
    kv0 = dc.max_kv_len
    kv_fused = ((kv0 + 15) // 16) * 16 + nsel
    # pi and kv_len live in one buffer, so that one copy restores the un-fused
    # cache before every step
    npos = dc.kv_pos.numel()
    state0 = torch.cat([dc.kv_pos.reshape(-1), dc.kv_len.reshape(-1)])
    state = state0.clone()
    dc.kv_pos = state[:npos].view(dc.kv_pos.shape)
    dc.kv_len = state[npos:]
    kv_pos0 = state0[:npos].view(dc.kv_pos.shape)

    out1 = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.int16, device=dev)
    lse1 = torch.empty((w.total_q, w.num_q_heads), dtype=torch.float32, device=dev)
    out2 = torch.empty_like(out1)
    sel = torch.empty(nsel, dtype=torch.int32, device=dev)
    req_off = t(np.array([0, nsel], np.int32))
    fk, fv = t(w.fresh_k[:nsel]), t(w.fresh_v[:nsel])
    q_dec = dc.q[-1:].clone()
    qpos_dec = t(np.array([int(w.q_pos[-1]) + 1], np.int32))
    out3 = torch.empty_like(q_dec)
    dcd = pic.DeviceCache(dc.pool_k, dc.pool_v, dc.block_table, dc.kv_len, dc.kv_pos, kv_fused)

    req_fused = pic.PicReqTable(1, dc.block_table.shape[1], kv_fused, 0, 0, 0)
    need = max(
        pic.pic_workspace_bytes(ctx, pic.PIC_OP_PREFILL, dc.req(), dc.total_q, dc.max_q_len),
        pic.pic_workspace_bytes(ctx, pic.PIC_OP_PREFILL, req_fused, dc.total_q, dc.max_q_len),
        pic.pic_workspace_bytes(ctx, pic.PIC_OP_SELECT, dc.req(), dc.total_q, dc.max_q_len),
        pic.pic_workspace_bytes(ctx, pic.PIC_OP_DECODE, req_fused, 0, 0))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    names = ["prefill", "select", "fuse", "prefill_fused", "decode"]

    def step(evs=None, st=None):
        st = stream if st is None else st
        state.copy_(state0)
        dc.max_kv_len = kv0
        if evs: evs[0].record(st)
        pic.pic_attn_prefill(ctx, dc, out1, lse1, ws=ws, stream=st)
        if evs: evs[1].record(st)
        pic.qc_score_select(ctx, dc, lse1, nsel, sel, None, ws=ws, stream=st)
        if evs: evs[2].record(st)
        pic.kv_fuse_scatter(ctx, dc, sel, req_off, fk, fv, nsel, nsel, stream=st)
        if evs: evs[3].record(st)
        dc.max_kv_len = kv_fused
        pic.pic_attn_prefill(ctx, dc, out2, None, ws=ws, stream=st)
        if evs: evs[4].record(st)
        pic.pic_attn_decode(ctx, dcd, q_dec, qpos_dec, out3, None, ws=ws, stream=st)
        if evs: evs[5].record(st)

    # clock warm-up: eager steps for a fixed time before anything is timed
    n_clock = settle(step, args.clock_warmup_s)
    log(f"clock warm-up: {n_clock} eager steps")

    result = {"metric": METRIC, "value": None, "unit": "attended KV tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup}
    if "step" in only:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(args.steps):
            step(evs[k])
        stop.record(stream)
        torch.cuda.synchronize()
        ms_eager = start.elapsed_time(stop) / args.steps
        op_ms = {n: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
                 for i, n in enumerate(names)}
        log("per-op ms:", {k: round(v, 4) for k, v in op_ms.items()})

        # The same step captured once as a HIP graph and replayed K times: a
        # replay drops the launches' host-side work and most of the gaps between
        # them.  Every replay is first checked bit for bit against an eager step
        # (with eager work and synchronisations in between).
        ms_graph, graph_note, n_clock_graph = None, "off", 0
        if not args.no_graph:
            outs = (out1, lse1, sel, out2, out3)
            step()
            torch.cuda.synchronize()
            ref = [o.clone() for o in outs]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(st=torch.cuda.current_stream())
            same = True
            for _ in range(3):
                for o in outs:
                    o.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                same = same and all(torch.equal(o, r) for o, r in zip(outs, ref))
            if same:
                # the capture and the checks left the GPU idle: warm up again
                n_clock_graph = settle(g.replay, args.clock_warmup_s)
                for _ in range(args.warmup):
                    g.replay()
                torch.cuda.synchronize()
                start.record(stream)
                for _ in range(args.steps):
                    g.replay()
                stop.record(stream)
                torch.cuda.synchronize()
                ms_graph = start.elapsed_time(stop) / args.steps
                graph_note = "hip graph, one replay per step (replays checked bitwise against an eager step)"
            else:
                graph_note = "graph replay differed from the eager step: eager timing reported"
                log(graph_note)
            del g
        # The main kernel of each op, timed by the event pair the library has
        # stamped with its start and end, in back-to-back calls of that op on
        # the step's own inputs (the
        # eager step loop above is host-bound on slow hosts: its gaps let the
        # clock drop).
        state.copy_(state0)
        dc.max_kv_len = kv0
        kern, calls, loops = {}, {}, {}
        kfns = [("fwd_kernel step 1", lambda: pic.pic_attn_prefill(ctx, dc, out1, lse1, ws=ws, stream=stream)),
                ("mass_kernel step 2", lambda: pic.qc_score_select(ctx, dc, lse1, nsel, sel, None, ws=ws,
                                                                   stream=stream)),
                ("fwd_kernel step 4", lambda: pic.pic_attn_prefill(ctx, dc, out2, None, ws=ws, stream=stream)),
                ("decode_kernel step 5", lambda: pic.pic_attn_decode(ctx, dcd, q_dec, qpos_dec, out3, None, ws=ws,
                                                                     stream=stream))]
        for i, (kname, fn) in enumerate(kfns):
            if i == 2:
                step()   # leaves the fused cache
            loops[kname] = {}
            calls[kname], kern[kname] = time_calls(fn, reps=args.steps, warm=args.warmup, kctx=ctx,
                                                   info=loops[kname])
        log("kernel ms:", {k: round(v, 4) for k, v in kern.items()})
        kern_ms = kern
        ms_per_step = ms_graph if ms_graph is not None else ms_eager
        value = step_tokens / (ms_per_step / 1e3)
        flops = pairs * w.num_q_heads * 4 * w.head_dim
        achieved = flops / (kern_ms["fwd_kernel step 1"] / 1e3) / 1e12
        result.update({
            "value": round(value, 1), "ms_per_step": round(ms_per_step, 5),
            "ms_per_step_eager": round(ms_eager, 5), "launch": graph_note,
            "clock_warmup": {"seconds": args.clock_warmup_s, "eager_steps": n_clock,
                             "graph_replays": n_clock_graph if ms_graph is not None else 0,
                             "what": "untimed steps run back to back for that long before the W warm-up "
                                     "steps of each timed loop"},
            "cache_state": "warm: the step's ~200 MB working set stays in the 256 MB Infinity Cache between steps",
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "long_context_qc_fusion", "batch": 1, "kv_slots": int(w.max_kv_len),
                       "spans": "32 x 1024 reused at shuffled offsets", "query_tokens": int(w.total_q),
                       "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                       "rope_theta": w.rope_theta, "select_ratio": w.ratio, "fused_rows": nsel,
                       "step": "prefill+lse, qc_score_select, kv_fuse_scatter, prefill(fused), decode(1)"},
            "roofline": roof("mfma", achieved, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                             traffic=measured_traffic(),
                             kernel="fwd_kernel<128, 2, 8, 0, false, true>, step 1 (pic_attn_prefill's split "
                                    "partials; the merge kernel after it is not included)",
                             algorithmic_flops=flops, avg_ms=round(kern_ms["fwd_kernel step 1"], 5),
                             qk_pairs_per_s=round(pairs * w.num_q_heads / (kern_ms["fwd_kernel step 1"] / 1e3), 1),
                             timing=f"HIP events stamped at the kernel's own start and end (the library launches "
                                    f"it with hipExtLaunchKernelGGL while timing is on), over {args.steps} "
                                    f"back-to-back step-1 prefill calls",
                             call=roof("mfma", flops / (calls["fwd_kernel step 1"] / 1e3) / 1e12, PEAK_BF16_TFLOPS,
                                       "TFLOP/s", mp_tf, avg_ms=round(calls["fwd_kernel step 1"], 5),
                                       what="the whole pic_attn_prefill call (kernel + split merge), same calls")),
            "ops_ms": {k: round(v, 5) for k, v in op_ms.items()},
            "kernels_ms": {k: round(v, 5) for k, v in kern_ms.items()},
            "kernel_calls_ms": {k: round(v, 5) for k, v in calls.items()},
            "kernel_loops": loops,
            "select_mass_kernel_traffic": measured_traffic(TRAFFIC_RECORDS["mass_long_context"])})
    else:
        result.update({"higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                       "data": "synthetic", "config": {"workload": "long_context_qc_fusion"}})
    if peaks:
        result["measured_peaks"] = peaks

    if "select_lse_null" in only:
        # qc_score_select with no caller LSE: the K-only LSE pass (split
        # partials + merge) runs first, then the mass pass, the column reduction
        # and the top-k; both passes read K only
        state.copy_(state0)
        dc.max_kv_len = kv0
        msn, kmn = time_calls(lambda: pic.qc_score_select(ctx, dc, None, nsel, sel, None, ws=ws, stream=stream),
                              reps=args.steps, warm=args.warmup, kctx=ctx)
        qk2 = 2 * pairs * w.num_q_heads * 2 * w.head_dim
        result["select_lse_null"] = {
            "workload": "qc_score_select of the long-context step's 256 query tokens with lse = NULL "
                        "(the selection computes its own LSE), top 15% per span",
            "ms_per_call": round(msn, 5), "mass_kernel_ms": round(kmn, 5),
            "roofline": roof("mfma", qk2 / (msn / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                             algorithmic_flops=qk2, avg_ms=round(msn, 5),
                             note="QK^T twice (the LSE pass and the mass pass) over the whole call; "
                                  "the exp count is the same twice, 2 x 269.5 M")}

    if "llama_layer" in only:
        # One Llama-3-8B-like layer: 64 query tokens over a 64-token private
        # prefix and eight reused 512-token spans (4,224 slots), 32 q / 8 kv heads
        wl = W.llama_layer()
        dl = pic.to_device(wl, dev)
        ol = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device=dev)
        ll = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device=dev)
        wsl = torch.empty(max(1, pic.pic_workspace_bytes(ctx, pic.PIC_OP_PREFILL, dl.req(), wl.total_q,
                                                         wl.max_q_len)), dtype=torch.uint8, device=dev)
        lfn = lambda st=stream: pic.pic_attn_prefill(ctx, dl, ol, ll, ws=wsl, stream=st)
        ml, kl = time_calls(lfn, reps=50, warm=5, kctx=ctx)
        lg = graph_ms(lfn, (ol, ll))   # the call's GPU time without the host's launch work
        tl, pl = attended_tokens(wl), visible_pairs(wl)
        fl = pl * wl.num_q_heads * 4 * wl.head_dim
        kvb = tl * wl.num_kv_heads * wl.head_dim * 2 * 2
        result["llama_layer"] = {
            "workload": f"1 request, {tl} KV slots (64-token private prefix + 8 x 512 reused spans) + "
                        f"{wl.total_q} query tokens, 32 q / 8 kv heads, d 128: pic_attn_prefill with lse",
            "ms_per_call": round(ml, 5), "kernel_ms": round(kl, 5),
            "graph_ms_per_call": round(lg, 5) if lg is not None else None,
            "attended_kv_tokens_per_s": round(tl / ((lg if lg is not None else ml) / 1e3), 1),
            "roofline": roof("mfma", fl / (kl / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                             algorithmic_flops=fl, avg_ms=round(kl, 5), kernel="the prefill kernel",
                             qk_pairs_per_s=round(pl * wl.num_q_heads / (kl / 1e3), 1),
                             note="near the MFMA/HBM ridge and launch-bound at one request"),
            "hbm": roof("hbm", kvb / (kl / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s", mp_hbm, algorithmic_bytes=kvb,
                        avg_ms=round(kl, 5))}
        del dl, ol, ll, wsl

    ablation = None
    if "ablation" in only:
        # Rotation-overhead ablation (MiniPIC reports 5.7% end to end): the same
        # prefill call with keys_prerotated = 1, i.e. the keys used as stored.  It
        # runs on the same pool bytes: the kernels' work does not depend on the
        # key values.
        state.copy_(state0)
        dc.max_kv_len = kv0
        ctx_pr = pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position,
                             keys_prerotated=True)
        t_rot, k_rot = time_calls(lambda: pic.pic_attn_prefill(ctx, dc, out1, lse1, ws=ws, stream=stream),
                                  kctx=ctx)
        t_pre, k_pre = time_calls(lambda: pic.pic_attn_prefill(ctx_pr, dc, out1, lse1, ws=ws, stream=stream),
                                  kctx=ctx_pr)
        ctx_pr.close()
        ablation = {"what": "same kernels with keys stored rotated (keys_prerotated = 1) vs rotated in-kernel "
                            "at each key's logical position; timed on the same bytes",
                    "prefill_step1_ms": {"in_kernel": round(t_rot, 5), "prerotated": round(t_pre, 5),
                                         "overhead": round(t_rot / t_pre - 1.0, 4)},
                    "prefill_step1_kernel_ms": {"in_kernel": round(k_rot, 5), "prerotated": round(k_pre, 5),
                                                "overhead": round(k_rot / k_pre - 1.0, 4)}}
        result["rotation_ablation"] = ablation

    if "selection_64q" in only:
        # The selection with the first 64 query tokens over the long-context
        # cache: K only (QCFuse's selection pass reads no V), 256 rows per kv
        # head, where its work per K byte is near the HBM/MFMA ridge.
        w64 = W.long_context(q_len=64)
        s_off = pic.pic_select_offsets(w64.span_len, w64.ratio)
        n64 = int(s_off[-1])
        d64 = pic.to_device(w64, dev, sel_off=s_off)
        o64 = torch.empty((w64.total_q, w64.num_q_heads, w64.head_dim), dtype=torch.int16, device=dev)
        l64 = torch.empty((w64.total_q, w64.num_q_heads), dtype=torch.float32, device=dev)
        ws64 = torch.empty(max(pic.pic_workspace_bytes(ctx, pic.PIC_OP_PREFILL, d64.req(), 64, 64),
                               pic.pic_workspace_bytes(ctx, pic.PIC_OP_SELECT, d64.req(), 64, 64)),
                           dtype=torch.uint8, device=dev)
        pic.pic_attn_prefill(ctx, d64, o64, l64, ws=ws64, stream=stream)
        s64 = torch.empty(n64, dtype=torch.int32, device=dev)
        sfn = lambda st=stream: pic.qc_score_select(ctx, d64, l64, n64, s64, None, ws=ws64, stream=st)
        sms, skms = time_calls(sfn, reps=20, warm=3, kctx=ctx)
        sg = graph_ms(sfn, (s64,))   # the call's GPU time without the host's launch work
        scall = sg if sg is not None else sms
        tok64 = attended_tokens(w64)
        kbytes = tok64 * w64.num_kv_heads * w64.head_dim * 2
        p64 = visible_pairs(w64)
        qk_flops = p64 * w64.num_q_heads * 2 * w64.head_dim
        result["selection_64q"] = {
            "workload": f"qc_score_select (caller's lse) of 64 query tokens over the {w64.max_kv_len}-slot "
                        "long-context cache, top 15% per span",
            "ms_per_call": round(sms, 5), "graph_ms_per_call": round(sg, 5) if sg is not None else None,
            "attended_kv_tokens_per_s": round(tok64 / (scall / 1e3), 1),
            "roofline": roof("hbm", kbytes / (skms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s", mp_hbm,
                             algorithmic_bytes=kbytes, avg_ms=round(skms, 5),
                             traffic=measured_traffic(TRAFFIC_RECORDS["mass_selection_64q"]),
                             kernel="mass_kernel<128, 2, 8, true> (the mass pass; K only, read once)",
                             call=roof("hbm", kbytes / (scall / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s", mp_hbm,
                                       avg_ms=round(scall, 5),
                                       what="the whole qc_score_select call (mass pass, column reduction, "
                                            "top-k), GPU time per call from graph replays of 20 calls")),
            "mfma": roof("mfma", qk_flops / (skms / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                         algorithmic_flops=qk_flops, avg_ms=round(skms, 5), kernel="mass_kernel")}
        del d64, o64, l64, ws64, s64

    if "shared_serving" in only:
        # Shared-span serving: 16 requests, each 8 spans of a 64-span pool in its
        # own order (the same blocks at different offsets), 128 queries each.
        wss = W.shared_serving()
        dss = pic.to_device(wss, dev)
        oss = torch.empty((wss.total_q, wss.num_q_heads, wss.head_dim), dtype=torch.int16, device=dev)
        lss = torch.empty((wss.total_q, wss.num_q_heads), dtype=torch.float32, device=dev)
        wsss = torch.empty(max(1, pic.pic_workspace_bytes(ctx, pic.PIC_OP_PREFILL, dss.req(), wss.total_q,
                                                          wss.max_q_len)), dtype=torch.uint8, device=dev)
        ms_ss, k_ss = time_calls(lambda: pic.pic_attn_prefill(ctx, dss, oss, lss, ws=wsss, stream=stream),
                                 reps=20, kctx=ctx)
        pss = visible_pairs(wss)
        fl = pss * wss.num_q_heads * 4 * wss.head_dim
        tss = attended_tokens(wss)
        result["shared_serving"] = {
            "workload": "16 requests x 8,320 slots (8 of 64 pooled 1024-token spans each, at their own offsets) "
                        "+ 128 queries each, 32 q / 8 kv heads, d 128: pic_attn_prefill with lse",
            "ms_per_call": round(ms_ss, 5), "attended_kv_tokens_per_s": round(tss / (ms_ss / 1e3), 1),
            "roofline": roof("mfma", fl / (k_ss / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                             algorithmic_flops=fl, avg_ms=round(k_ss, 5), kernel="the prefill kernel",
                             qk_pairs_per_s=round(pss * wss.num_q_heads / (k_ss / 1e3), 1),
                             call=roof("mfma", fl / (ms_ss / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                                       avg_ms=round(ms_ss, 5), what="the whole pic_attn_prefill call"))}
        del dss, oss, lss, wsss

    if "recompute" in only:
        # Discrete-token recompute (QCFuse's sparse recompute): the 4,928 selected
        # tokens as queries at their own logical positions over the fused cache.
        step()   # leaves the fused cache and this step's selection in `sel`
        torch.cuda.synchronize()
        pos_r = np.sort(kv_pos0.cpu().numpy()[0, sel.cpu().numpy()]).astype(np.int32)
        qr = t(W.fresh_queries(nsel, w.num_q_heads, w.head_dim, seed=7))
        dcr = pic.DeviceCache(dc.pool_k, dc.pool_v, dc.block_table, dc.kv_len, dc.kv_pos, kv_fused,
                              q=qr, q_start=t(np.array([0, nsel], np.int32)), q_pos=t(pos_r),
                              total_q=nsel, max_q_len=nsel)
        outr = torch.empty((nsel, w.num_q_heads, w.head_dim), dtype=torch.int16, device=dev)
        wsr = torch.empty(max(1, pic.pic_workspace_bytes(ctx, pic.PIC_OP_PREFILL, dcr.req(), nsel, nsel)),
                          dtype=torch.uint8, device=dev)
        rms, krms = time_calls(lambda: pic.pic_attn_prefill(ctx, dcr, outr, None, ws=wsr, stream=stream),
                               kctx=ctx)
        fpi = dc.kv_pos.cpu().numpy()[0, :kv_fused]
        fpi = np.sort(fpi[fpi >= 0])
        pairs_r = int(np.searchsorted(fpi, pos_r, side="right").sum())
        flops_r = pairs_r * w.num_q_heads * 4 * w.head_dim
        result["sparse_recompute"] = {
            "workload": f"{nsel} selected tokens as queries at their logical positions over the fused "
                        f"{kv_fused}-slot cache, causal by position",
            "ms_per_call": round(rms, 5), "visible_pairs": pairs_r,
            "roofline": roof("mfma", flops_r / (krms / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                             algorithmic_flops=flops_r, avg_ms=round(krms, 5),
                             qk_pairs_per_s=round(pairs_r * w.num_q_heads / (krms / 1e3), 1),
                             kernel="fwd_kernel<128, 2, 8, 0, true, true> (tile skipping)",
                             call=roof("mfma", flops_r / (rms / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", mp_tf,
                                       avg_ms=round(rms, 5), what="the whole pic_attn_prefill call"))}
        del dcr, outr, wsr

    if "anchor" in only:
        # Anchor extraction: per-span top 5% of slots by stored-key norm over the
        # un-fused long-context cache (reads K once: HBM-bound).
        state.copy_(state0)
        dc.max_kv_len = kv0
        a_off = pic.pic_select_offsets(w.span_len, ANCHOR_RATIO)
        na = int(a_off[-1])
        dca = pic.DeviceCache(dc.pool_k, dc.pool_v, dc.block_table, dc.kv_len, dc.kv_pos, kv0,
                              span_req=t(w.span_req), span_start=t(w.span_start), span_len=t(w.span_len),
                              sel_off=t(a_off), n_spans=len(w.span_req))
        asel = torch.empty(max(na, 1), dtype=torch.int32, device=dev)
        anorm = torch.empty(w.kv_pos.shape, dtype=torch.float32, device=dev)
        afn = lambda st=stream: pic.qc_anchor_select(ctx, dca, na, asel, anorm, stream=st)
        ams = time_calls(afn, reps=20, warm=3)
        # the two short kernels of a call finish before the host has issued
        # the next call: the eager loop times the host; graph replays the GPU
        ags = graph_ms(afn, (asel, anorm[:, :kv0]))   # the norms of slots past kv_len are not written
        gms = ags if ags is not None else ams
        kbytes = tokens * w.num_kv_heads * w.head_dim * 2
        result["anchor_extraction"] = {
            "workload": f"{len(w.span_req)} spans x 1024 slots of the long-context cache, top "
                        f"{ANCHOR_RATIO:.0%} per span by key norm ({na} anchors)",
            "ms_per_call": round(ams, 5),
            "graph_ms_per_call": round(ags, 5) if ags is not None else None,
            "roofline": roof("hbm", kbytes / (gms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s", mp_hbm,
                             algorithmic_bytes=kbytes, avg_ms=round(gms, 5),
                             timing="20 calls captured as one HIP graph, GPU time per call (both kernels "
                                    "and the gap between them)" if ags is not None else
                                    "eager back-to-back calls (graph check failed)")}
        del dca, asel, anorm

    if "decode" in only:
        dlines = {}
        pools = [x.strip() for x in args.decode_pools.split(",") if x.strip()]
        for private in [x == "private" for x in pools]:
            # the private control's 4 GiB pool is drawn on the device (seeded);
            # its block tables, positions and queries come from the workload
            wd = W.decode_heavy(private_spans=private, pool_values=not private)
            ctxd = pic.Context(wd.num_q_heads, wd.num_kv_heads, wd.head_dim, wd.rope_theta, wd.max_position)
            if private:
                gen = torch.Generator(device=dev)
                gen.manual_seed(wd.seed)
                pk = torch.empty(wd.pool_k.shape, dtype=torch.bfloat16, device=dev)
                pv = torch.empty(wd.pool_v.shape, dtype=torch.bfloat16, device=dev)
                for buf in (pk, pv):
                    flat = buf.view(-1)
                    for s0 in range(0, flat.numel(), 1 << 28):
                        n_ = min(1 << 28, flat.numel() - s0)
                        flat[s0:s0 + n_] = torch.randn(n_, generator=gen, device=dev, dtype=torch.float32)
                dd = pic.DeviceCache(pk.view(torch.int16), pv.view(torch.int16), t(wd.block_table), t(wd.kv_len),
                                     t(wd.kv_pos), wd.max_kv_len, q=t(wd.q), q_start=t(wd.q_start),
                                     q_pos=t(wd.q_pos), total_q=wd.total_q, max_q_len=wd.max_q_len)
            else:
                dd = pic.to_device(wd, dev)
            outd = torch.empty((wd.batch, wd.num_q_heads, wd.head_dim), dtype=torch.int16, device=dev)
            wsd = torch.empty(max(1, pic.pic_workspace_bytes(ctxd, pic.PIC_OP_DECODE, dd.req(), 0, 0)),
                              dtype=torch.uint8, device=dev)
            call = lambda: pic.pic_attn_decode(ctxd, dd, dd.q, dd.q_pos, outd, None, ws=wsd, stream=stream)
            dms, kdms = time_calls(call, reps=20, warm=3, kctx=ctxd)
            dtok = attended_tokens(wd)
            kvbytes = dtok * wd.num_kv_heads * wd.head_dim * 2 * 2
            line = {"ms_per_call": round(dms, 5), "attended_kv_tokens_per_s": round(dtok / (dms / 1e3), 1),
                    "kernel_ms": round(kdms, 5)}
            dcall = dict(avg_ms=round(dms, 5), what="the whole pic_attn_decode call (kernel + split merge)")
            if private:
                line["workload"] = ("64 requests x 16,385 KV slots, each over 16 spans of its own (a 4 GiB pool, "
                                    "far above the 256 MB Infinity Cache), 64 q / 8 kv heads, d 128")
                line["roofline"] = roof("hbm", kvbytes / (kdms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s", mp_hbm,
                                        algorithmic_bytes=kvbytes, avg_ms=round(kdms, 5),
                                        kernel="decode_kernel<128>",
                                        traffic=measured_traffic(TRAFFIC_RECORDS["decode_private"]),
                                        call=roof("hbm", kvbytes / (dms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                                  mp_hbm, **dcall))
                dlines["decode_heavy_private"] = line
            else:
                line["workload"] = ("64 requests x 16,385 KV slots over the same 16 shared spans at per-request "
                                    "offsets (64 MiB unique K/V), 64 q / 8 kv heads, d 128")
                line["roofline"] = roof("cache-resident", kvbytes / (kdms / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                        mp_hbm, algorithmic_bytes=kvbytes, avg_ms=round(kdms, 5),
                                        kernel="decode_kernel<128>",
                                        traffic=measured_traffic(TRAFFIC_RECORDS["decode_shared"]),
                                        call=roof("cache-resident", kvbytes / (dms / 1e3) / 1e9, PEAK_HBM_GBS,
                                                  "GB/s", mp_hbm, **dcall),
                                        note="warm: the 64 MiB of unique K/V stay in the Infinity Cache, so "
                                             "most algorithmic bytes do not come from HBM; the HBM roofline "
                                             "is the private-pool line.  traffic (FETCH_SIZE + WRITE_SIZE) "
                                             "counts what the L2 fetches from beyond it: the Infinity Cache "
                                             "or HBM")
                # cold: a 1 GiB write evicts L2 and the Infinity Cache before each call
                flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
                cold = []
                for k in range(12):
                    flush.fill_(k & 255)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    call()
                    b.record(stream)
                    torch.cuda.synchronize()
                    if k >= 2:
                        cold.append(a.elapsed_time(b))
                del flush
                cms = float(np.median(cold))
                line["cold"] = {"ms_per_call": round(cms, 5),
                                "attended_kv_tokens_per_s": round(dtok / (cms / 1e3), 1),
                                "algorithmic_gbs": round(kvbytes / (cms / 1e3) / 1e9, 1),
                                "traffic": measured_traffic(TRAFFIC_RECORDS["decode_shared_cold"]),
                                "what": "median of 10 calls, each after a 1 GiB device write that evicts the "
                                        "L2 caches and the Infinity Cache; within a call the 64 requests "
                                        "re-read the same 64 MiB, so all but the first pass over it come "
                                        "from the caches again"}
                if ablation is not None:
                    ctxd_pr = pic.Context(wd.num_q_heads, wd.num_kv_heads, wd.head_dim, wd.rope_theta,
                                          wd.max_position, keys_prerotated=True)
                    d_pre = time_calls(lambda: pic.pic_attn_decode(ctxd_pr, dd, dd.q, dd.q_pos, outd, None,
                                                                   ws=wsd, stream=stream), reps=20, warm=3)
                    ctxd_pr.close()
                    ablation["decode_heavy_ms"] = {"in_kernel": round(dms, 5), "prerotated": round(d_pre, 5),
                                                   "overhead": round(dms / d_pre - 1.0, 4)}
                dlines["decode_heavy_shared"] = line
            del dd, outd, wsd
            if private:
                del pk, pv
            ctxd.close()
            torch.cuda.empty_cache()
        result.update(dlines)

    if "hashing" in only:
        # Span reuse by block hashing (host): 64 requests, each a private prompt
        # and 16 SSEP spans of 1,024 tokens drawn from a pool of 64 spans.
        rng = np.random.default_rng(11)
        bs = pic.PIC_BLOCK_SIZE
        pool_sp = []
        for _ in range(64):
            sp = [1] + rng.integers(10, 50000, 1024).tolist()
            pool_sp.append(sp + [-1] * ((-len(sp)) % bs))
        reqs = []
        for _ in range(64):
            pr = rng.integers(10, 50000, int(rng.integers(16, 200))).tolist()
            tk = pr + [-1] * ((-len(pr)) % bs)
            for k in rng.integers(0, 64, 16):
                tk += pool_sp[int(k)]
            reqs.append(np.asarray(tk, np.int32))
        ntok = sum(len(x) for x in reqs)
        cache = pic.BlockCache(200000)
        c0 = time.perf_counter()
        misses = blocks = 0
        for x in reqs:
            _, _, m = cache.map_request(x, -1, 1, 2)
            misses += int(m.sum())
            blocks += len(m)
        hsec = time.perf_counter() - c0
        cache.close()
        result["block_hashing"] = {
            "workload": f"64 requests, {ntok} tokens: private prompts + 16 SSEP spans of 1,024 tokens each from a "
                        "pool of 64", "host_ms": round(hsec * 1e3, 3), "tokens_per_s": round(ntok / hsec, 1),
            "blocks": blocks, "reused_blocks": blocks - misses, "where": "host CPU (pic_block_map)"}

    if cpu is not None:
        result["cpu_baseline"] = cpu
    ctx.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
