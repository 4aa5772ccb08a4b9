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
times it eagerly.  Per-op times come from an eager run with events between
the calls.

metric: attended KV tokens per second, where each attention-type call over a
request attends its kv_len minus masked slots (33,024 here) and the step makes
four such calls.  The roofline object is for the dominant kernel (step 1,
MFMA-bound: visible (query, key) pairs x Hq x 4d flops against the bf16 dense
peak), timed with HIP events on the launch stream.  A decode-heavy line (64
requests x 16,385 KV slots from 16 shared spans, 64 q / 8 kv heads) reports
HBM-roofline throughput of pic_attn_decode.  cpu_baseline is the double-
precision CPU oracle, single-threaded, timed on a sample of step 1's rows and
scaled by visible (row, key) pairs to the whole step.

    python bench.py [--steps K] [--warmup W]

HBM traffic of the dominant kernel (roofline.traffic) comes from two
rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) of this script, each scaled by
what the same counter reads for a plain device copy of known size
(--calibrate-copy); --traffic-from turns the four runs into
profiles/prefill_traffic.json, which records a hash of the kernel sources:
the field is null once those sources differ from the measured ones.
"""
import argparse
import csv
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
TRAFFIC_KERNEL = "fwd_kernel<128, 2, 8, 0, false, true>"
# the files whose change invalidates a traffic measurement of that kernel
TRAFFIC_SOURCES = ["position_independent_attention_amd/csrc/attn_fwd.hip",
                   "position_independent_attention_amd/csrc/pic_internal.h",
                   "position_independent_attention_amd/csrc/api.cpp",
                   "position_independent_attention_amd/build.py"]
COPY_BYTES = 512 << 20
ANCHOR_RATIO = 0.05   # anchor fraction per span (the pages say only "a small fraction")
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


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


def sources_hash():
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per launch from profiles/prefill_traffic.json, or None if absent or
    taken from other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
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


def _pmc(d, counter, name_part, every=1):
    """Mean counter value over the dispatches of kernels named like name_part
    (every: take every n-th of them in dispatch order, from the first).  With
    every > 1 the dispatches must all have one grid size and come in whole
    groups of `every`, else the run held other launches of the kernel."""
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), r.get("Grid_Size", "")))
    rows = sorted(rows)
    if every > 1 and (len({g for _, _, g in rows}) > 1 or len(rows) % every):
        raise SystemExit(f"{d}: {len(rows)} dispatches of '{name_part}' with grids {sorted({g for _, _, g in rows})}; "
                         "profile the step alone (--no-decode --no-recompute --no-anchor --no-ablation --no-hashing)")
    rows = rows[::every]
    if not rows:
        raise SystemExit(f"no {counter} rows for '{name_part}' under {d}")
    return float(np.mean([v for _, v, _ in rows])), len(rows)


def traffic_from(copy_fetch, copy_write, fetch, write):
    """Scale the kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the
    reading of the same counters for the calibration copy."""
    cf, _ = _pmc(copy_fetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = _pmc(copy_write, "WRITE_SIZE", "copyBuffer")
    # each step launches the kernel twice (step 1, then the pass over the fused
    # cache): the step-1 dispatches are every other one from the first
    kf, nf = _pmc(fetch, "FETCH_SIZE", TRAFFIC_KERNEL, every=2)
    kw, nw = _pmc(write, "WRITE_SIZE", TRAFFIC_KERNEL, every=2)
    ff, fw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    out = {"kernel": TRAFFIC_KERNEL, "workload": "long_context_qc_fusion step 1 (pic_attn_prefill)",
           "sources_sha256": sources_hash(),
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES,
           "fetch_scale": ff, "write_scale": fw,
           "kernel_fetch_kib": kf, "kernel_write_kib": kw, "dispatches": [nf, nw],
           "fetch_bytes_per_launch": kf * 1024.0 * ff, "write_bytes_per_launch": kw * 1024.0 * fw}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


def attended_tokens(w):
    return int(sum(int((w.kv_pos[r, :w.kv_len[r]] >= 0).sum()) for r in range(w.batch)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU's clock rises over the first tens of steps: 3 warm-up steps
    # time a 20-step loop about 14% slower than the clock settles at.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-sample-tokens", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-recompute", action="store_true")
    ap.add_argument("--no-anchor", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-hashing", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time the step eagerly, without a HIP graph")
    ap.add_argument("--decode-private", action="store_true",
                    help="decode line on the unshared control (4 GiB pool)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the device copy the traffic counters are scaled by")
    ap.add_argument("--traffic-from", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                    help="rocprofv3 --pmc output dirs -> profiles/prefill_traffic.json")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (requests and kv heads "
              "shard without exchange; a split KV range needs one exchange of partial O + LSE); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from position_independent_attention_amd import pic, workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    w = W.long_context()
    log(f"workload built in {time.time() - t0:.1f}s: kv_len {w.max_kv_len}, q {w.total_q}")
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

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

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
    stream = torch.cuda.current_stream()
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

    # The same step captured once as a HIP graph and replayed K times: the step
    # makes 14 launches, and a replay drops their host-side launch work and most
    # of the gaps between them.  Every replay is first checked bit for bit
    # against an eager step (with eager work and synchronisations in between).
    ms_graph, graph_note = None, "off"
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
    ms_per_step = ms_graph if ms_graph is not None else ms_eager

    tokens = attended_tokens(w)
    step_tokens = 4 * tokens
    value = step_tokens / (ms_per_step / 1e3)
    pairs = visible_pairs(w)
    flops = pairs * w.num_q_heads * 4 * w.head_dim
    achieved = flops / (op_ms["prefill"] / 1e3) / 1e12
    roofline = {"kernel": "pic_attn_prefill, step 1: fwd_kernel<128, 2, 8, 0, false, true> (split partials) + merge_kernel; "
                          "the duration is the whole call's",
                "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                "algorithmic_flops": flops, "avg_ms": round(op_ms["prefill"], 5)}

    result = {"metric": METRIC, "value": round(value, 1), "unit": "attended KV tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
              "ms_per_step_eager": round(ms_eager, 5), "launch": graph_note,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic",
              "config": {"workload": "long_context_qc_fusion", "batch": 1, "kv_slots": int(w.max_kv_len),
                         "spans": "32 x 1024 reused at shuffled offsets", "query_tokens": int(w.total_q),
                         "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                         "rope_theta": w.rope_theta, "select_ratio": w.ratio, "fused_rows": nsel,
                         "step": "prefill+lse, qc_score_select, kv_fuse_scatter, prefill(fused), decode(1)"},
              "roofline": roofline, "ops_ms": {k: round(v, 5) for k, v in op_ms.items()}}

    def time_calls(fn, reps=10, warm=2):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ablation = None
    if not args.no_ablation:
        # Rotation-overhead ablation (MiniPIC reports 5.7% end to end): the same
        # prefill call with keys_prerotated = 1, i.e. the keys used as stored.  It
        # runs on the same pool bytes: the kernels' work does not depend on the
        # key values.
        state.copy_(state0)
        dc.max_kv_len = kv0
        ctx_pr = pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position,
                             keys_prerotated=True)
        t_rot = time_calls(lambda: pic.pic_attn_prefill(ctx, dc, out1, lse1, ws=ws, stream=stream))
        t_pre = time_calls(lambda: pic.pic_attn_prefill(ctx_pr, dc, out1, lse1, ws=ws, stream=stream))
        ctx_pr.close()
        ablation = {"what": "same kernels with keys stored rotated (keys_prerotated = 1) vs rotated in-kernel "
                            "at each key's logical position; timed on the same bytes",
                    "prefill_step1_ms": {"in_kernel": round(t_rot, 5), "prerotated": round(t_pre, 5),
                                         "overhead": round(t_rot / t_pre - 1.0, 4)}}
        result["rotation_ablation"] = ablation

    if not args.no_recompute:
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
        for _ in range(2):
            pic.pic_attn_prefill(ctx, dcr, outr, None, ws=wsr, stream=stream)
        torch.cuda.synchronize()
        reps = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pic.pic_attn_prefill(ctx, dcr, outr, None, ws=wsr, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / reps
        fpi = dc.kv_pos.cpu().numpy()[0, :kv_fused]
        fpi = np.sort(fpi[fpi >= 0])
        pairs_r = int(np.searchsorted(fpi, pos_r, side="right").sum())
        flops_r = pairs_r * w.num_q_heads * 4 * w.head_dim
        result["sparse_recompute"] = {
            "workload": f"{nsel} selected tokens as queries at their logical positions over the fused "
                        f"{kv_fused}-slot cache, causal by position",
            "ms_per_call": round(rms, 5), "visible_pairs": pairs_r,
            "roofline": {"bound": "mfma", "achieved": round(flops_r / (rms / 1e3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops_r / (rms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flops": flops_r}}
        del dcr, outr, wsr

    if not args.no_anchor:
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
        for _ in range(3):
            pic.qc_anchor_select(ctx, dca, na, asel, anorm, stream=stream)
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pic.qc_anchor_select(ctx, dca, na, asel, anorm, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ams = e0.elapsed_time(e1) / reps
        kbytes = tokens * w.num_kv_heads * w.head_dim * 2
        result["anchor_extraction"] = {
            "workload": f"{len(w.span_req)} spans x 1024 slots of the long-context cache, top "
                        f"{ANCHOR_RATIO:.0%} per span by key norm ({na} anchors)",
            "ms_per_call": round(ams, 5),
            "roofline": {"bound": "hbm", "achieved": round(kbytes / (ams / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(kbytes / (ams / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": kbytes}}
        del dca, asel, anorm

    if not args.no_decode:
        wd = W.decode_heavy(private_spans=args.decode_private)
        ctxd = pic.Context(wd.num_q_heads, wd.num_kv_heads, wd.head_dim, wd.rope_theta, wd.max_position)
        dd = pic.to_device(wd, dev)
        outd = torch.empty((wd.batch, wd.num_q_heads, wd.head_dim), dtype=torch.int16, device=dev)
        wsd = torch.empty(max(1, pic.pic_workspace_bytes(ctxd, pic.PIC_OP_DECODE, dd.req(), 0, 0)),
                          dtype=torch.uint8, device=dev)
        for _ in range(3):
            pic.pic_attn_decode(ctxd, dd, dd.q, dd.q_pos, outd, None, ws=wsd, stream=stream)
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pic.pic_attn_decode(ctxd, dd, dd.q, dd.q_pos, outd, None, ws=wsd, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / reps
        if ablation is not None:
            ctxd_pr = pic.Context(wd.num_q_heads, wd.num_kv_heads, wd.head_dim, wd.rope_theta, wd.max_position,
                                  keys_prerotated=True)
            d_pre = time_calls(lambda: pic.pic_attn_decode(ctxd_pr, dd, dd.q, dd.q_pos, outd, None, ws=wsd,
                                                           stream=stream), reps=20, warm=3)
            ctxd_pr.close()
            ablation["decode_heavy_ms"] = {"in_kernel": round(dms, 5), "prerotated": round(d_pre, 5),
                                           "overhead": round(dms / d_pre - 1.0, 4)}
        dtok = attended_tokens(wd)
        kvbytes = dtok * wd.num_kv_heads * wd.head_dim * 2 * 2
        result["decode_heavy"] = {
            "workload": "decode_heavy" + ("_private" if args.decode_private else "") +
                        ": 64 requests x 16,385 KV slots, 64 q / 8 kv heads, d 128",
            "ms_per_call": round(dms, 5), "attended_kv_tokens_per_s": round(dtok / (dms / 1e3), 1),
            "roofline": {"bound": "hbm", "achieved": round(kvbytes / (dms / 1e3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(kvbytes / (dms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": kvbytes}}
        del dd, outd, wsd
        ctxd.close()

    if not args.no_hashing:
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
            t = pr + [-1] * ((-len(pr)) % bs)
            for k in rng.integers(0, 64, 16):
                t += pool_sp[int(k)]
            reqs.append(np.asarray(t, np.int32))
        ntok = sum(len(t) for t in reqs)
        cache = pic.BlockCache(200000)
        c0 = time.perf_counter()
        misses = blocks = 0
        for t in reqs:
            _, _, m = cache.map_request(t, -1, 1, 2)
            misses += int(m.sum())
            blocks += len(m)
        hsec = time.perf_counter() - c0
        cache.close()
        result["block_hashing"] = {
            "workload": f"64 requests, {ntok} tokens: private prompts + 16 SSEP spans of 1,024 tokens each from a "
                        "pool of 64", "host_ms": round(hsec * 1e3, 3), "tokens_per_s": round(ntok / hsec, 1),
            "blocks": blocks, "reused_blocks": blocks - misses, "where": "host CPU (pic_block_map)"}

    if not args.no_cpu_baseline:
        import oracle
        nt = min(args.cpu_sample_tokens, w.total_q)
        ts = np.repeat(np.arange(nt), w.num_q_heads)
        hs = np.tile(np.arange(w.num_q_heads), nt)
        c0 = time.perf_counter()
        oracle.attention(w, (ts, hs))
        csec = time.perf_counter() - c0
        pi = np.sort(w.kv_pos[0, :w.kv_len[0]][w.kv_pos[0, :w.kv_len[0]] >= 0])
        sample_pairs = int(np.searchsorted(pi, w.q_pos[:nt], side="right").sum()) * w.num_q_heads
        step_pairs = 3 * pairs * w.num_q_heads + tokens * w.num_q_heads   # 3 prefill-shaped passes + decode
        cpu_step_s = csec * step_pairs / sample_pairs
        result["cpu_baseline"] = {
            "value": round(step_tokens / cpu_step_s, 2), "unit": "attended KV tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle.attention on {nt} query tokens x {w.num_q_heads} heads of step 1 at the full "
                      f"33,024-slot context ({csec:.1f} s), scaled by visible (row, key) pairs to the whole step"}
    ctx.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
