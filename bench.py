#!/usr/bin/env python3
"""Benchmark: effective input GB/s of one DeepSelect top-k call on one MI355X.

A step is one whole top-k call (select kernel over every row slice, then the merge kernel)
over one batch of synthetic input already resident in HBM. Each step reads a different copy
of the input from a pool of >= 512 MiB, so the 256 MB Infinity Cache cannot serve it (cold).
Timing: W warmup steps, then K steps recorded into one HIP graph and replayed between two
events (the headline: no host launch gaps); K select launches alone in one graph (the select
kernel's average duration per launch, the roofline figure; it agrees with the profiler's
kernel time); and the same K steps launched one by one (eager). The same loops over one
buffer are reported as the warm figures. The CPU oracle is
timed on the host cores on a bounded sample of the same workload.

Two more modes serve the committed rocprofv3 counter summary: --counter-pass runs the
select kernel and a calibration copy of known size under the profiler, and
--write-counters turns the profiler's FETCH_SIZE / WRITE_SIZE tables into that summary.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "effective input GB/s per top-k call (and % of HBM peak) at 1 MI355X"


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def upload(x, torch):
    import numpy as np
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def source_digest() -> str:
    """Digest of the library's code: comments and whitespace do not count, so a change to
    a comment keeps counter summaries taken on the same code valid."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_selection_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, digest: str):
    """HBM bytes per select launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"select_kernel_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("traffic:"):
                for kv in line.split()[1:]:
                    key, _, val = kv.partition("=")
                    vals[key] = val
    if vals.get("source") != digest or "bytes_per_launch" not in vals:
        return None
    return float(vals["bytes_per_launch"])


def time_workload(ts, torch, w, k, steps, warmup, pool_mib, seed=1, verify=True):
    import numpy as np
    from workloads import gen

    log(f"[bench] generating {w.name}: {w.rows} x {w.n} {gen.DTYPE_NAMES[w.dtype]}")
    x = w.make()
    xd = upload(x, torch)
    in_bytes = w.input_bytes()
    copies = max(1, math.ceil(pool_mib * 2 ** 20 / in_bytes))
    pool = [xd] + [xd.clone() for _ in range(copies - 1)]
    rows, n = w.rows, w.n
    plan = ts.ds_topk_plan(rows, n, k, w.dtype)
    wsb = ts.ds_topk_workspace_size(rows, n, k, w.dtype)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    vals = torch.empty((rows, k), dtype=xd.dtype, device="cuda")
    idx = None if w.values_only else torch.empty((rows, k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(src):  # one library call: the select launch and the merge launches
        ts.ds_topk_ex(src, k, seed=seed, workspace=ws, out_vals=vals, out_idx=idx, indices=idx is not None)

    log(f"[bench] {w.name}: plan {plan}, pool {copies} copies, warmup {warmup}")
    for i in range(warmup):
        step(pool[i % copies])
    torch.cuda.synchronize()

    def timed(get_src):
        """K steps launched one by one (one library call each) between two events; then K
        select launches with an event pair around each (host launch latency included)."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            step(get_src(i))
        t1.record(stream)
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1)
        mids = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            a, b = mids[i]
            a.record(stream)
            ts.ds_topk_slices(get_src(i), k, seed=seed, workspace=ws, out_vals=vals, out_idx=idx,
                              indices=idx is not None)
            b.record(stream)
            ts.ds_topk_merge(rows, n, k, w.dtype, seed=seed, workspace=ws, out_vals=vals, out_idx=idx)
        torch.cuda.synchronize()
        sel = [a.elapsed_time(b) for a, b in mids]
        return total / steps, sum(sel) / len(sel)

    def select_only(src):
        ts.ds_topk_slices(src, k, seed=seed, workspace=ws, out_vals=vals, out_idx=idx, indices=idx is not None)

    def per_call_times(get_src):
        """Each step's own duration: K steps in one graph with an event recorded between
        consecutive steps (event record nodes); eager launches between events if the graph
        cannot hold such nodes. Returns (list of us, method)."""
        try:
            evs = [torch.cuda.Event(enable_timing=True, external=True) for _ in range(steps + 1)]
            gs = torch.cuda.Stream()
            gs.wait_stream(stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                evs[0].record(gs)
                for i in range(steps):
                    step(get_src(i))
                    evs[i + 1].record(gs)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)]
            return us, "one HIP graph of K steps with an event record node between consecutive steps"
        except Exception as e:  # noqa: BLE001 (the fallback names the reason)
            log(f"[bench] graph events unavailable ({e}); timing eager steps")
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            torch.cuda.synchronize()
            evs[0].record(stream)
            for i in range(steps):
                step(get_src(i))
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            return [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)], "eager steps between events"

    def graph_timed(get_src, fn=step):
        """K steps (or K launches of fn) captured into one graph, replayed once between two
        events; returns ms per step."""
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            fn(get_src(0))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for i in range(steps):
                fn(get_src(i))
        torch.cuda.synchronize()
        g.replay()  # warm the graph once
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms_cold, sel_cold = timed(lambda i: pool[i % copies])
    log(f"[bench] {w.name} cold eager: {ms_cold * 1e3:.2f} us/call, select {sel_cold * 1e3:.2f} us")
    ms_warm, sel_warm = timed(lambda i: pool[0])
    log(f"[bench] {w.name} warm eager: {ms_warm * 1e3:.2f} us/call, select {sel_warm * 1e3:.2f} us")
    ms_graph = graph_timed(lambda i: pool[i % copies])
    log(f"[bench] {w.name} cold graph: {ms_graph * 1e3:.2f} us/call")
    ms_graph_warm = graph_timed(lambda i: pool[0])
    log(f"[bench] {w.name} warm graph: {ms_graph_warm * 1e3:.2f} us/call")
    # the select kernel alone, back to back in a graph: its average duration per launch
    ms_select = graph_timed(lambda i: pool[i % copies], select_only)
    log(f"[bench] {w.name} select kernel (graph, cold): {ms_select * 1e3:.2f} us/launch")
    # the read ceiling: the probe streams the same bytes with the scan's loads, same pool
    sink = torch.empty(int(ts.lib().ds_probe_sink_words(in_bytes)), dtype=torch.int32, device="cuda")
    ms_probe = graph_timed(lambda i: pool[i % copies], lambda src: ts.ds_probe_read(src, sink=sink))
    log(f"[bench] {w.name} probe read (graph, cold): {ms_probe * 1e3:.2f} us/read")
    per_call = per_call_times(lambda i: pool[i % copies])

    parity = None
    if verify:
        from oracle import topk as otk
        step(pool[-1])
        torch.cuda.synchronize()
        want_v, want_i = otk.topk(x, k, indices=idx is not None)
        got_v = vals.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == np.uint16 else vals.cpu().numpy()
        ok = np.array_equal(got_v.view(np.uint8), want_v.view(np.uint8))
        if idx is not None:
            ok = ok and np.array_equal(idx.cpu().numpy(), want_i)
        parity = "bit-exact" if ok else "MISMATCH"
        log(f"[bench] {w.name} parity vs oracle: {parity}")
    del pool
    return dict(x=x, plan=plan, copies=copies, ms_cold=ms_graph, ms_eager=ms_cold, sel_cold=ms_select, sel_eager=sel_cold,
                ms_warm=ms_graph_warm, ms_warm_eager=ms_warm, sel_warm=sel_warm, in_bytes=in_bytes, parity=parity,
                ws_bytes=wsb, ms_probe=ms_probe, per_call=per_call)


def percentiles(us_method):
    import numpy as np
    us, method = us_method
    a = np.asarray(us)
    return {"p10": round(float(np.percentile(a, 10)), 3), "p50": round(float(np.percentile(a, 50)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "unit": "us", "calls": int(a.size), "method": method}


CALIB_BYTES = 256 * 2 ** 20  # calibration copy: reads and writes exactly this many bytes

# the other workloads timed on every run: (workload, k, timed steps at most)
SECONDARY = [("c3_sampler", 512, 100), ("c4_long", 512, 100), ("c4_long", 4096, 50), ("c5_giant", 32, 50)]


def counter_pass(ts, torch, w, k, launches, pool_mib):
    """Workload for a rocprofv3 --pmc run: `launches` cold select launches (plus merges), then
    three calibration copies of CALIB_BYTES with the plain copy kernel."""
    x = w.make()
    xd = upload(x, torch)
    copies = max(1, math.ceil(pool_mib * 2 ** 20 / w.input_bytes()))
    pool = [xd] + [xd.clone() for _ in range(copies - 1)]
    rows, n = w.rows, w.n
    wsb = ts.ds_topk_workspace_size(rows, n, k, w.dtype)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    vals = torch.empty((rows, k), dtype=xd.dtype, device="cuda")
    idx = None if w.values_only else torch.empty((rows, k), dtype=torch.int32, device="cuda")
    for i in range(launches):
        ts.ds_topk_slices(pool[i % copies], k, seed=1, workspace=ws, out_vals=vals, out_idx=idx,
                          indices=idx is not None)
        ts.ds_topk_merge(rows, n, k, w.dtype, seed=1, workspace=ws, out_vals=vals, out_idx=idx)
    torch.cuda.synchronize()
    del pool
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        ts.ds_probe_copy(dst, src)
    torch.cuda.synchronize()
    log(f"[bench] counter pass done: {launches} select launches of {w.name}, 3 copies of {CALIB_BYTES} B")


def read_counter_csv(folder, counter):
    """Mean per-dispatch value of `counter` for the select kernel and the calibration copy."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                kind = "select" if "select_kernel" in name else ("copy" if "probe_copy_kernel" in name else None)
                if kind is None:
                    continue
                key = (kind, row.get("Dispatch_Id"))
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for kind in ("select", "copy"):
        vals = [v for (kd, _), v in per.items() if kd == kind]
        out[kind] = (sum(vals) / len(vals), len(vals)) if vals else (None, 0)
    return out


def write_counters(workload, fetch_dir, write_dir, command):
    """Summary of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), scaled by the copy's."""
    from workloads import gen
    w = gen.WORKLOADS[workload]
    f = read_counter_csv(fetch_dir, "FETCH_SIZE")
    wr = read_counter_csv(write_dir, "WRITE_SIZE")
    (fs, nfs), (fc, nfc) = f["select"], f["copy"]
    (ws_, nws), (wc, nwc) = wr["select"], wr["copy"]
    if None in (fs, fc, ws_, wc):
        raise SystemExit("counter tables lack the select or the copy kernel")
    kf = CALIB_BYTES / (fc * 1024.0)   # bytes per reported KiB, from the copy's known reads
    kw = CALIB_BYTES / (wc * 1024.0)
    rd = fs * 1024.0 * kf
    wt = ws_ * 1024.0 * kw
    total = rd + wt
    algo = w.input_bytes()
    digest = source_digest()
    lines = [
        f"# select_kernel HBM traffic, {workload}",
        "",
        f"Workload: {w.description}. Algorithmic bytes per launch (the input, read once): {algo}.",
        "",
        "Commands (rocprofv3 3.x on one MI355X; counters in runs of their own):",
        "",
        "```",
        command.replace("COUNTER", "FETCH_SIZE"),
        command.replace("COUNTER", "WRITE_SIZE"),
        "```",
        "",
        "| counter | select_kernel (KiB/dispatch, mean) | dispatches | copy of 256 MiB (KiB/dispatch) | bytes per KiB |",
        "|---|---|---|---|---|",
        f"| FETCH_SIZE | {fs:.1f} | {nfs} | {fc:.1f} | {kf:.4f} |",
        f"| WRITE_SIZE | {ws_:.1f} | {nws} | {wc:.1f} | {kw:.4f} |",
        "",
        f"Read bytes per launch (scaled): {rd:.0f} = {rd / algo:.4f} x the input.",
        f"Written bytes per launch (scaled): {wt:.0f}.",
        "",
        f"traffic: source={digest} bytes_per_launch={total:.0f} read_bytes={rd:.0f} write_bytes={wt:.0f}",
        "",
    ]
    path = os.path.join(ROOT, "profiles", f"select_kernel_{workload}_counters.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    log(f"[bench] wrote {path}: {total:.0f} B per launch ({total / algo:.3f} x algorithmic)")


SQ_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_ANY",
               "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"]


def write_sq(workload, k, folder, command):
    """Summary of one rocprofv3 --pmc run of the SQ counters over the select kernel."""
    from workloads import gen
    w = gen.WORKLOADS[workload]
    vals = {c: read_counter_csv(folder, c)["select"] for c in SQ_COUNTERS}
    missing = [c for c, (v, _) in vals.items() if v is None]
    if missing:
        raise SystemExit(f"counter tables lack {missing} for the select kernel")
    m = {c: v for c, (v, _) in vals.items()}
    elems = w.rows * w.n
    lines = [
        f"# select_kernel SQ counters, {workload} (k = {k})",
        "",
        f"Workload: {w.description}. Elements per launch: {elems}.",
        "",
        "Command (rocprofv3 on one MI355X, one --pmc run; R is the repository path):",
        "",
        "```",
        command,
        "```",
        "",
        "| counter | mean per select dispatch | dispatches |",
        "|---|---|---|",
    ]
    for c in SQ_COUNTERS:
        lines.append(f"| {c} | {m[c]:.0f} | {vals[c][1]} |")
    lines += [
        "",
        "Derived (per dispatch):",
        "",
        f"- VALU wave-instructions per 64 elements (each lane's VALU instructions per element it holds): "
        f"{m['SQ_INSTS_VALU'] / (elems / 64.0):.2f}",
        f"- SALU instructions per 64 elements: {m['SQ_INSTS_SALU'] / (elems / 64.0):.2f}; LDS instructions per 64 "
        f"elements: {m['SQ_INSTS_LDS'] / (elems / 64.0):.2f}",
        f"- LDS bank-conflict cycles per LDS instruction: {m['SQ_LDS_BANK_CONFLICT'] / max(m['SQ_INSTS_LDS'], 1):.3f}",
        f"- waves resident on average (SQ_WAVE_CYCLES / SQ_BUSY_CYCLES): "
        f"{m['SQ_WAVE_CYCLES'] / max(m['SQ_BUSY_CYCLES'], 1):.2f}",
        f"- share of wave cycles spent waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES): "
        f"{m['SQ_WAIT_ANY'] / max(m['SQ_WAVE_CYCLES'], 1):.3f}",
        f"- waves per dispatch (SQ_WAVES): {m['SQ_WAVES']:.0f}",
        "",
        f"source={source_digest()}",
        "",
    ]
    path = os.path.join(ROOT, "profiles", f"select_kernel_{workload}_k{k}_sq.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    log(f"[bench] wrote {path}")


def write_trace(workload, k, trace_dir, command):
    """Summary of a rocprofv3 --kernel-trace --stats run of bench.py into profiles/."""
    import csv
    import glob
    from workloads import gen
    w = gen.WORKLOADS[workload]
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    with open(paths[0]) as f:
        rows = list(csv.DictReader(f))
    lines = [
        f"# Kernel trace, {workload} (k = {k})",
        "",
        f"Workload: {w.description} (k = {k} here); the bench's default plan, its timed steps plus warmup "
        f"(graph, eager and warm passes, the select-only graph, the probe reads, the per-call steps and one "
        f"parity call).",
        "",
        "Command (on one MI355X, from the repository root; R is the repository path):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows[:8]:
        name = r["Name"].replace("void ds::(anonymous namespace)::", "")
        if len(name) > 70:
            name = name[:67] + "..."
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")
    lines.append("")
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}_k{k}_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    log(f"[bench] wrote {path}")


def cpu_identity():
    """(model name, sockets) of the host from /proc/cpuinfo."""
    model, sockets = "unknown", set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "model name" and model == "unknown":
                    model = val.strip()
                elif key == "physical id":
                    sockets.add(val.strip())
    except OSError:
        pass
    return model, max(1, len(sockets))


def cpu_baseline(w, k, x, seconds):
    from oracle import topk as otk
    threads = otk.hw_threads()
    model, sockets = cpu_identity()
    reps, t0 = 0, time.perf_counter()
    while True:
        otk.topk(x, k, indices=not w.values_only, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = w.input_bytes() * reps / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": model,
            "sockets": sockets, "host_cpus_visible": os.cpu_count(),
            "sample": f"{reps} full passes of the {w.name} batch ({w.rows} rows x {w.n}) in {el:.1f} s: "
                      f"C++ full sort per row, rows spread over {threads} threads"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2_indexer")
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--pool-mib", type=float, default=512.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run select launches and a calibration copy for a rocprofv3 --pmc run, then exit")
    ap.add_argument("--write-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COMMAND"),
                    help="summarise two rocprofv3 --pmc output folders into profiles/ (no GPU needed)")
    ap.add_argument("--write-trace", nargs=2, metavar=("TRACE_DIR", "COMMAND"),
                    help="summarise a rocprofv3 --kernel-trace --stats output folder into profiles/ (no GPU needed)")
    ap.add_argument("--write-sq", nargs=2, metavar=("PMC_DIR", "COMMAND"),
                    help="summarise a rocprofv3 --pmc run of the SQ counters into profiles/ (no GPU needed)")
    args = ap.parse_args()

    if args.write_counters:
        write_counters(args.workload, *args.write_counters)
        return 0
    if args.write_trace:
        from workloads import gen as _gen
        write_trace(args.workload, args.k or _gen.WORKLOADS[args.workload].ks[0], *args.write_trace)
        return 0
    if args.write_sq:
        from workloads import gen as _gen
        write_sq(args.workload, args.k or _gen.WORKLOADS[args.workload].ks[0], *args.write_sq)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (rows would shard "
              "across GPUs without communication). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import top_selection_amd as ts
    from workloads import gen

    torch.cuda.set_device(0)
    w = gen.WORKLOADS[args.workload]
    k = args.k or w.ks[0]
    if args.counter_pass:
        counter_pass(ts, torch, w, k, args.steps, args.pool_mib)
        return 0
    r = time_workload(ts, torch, w, k, args.steps, args.warmup, args.pool_mib)
    value = r["in_bytes"] / (r["ms_cold"] * 1e-3) / 1e9
    sel_gbs = r["in_bytes"] / (r["sel_cold"] * 1e-3) / 1e9
    digest = source_digest()
    traffic = read_traffic(w.name, digest)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_cold"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gen.DTYPE_NAMES[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "n": w.n, "k": k, "elem": gen.DTYPE_NAMES[w.dtype],
                   "values_only": w.values_only, "block": r["plan"]["block"], "slack": r["plan"]["slack"],
                   "slices": r["plan"]["slices"], "waves": r["plan"]["waves"], "input_pool_copies": r["copies"],
                   "cold_inputs": True, "description": w.description},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "timing": "K steps captured in one HIP graph, replayed between two events",
        "eager": {"value": round(r["in_bytes"] / (r["ms_eager"] * 1e-3) / 1e9, 2),
                  "ms_per_step": round(r["ms_eager"], 6), "select_us": round(r["sel_eager"] * 1e3, 3),
                  "note": "the same K steps launched one by one (one ds_topk_ex call each); select_us spans "
                          "event to event around each select launch (host launch latency included)"},
        "warm": {"value": round(r["in_bytes"] / (r["ms_warm"] * 1e-3) / 1e9, 2), "ms_per_step": round(r["ms_warm"], 6),
                 "note": "same input buffer every step (may be served by the Infinity Cache)"},
        "pages_style_gbs": round((r["in_bytes"] + w.rows * k * (w.elem_bytes + (0 if w.values_only else 4)))
                                 / (r["ms_cold"] * 1e-3) / 1e9, 2),
        "parity": r["parity"],
        "probe": {"us_per_read": round(r["ms_probe"] * 1e3, 3),
                  "gbs": round(r["in_bytes"] / (r["ms_probe"] * 1e-3) / 1e9, 2),
                  "note": "ds_probe_read of the same bytes from the same pool (the scan's 16-byte loads, nothing "
                          "else), K reads in one HIP graph: the read ceiling this input size reaches"},
        "pct_of_probe": round(100.0 * r["ms_probe"] / r["ms_cold"], 2),
        "select_pct_of_probe": round(100.0 * r["ms_probe"] / r["sel_cold"], 2),
        "per_call": percentiles(r["per_call"]),
        "roofline": {"bound": "hbm", "kernel": "select_kernel", "achieved": round(sel_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(sel_gbs / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(r["sel_cold"] * 1e3, 3),
                     "timing": "K select launches back to back in one HIP graph, events on its stream",
                     "algorithmic_bytes_per_launch": r["in_bytes"],
                     "traffic": traffic, "source": digest},
    }
    if not args.no_secondary:
        sec = {}
        for name, sk, nsteps in SECONDARY:
            if name == w.name and sk == k:
                continue
            sw = gen.WORKLOADS[name]
            s = time_workload(ts, torch, sw, sk, min(nsteps, args.steps), args.warmup, args.pool_mib)
            sv = s["in_bytes"] / (s["ms_cold"] * 1e-3) / 1e9
            ssel = s["in_bytes"] / (s["sel_cold"] * 1e-3) / 1e9
            sec[f"{name}_k{sk}"] = {
                "value": round(sv, 2), "unit": "GB/s", "pct_of_hbm_peak": round(100 * sv / HBM_PEAK_GBS, 2),
                "k": sk, "ms_per_step": round(s["ms_cold"], 6), "select_us": round(s["sel_cold"] * 1e3, 3),
                "select_frac_of_hbm_peak": round(ssel / HBM_PEAK_GBS, 4),
                "probe_us": round(s["ms_probe"] * 1e3, 3), "pct_of_probe": round(100.0 * s["ms_probe"] / s["ms_cold"], 2),
                "per_call": percentiles(s["per_call"]),
                "warm_value": round(s["in_bytes"] / (s["ms_warm"] * 1e-3) / 1e9, 2),
                "plan": s["plan"], "parity": s["parity"], "input_pool_copies": s["copies"]}
        out["secondary"] = sec
    if not args.no_cpu:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(w, k, r["x"], args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0 if r["parity"] != "MISMATCH" else 1


if __name__ == "__main__":
    sys.exit(main())
