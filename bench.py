#!/usr/bin/env python3
"""Bandwidth bench of the temperature softmax over the vocabulary on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ts_softmax call over one batch: B=64 rows of V=262144 float32
logits (N(0,1)*4, temperatures U[0.5, 1.5), one quarter of the rows each
unmasked / first 16384 columns -inf / a random 20000-column -inf block / all
but 3 ids -inf). Inputs are resident in HBM before timing. Calls rotate over
enough buffer sets (>= 1 GiB of logits + probs, 512 MiB of logits alone) that
each call finds its logits outside the 256 MiB Infinity Cache: the headline
is this cold rate.

Prints one JSON line. `value` is the algorithmic HBM rate 2*B*V*4 bytes per
call over the timed region (GB/s); `roofline` compares the per-launch rate of
the dominant kernel with MI355X's 8 TB/s; `cpu_baseline` times the float64
oracle on the host over the same workload.

Extra mode: `python bench.py --summarize-counters FETCH_DIR WRITE_DIR` turns
two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench into the
per-dispatch counter summary under profiles/ that the JSON line's
`roofline.traffic` is read from.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "µs/call and HBM GB/s (% of peak) for B×V fp32 temperature softmax"
DEFAULT_WORKLOAD = "B64_V262144_masked_quarters"
COLD_FOOTPRINT = 1 << 30   # bytes of logits + probs the timed calls rotate over: 4x the 256 MiB Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "temperature_softmax_vocabulary_amd", "csrc")


# The sources each profiled kernel is built and launched from: a summary stays
# valid until one of them changes.
KERNEL_SOURCES = {
    "ts_fused": ["softmax_kernels.hip", "ts_device.h", "ts_exchange.h", "ts_launch.h", "tsoftmax_api.cpp"],
    "ts_split": ["softmax_kernels.hip", "ts_device.h", "ts_launch.h", "tsoftmax_api.cpp"],
    "ts_rowwise": ["softmax_kernels.hip", "ts_device.h", "ts_launch.h", "tsoftmax_api.cpp"],
    "ts_draw": ["draw_kernels.hip", "ts_sample_device.h", "ts_device.h", "ts_launch.h", "tsoftmax_api.cpp"],
}


def kernel_source_hash(kernel_tag: str = "") -> str:
    """sha256 prefix over the sources of the kernel family `kernel_tag` starts
    with (every source under csrc/ when it names none of them)."""
    files = None
    for family, names in KERNEL_SOURCES.items():
        if kernel_tag.startswith(family):
            files = [os.path.join(CSRC, n) for n in names]
    if files is None:
        files = glob.glob(os.path.join(CSRC, "*"))
    h = hashlib.sha256()
    for p in sorted(files):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counters_file(kernel_tag: str, workload: str) -> str:
    return os.path.join(PROFILES, f"{kernel_tag}_{workload}_hbm_counters.txt")


def read_traffic(kernel_tag: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken from different kernel sources."""
    path = counters_file(kernel_tag, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(kernel_tag):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------
# counters summary (host-side parsing of rocprofv3 CSV output)
# ----------------------------------------------------------------------------

def _counter_rows(d: str):
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter: str, name_part: str):
    by_dispatch = {}
    for r in rows:
        if r.get("Counter_Name") != counter or name_part not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        by_dispatch[key] = by_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    vals = list(by_dispatch.values())
    return (statistics.mean(vals), len(vals)) if vals else (None, 0)


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, kernel_name: str, kernel_tag: str,
                       command: str, alg_bytes=None) -> str:
    """Per-dispatch HBM bytes of one kernel from two rocprofv3 --pmc runs, scaled
    by the copy kernel's counters; alg_bytes: the kernel's algorithmic bytes per
    launch (default: the softmax's 2 B V 4)."""
    from temperature_softmax_vocabulary_amd import workloads
    c = workloads.CONFIGS[workload]
    n_bytes = c["B"] * c["V"] * 4
    alg = 2 * n_bytes if alg_bytes is None else int(alg_bytes)
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    f_k, nf = _per_dispatch(fr, "FETCH_SIZE", kernel_name)
    w_k, nw = _per_dispatch(wr, "WRITE_SIZE", kernel_name)
    f_c, ncf = _per_dispatch(fr, "FETCH_SIZE", "ts_copy_vec")
    w_c, ncw = _per_dispatch(wr, "WRITE_SIZE", "ts_copy_vec")
    if None in (f_k, w_k, f_c, w_c):
        raise SystemExit(f"missing counters: kernel fetch={f_k} write={w_k} copy fetch={f_c} write={w_c}")
    # The copy reads and writes exactly n_bytes each: KiB-per-dispatch -> bytes factor.
    ff = n_bytes / (f_c * 1024.0)
    wf = n_bytes / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * ff
    write_b = w_k * 1024.0 * wf
    out = counters_file(kernel_tag, workload)
    os.makedirs(PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write(f"# HBM byte counters per dispatch for {kernel_name} on {workload}\n")
        f.write(f"# rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, on: {command}\n")
        f.write("# raw values in KiB per dispatch; scaled by a plain copy of the same bytes\n")
        f.write(f"kernel_source_sha256={kernel_source_hash(kernel_tag)}\n")
        f.write(f"kernel={kernel_name}\n")
        f.write(f"dispatches_fetch={nf}\ndispatches_write={nw}\n")
        f.write(f"fetch_kib={f_k:.1f}\nwrite_kib={w_k:.1f}\n")
        f.write(f"copy_kernel=ts_copy_vec\ncopy_dispatches={ncf},{ncw}\n")
        f.write(f"copy_bytes_each_way={n_bytes}\ncopy_fetch_kib={f_c:.1f}\ncopy_write_kib={w_c:.1f}\n")
        f.write(f"fetch_factor={ff:.4f}\nwrite_factor={wf:.4f}\n")
        f.write(f"fetch_bytes_per_launch={fetch_b:.0f}\nwrite_bytes_per_launch={write_b:.0f}\n")
        f.write(f"traffic_bytes_per_launch={fetch_b + write_b:.0f}\n")
        f.write(f"algorithmic_bytes_per_launch={alg}\n")
        f.write(f"traffic_over_algorithmic={(fetch_b + write_b) / alg:.4f}\n")
    return out


def summarize_trace(trace_dir: str, workload: str, kernel_name: str, kernel_tag: str, command: str) -> str:
    """Per-kernel duration table from a rocprofv3 --kernel-trace --stats run."""
    rows = []
    for p in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = os.path.join(PROFILES, f"{kernel_tag}_{workload}_kernel_trace.txt")
    os.makedirs(PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel trace summary for {workload}; dominant kernel {kernel_name}\n")
        f.write(f"# command: {command}\n")
        f.write(f"# kernel_source_sha256={kernel_source_hash(kernel_tag)}\n")
        f.write(f"{'kernel':<72} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}\n")
        for r in rows:
            name = r["Name"].replace("(anonymous namespace)::", "")
            f.write(f"{name[:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.3f} "
                    f"{float(r['MinNs']) / 1e3:>9.3f} {float(r['MaxNs']) / 1e3:>9.3f}\n")
    return out


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------

def _elapsed_us(torch, fn, n):
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for i in range(n):
        fn(i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / n


def _side_us(torch, fn, n=500, reps=3, warmup=30):
    """µs per call of a side measurement: warm-up calls, then the median of
    `reps` timed runs of n calls (steadier than one short run)."""
    for i in range(warmup):
        fn(i)
    return statistics.median(_elapsed_us(torch, fn, n) for _ in range(reps))


def graph_cold_us(torch, tsv, dev, w, op: str = "softmax", reps: int = 5) -> float:
    """µs per call, cold, from graph replay (launch gaps removed): rotating
    slices of one >= 512 MiB buffer pair, all captured into one graph and
    replayed `reps` times. op: "softmax" (ts_softmax), "copy" (the same-bytes
    copy), "sample" (ts_sample on the slices' probabilities), "ids" and
    "probs" (ts_softmax_sample without and with writing the probabilities),
    with w's uniforms."""
    B, V = w.B, w.V
    nsets = min(512, max(2, math.ceil((512 << 20) / (2 * B * V * 4))))
    x = torch.from_numpy(w.logits).to(dev).unsqueeze(0).repeat(nsets, 1, 1)
    t = torch.from_numpy(w.temps).to(dev)
    y = torch.empty_like(x)
    u = torch.from_numpy(w.uniforms).to(dev)
    ids = torch.empty((nsets, B, u.shape[1]), dtype=torch.int32, device=dev)
    s = torch.cuda.Stream(device=dev)
    tsv.ts_reserve(B, V, device=dev, stream=s)
    if op == "sample":
        with torch.cuda.stream(s):
            for i in range(nsets):
                tsv.ts_softmax(x[i], t, out=y[i])

    def calls():
        for i in range(nsets):
            if op == "copy":
                tsv.ts_copy_f32(x[i], y[i])
            elif op == "sample":
                tsv.ts_sample(y[i], u, out_ids=ids[i])
            elif op == "ids":
                tsv.ts_softmax_sample(x[i], t, u, out_ids=ids[i])
            elif op == "probs":
                tsv.ts_softmax_sample(x[i], t, u, out_ids=ids[i], probs_out=y[i])
            else:
                tsv.ts_softmax(x[i], t, out=y[i])
    with torch.cuda.stream(s):
        calls()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (reps * nsets)
    del x, y, ids, g
    return round(us, 3)


def configs_graph_us(torch, tsv, workloads, dev) -> dict:
    """µs per ts_softmax call for each of the five workloads, cold, by graph replay."""
    return {name: graph_cold_us(torch, tsv, dev, workloads.make_config(name)) for name in workloads.CONFIG_ORDER}


def shards_table(torch, tsv, workloads, dev, B: int, V: int) -> str:
    """One GPU's share of a (B, V) softmax split over G GPUs, by batch (B/G
    rows) and by vocabulary (V/G columns per row), for G in 1, 2, 4, 8: µs per
    call cold by graph replay, against a copy of the same bytes. The
    collectives the vocabulary split would add are not part of it."""
    lines = ["| G | share | B | V | softmax µs | copy µs | softmax / copy | GB/s |", "|---|---|---|---|---|---|---|---|"]
    for G in (1, 2, 4, 8):
        for kind, (b, v) in (("batch", (B // G, V)), ("vocabulary", (B, V // G))):
            if G == 1 and kind == "vocabulary":
                continue
            w = workloads.make(b, v, "quarters")
            sm = graph_cold_us(torch, tsv, dev, w)
            cp = graph_cold_us(torch, tsv, dev, w, "copy")
            gbs = 2 * b * v * 4 / sm / 1e3
            lines.append(f"| {G} | {kind if G > 1 else 'whole'} | {b} | {v} | {sm:.2f} | {cp:.2f} | "
                         f"{sm / cp:.3f} | {gbs:.0f} |")
            print(f"[shards] G={G} {kind} B={b} V={v} done", flush=True)
    return "\n".join(lines)


def _host_threads() -> int:
    """Host threads to give the oracle: the cores this process may run on,
    at most 16 (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_rate(w, target_s: float, threads: int):
    """Calls of the float64 oracle, as it stands, on the whole workload for
    about target_s seconds, after one untimed call; with threads > 1 the rows are split into that many
    blocks, each passed to the oracle on a thread of its own (numpy's loops
    release the GIL, and the oracle treats rows independently). Returns
    (GB/s of algorithmic bytes, calls, seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import softmax_ref
    bytes_per_call = 2 * w.B * w.V * 4
    blocks = [(lo, min(w.B, lo + -(-w.B // threads))) for lo in range(0, w.B, -(-w.B // threads))]
    pool = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None

    def one_call():
        if pool is None:
            softmax_ref(w.logits, w.temps)
        else:
            list(pool.map(lambda b: softmax_ref(w.logits[b[0]:b[1]], w.temps[b[0]:b[1]]), blocks))

    reps = 0
    try:
        one_call()   # untimed: the first touch of the oracle's temporaries
        t0 = time.perf_counter()
        while True:
            one_call()
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s or reps >= 1000:
                break
    finally:
        if pool is not None:
            pool.shutdown()
    return bytes_per_call * reps / el / 1e9, reps, el


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s: float):
    """The float64 oracle, as it stands, on the host over the same workload:
    first on one thread, then on every host core the process may use (rows
    split across threads). The all-cores rate is the value."""
    g1, r1, e1 = _oracle_rate(w, target_s / 2, 1)
    n = _host_threads()
    gn, rn, en = _oracle_rate(w, target_s / 2, n) if n > 1 else (g1, r1, e1)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"value": round(gn, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "cpu_model": _cpu_model(), "affinity_cores": affinity,
            "sample": f"full {w.name} workload (B={w.B}, V={w.V}), numpy float64; "
                      f"{n} threads over row blocks: {rn} calls in {en:.1f} s, us/call {en / rn * 1e6:.0f}; "
                      f"one thread: {r1} calls in {e1:.1f} s, {g1:.3f} GB/s, us/call {e1 / r1 * 1e6:.0f}"}


SWEEP_SHAPES = [(B, V) for V in (151936, 201088, 262144) for B in (1, 3, 8, 16, 32, 64, 128, 256)]


def sweep(torch, tsv, workloads, dev, shapes, steps: int) -> str:
    """Cold µs per call of every work split and chunk size, and of a copy of
    the same bytes, for each (B, V): the measurements behind the work-split
    table. Inputs rotate over >= 1 GiB as in the headline run; eager calls.
    Returns a markdown table (the plan's choice marked with *)."""
    splits = [(tsv.TS_VARIANT_FUSED, c) for c in tsv.CHUNKS] + \
             [(tsv.TS_VARIANT_SPLIT, c) for c in tsv.CHUNKS] + [(tsv.TS_VARIANT_ROWWISE, 0)]
    names = [f"{tsv.VARIANT_NAMES[v]} {c}" if c else tsv.VARIANT_NAMES[v] for v, c in splits]
    lines = ["| B | V | " + " | ".join(names) + " | copy | plan/best |",
             "|---|---|" + "---|" * (len(splits) + 2)]
    for B, V in shapes:
        w = workloads.make(B, V, "quarters")
        nsets = max(2, math.ceil(COLD_FOOTPRINT / (2 * B * V * 4)))
        xs = [torch.from_numpy(w.logits).to(dev) for _ in range(nsets)]
        t = torch.from_numpy(w.temps).to(dev)
        ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
        tsv.ts_reserve(B, V)
        plan = tsv.ts_plan(B, V)
        cells, best = [], (float("inf"), None)
        for v, c in splits:
            if v == tsv.TS_VARIANT_FUSED and -(-V // c) > 256:
                cells.append("—")
                continue
            def call(i, v=v, c=c):
                tsv.ts_softmax_variant(xs[i % nsets], t, v, c, out=ys[i % nsets])
            for i in range(10):
                call(i)
            us = _elapsed_us(torch, call, steps)
            mark = "*" if (v, c) == tuple(plan) or (v == plan[0] == tsv.TS_VARIANT_ROWWISE) else ""
            cells.append(f"{us:.2f}{mark}")
            if us < best[0]:
                best = (us, (v, c))
        cp = _elapsed_us(torch, lambda i: tsv.ts_copy_f32(xs[i % nsets], ys[i % nsets]), steps)
        pick = f"{tsv.VARIANT_NAMES[plan[0]]} {plan[1]} / {tsv.VARIANT_NAMES[best[1][0]]} {best[1][1]}"
        lines.append(f"| {B} | {V} | " + " | ".join(cells) + f" | {cp:.2f} | {pick} |")
        print(lines[-1], file=sys.stderr, flush=True)
        del xs, ys
    return "\n".join(lines)


PAGE_SHAPES = [(1, 151936), (4, 151936), (16, 201088), (64, 262144)]


def ab_guard(torch, tsv, workloads, dev, reps: int = 7, calls: int = 20) -> dict:
    """The pull-request page's A/B protocol on MI355X, with the library built
    with the -inf guard (libtsoftmax.so) and without it
    (libtsoftmax_noguard.so) in place of the page's main and fix: finite rows
    (seed B*7+V, logits N(0,1)*4, temperatures U[0.5, 1.5)) on the page's four
    shapes. It records, per shape, whether every work split gives bitwise the
    same probabilities in both builds, and the default plan's µs per call in
    both builds: graph replay of `calls` calls on the same buffers (hot, as the
    page timed), median of `reps` runs interleaved between the builds."""
    from temperature_softmax_vocabulary_amd import binding
    libs = {"guard": binding.lib(), "noguard": binding.load_library(binding.NOGUARD_LIB_PATH)}
    splits = [(tsv.TS_VARIANT_SPLIT, c) for c in tsv.CHUNKS] + \
             [(tsv.TS_VARIANT_FUSED, c) for c in tsv.CHUNKS] + [(tsv.TS_VARIANT_ROWWISE, 0)]
    dp = torch.cuda.get_device_properties(dev)
    out = {"device": dp.name, "gcn_arch": getattr(dp, "gcnArchName", ""), "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None), "calls_per_replay": calls, "runs": reps,
           "bitwise_equal": {}, "us_per_call": {}}
    for B, V in PAGE_SHAPES:
        w = workloads.make(B, V, "none")
        x = torch.from_numpy(w.logits).to(dev)
        t = torch.from_numpy(w.temps).to(dev)
        key = f"B{B}_V{V}"
        eq = {}
        for v, c in splits:
            ys = {}
            for name, L in libs.items():
                y = torch.empty_like(x)
                st = torch.cuda.current_stream().cuda_stream
                if L.ts_softmax_variant(x.data_ptr(), t.data_ptr(), None, B, V, y.data_ptr(), v, c, st) != 0:
                    raise SystemExit(f"{name} build failed on {key} {v}/{c}")
                ys[name] = y
            torch.cuda.synchronize()
            eq[f"{tsv.VARIANT_NAMES[v]}-{c}" if c else tsv.VARIANT_NAMES[v]] = bool(torch.equal(ys["guard"], ys["noguard"]))
        out["bitwise_equal"][key] = eq
        graphs = {}
        for name, L in libs.items():
            s = torch.cuda.Stream(device=dev)
            if L.ts_reserve(B, V, s.cuda_stream) != 0:
                raise SystemExit("ts_reserve failed")
            y = torch.empty_like(x)
            with torch.cuda.stream(s):
                L.ts_softmax(x.data_ptr(), t.data_ptr(), B, V, y.data_ptr(), s.cuda_stream)
            s.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(calls):
                    L.ts_softmax(x.data_ptr(), t.data_ptr(), B, V, y.data_ptr(), s.cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            graphs[name] = (g, y)
        runs = {name: [] for name in libs}
        for _ in range(reps):
            for name in libs:
                g = graphs[name][0]
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                runs[name].append(e0.elapsed_time(e1) * 1000.0 / calls)
        out["us_per_call"][key] = {name: round(statistics.median(r), 3) for name, r in runs.items()}
        out["us_per_call"][key]["plan"] = list(tsv.ts_plan(B, V))
        print(f"[ab-guard] {key}: bitwise {sum(eq.values())}/{len(eq)}, us {out['us_per_call'][key]}",
              file=sys.stderr, flush=True)
        del graphs
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", type=int, default=0, help="force a work split (0 = library's choice)")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extras", choices=("all", "copy", "draws", "draws-graph", "none"), default="all",
                    help="side measurements after the timed region: all, only the copy "
                         "(the counter runs' calibration), the copy and the eager draw calls "
                         "(the draw kernels' counter runs: no graph is captured), the draws "
                         "by graph replay only (the draw kernels' trace: every kernel queued "
                         "behind the one before, as in a busy stream), or none")
    ap.add_argument("--no-extras", action="store_true", help="same as --extras none")
    ap.add_argument("--ab-guard", action="store_true",
                    help="instead of the JSON line: the page's A/B (builds with and without the -inf "
                         "guard: bitwise map over every split, µs per call, median of 7 interleaved)")
    ap.add_argument("--shards", action="store_true",
                    help="print one GPU's share of the workload split over 2, 4, 8 GPUs (graph replay, cold)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the JSON line: a table of cold µs per call for every work split "
                         "and chunk size over B in {1..256} x V in {151936, 201088, 262144}")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--profile-command", default="python3 bench.py --steps 200 --warmup 20 --no-cpu-baseline",
                    help="the profiled command, recorded in the summaries")
    ap.add_argument("--summary-tag", default=None,
                    help="file tag of a summary (default: the profiled kernel's)")
    ap.add_argument("--kernel-name", default=None,
                    help="summarize this kernel (name substring) instead of the plan's")
    ap.add_argument("--alg-bytes", type=int, default=None,
                    help="algorithmic bytes per launch of --kernel-name (counter summaries)")
    args = ap.parse_args(argv)
    if args.no_extras:
        args.extras = "none"

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the softmax is sharded across GPUs by row or by vocabulary slice; "
              "the benchmark measures one GPU's share)", file=sys.stderr)
        return 2

    import torch
    import temperature_softmax_vocabulary_amd as tsv
    from temperature_softmax_vocabulary_amd import workloads

    if args.summarize_counters or args.summarize_trace:
        # host-side parsing only; the plan is given or read from the trace
        if args.kernel_name:
            name, tag = args.kernel_name, args.summary_tag or "kernel"
        elif not args.variant:
            raise SystemExit("--summarize-* needs --variant and --chunk of the profiled plan, or --kernel-name")
        else:
            name, tag = _kernel_names(tsv, (args.variant, args.chunk))
        if args.summarize_trace:
            print(summarize_trace(args.summarize_trace, args.workload, name, args.summary_tag or tag,
                                  args.profile_command))
        if args.summarize_counters:
            print(summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.workload,
                                     name, args.summary_tag or tag, args.profile_command, args.alg_bytes))
        return 0

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        print(sweep(torch, tsv, workloads, dev, SWEEP_SHAPES, min(args.steps, 200)), flush=True)
        return 0
    if args.shards:
        w = workloads.make_config(args.workload)
        print(shards_table(torch, tsv, workloads, dev, w.B, w.V), flush=True)
        return 0
    if args.ab_guard:
        print(json.dumps(ab_guard(torch, tsv, workloads, dev)), flush=True)
        return 0
    w = workloads.make_config(args.workload)
    B, V = w.B, w.V
    bytes_per_call = 2 * B * V * 4
    nsets = max(2, math.ceil(COLD_FOOTPRINT / bytes_per_call))
    xs = [torch.from_numpy(w.logits).to(dev) for _ in range(nsets)]
    ts = [torch.from_numpy(w.temps).to(dev) for _ in range(nsets)]
    ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
    plan = tsv.ts_plan(B, V) if not args.variant else (args.variant, args.chunk)
    kname, ktag = _kernel_names(tsv, plan)

    def step(i):
        j = i % nsets
        if args.variant:
            tsv.ts_softmax_variant(xs[j], ts[j], args.variant, args.chunk, out=ys[j])
        else:
            tsv.ts_softmax(xs[j], ts[j], out=ys[j])

    tsv.ts_reserve(B, V)
    print(f"[bench] workload={w.name} plan={plan} sets={nsets} warmup={args.warmup} steps={args.steps}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    us = _elapsed_us(torch, step, args.steps)            # the timed region: exactly K steps
    errs = tsv.ts_device_errors()
    y = ys[(args.steps - 1) % nsets]
    rowsum = y.double().sum(dim=1)
    sane = bool(torch.isfinite(y).all().item()) and float((rowsum - 1).abs().max().item()) < 1e-5
    print(f"[bench] cold {us:.2f} us/call, device errors {errs}, outputs sane {sane}", file=sys.stderr, flush=True)

    gbs = bytes_per_call / us / 1e3
    traffic = read_traffic(ktag, w.name)
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "us_per_call": round(us, 3),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "V": V, "masks": "quarters: none/first16384/block20000/allowed3",
                   "rotating_sets": nsets, "variant": tsv.VARIANT_NAMES[plan[0]], "chunk": plan[1],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "outputs_sane": sane,
    }

    extras = {}

    def leg(name):
        # names the leg on stderr before it starts, so that a run that ends
        # early (e.g. under a profiler) shows where
        print(f"[bench] leg {name}", file=sys.stderr, flush=True)

    if args.extras in ("all", "copy", "draws"):
        leg("copy")
        # same bytes through a plain streaming copy, cold (practical ceiling,
        # and the byte-counter calibration of the profile runs)
        def cp(i):
            j = i % nsets
            tsv.ts_copy_f32(xs[j], ys[j])
        for i in range(20):
            cp(i)
        cus = _elapsed_us(torch, cp, args.steps)
        extras["copy_us_per_call"] = round(cus, 3)
        extras["copy_GBps"] = round(bytes_per_call / cus / 1e3, 1)
        extras["softmax_over_copy"] = round(cus / us, 4)
    if args.extras in ("all", "draws"):
        # token draws on the same rows, 64 uniforms each (not part of the metric):
        # ts_sample on written probabilities, and the one-pass softmax + draw
        # with and without writing the probabilities (cold, rotating sets; eager)
        u = torch.from_numpy(w.uniforms).to(dev)
        ids = torch.empty((B, w.uniforms.shape[1]), dtype=torch.int32, device=dev)
        leg("draw: ts_sample")
        extras["sample_us_per_call"] = round(
            _side_us(torch, lambda i: tsv.ts_sample(ys[i % nsets], u, out_ids=ids)), 3)
        leg("draw: ids only")
        extras["softmax_sample_ids_only_us_per_call"] = round(
            _side_us(torch, lambda i: tsv.ts_softmax_sample(xs[i % nsets], ts[i % nsets], u, out_ids=ids)), 3)
        leg("draw: with probabilities")
        extras["softmax_sample_with_probs_us_per_call"] = round(
            _side_us(torch, lambda i: tsv.ts_softmax_sample(xs[i % nsets], ts[i % nsets], u, out_ids=ids,
                                                            probs_out=ys[i % nsets])), 3)
    if args.extras == "draws-graph":
        # the three draws by graph replay (cold): each call's kernels start as
        # the previous call's end, with no host gap between them
        leg("draws by graph replay")
        extras["graph_draw_us_per_call"] = {
            op: graph_cold_us(torch, tsv, dev, w, op, reps=40) for op in ("sample", "ids", "probs")}
    if args.extras == "all":
        # the softmax and the same-bytes copy in 7 interleaved runs of 200 cold
        # calls each: medians, and the median of the per-run ratios
        leg("interleaved")
        runs = []
        for _ in range(7):
            runs.append((_elapsed_us(torch, step, 200), _elapsed_us(torch, cp, 200)))
        extras["interleaved_7x200"] = {
            "softmax_us_median": round(statistics.median(r[0] for r in runs), 3),
            "copy_us_median": round(statistics.median(r[1] for r in runs), 3),
            "softmax_over_copy_median": round(statistics.median(r[1] / r[0] for r in runs), 4)}
        # hot: the same buffers every call (how the page timed, graph replays of one input)
        leg("hot")

        def hot(i):
            step(0)
        extras["hot_us_per_call"] = round(_side_us(torch, hot), 3)
        # graph replay of the same rotating calls (launch gaps removed)
        leg("graph")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        tsv.ts_reserve(B, V, stream=s)
        with torch.cuda.stream(s):
            for i in range(nsets):
                step(i)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(nsets * 8):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 5
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        extras["graph_us_per_call"] = round(e0.elapsed_time(e1) * 1000.0 / (reps * nsets * 8), 3)
        # the same masks applied from an allowed-id bitmask while the logits are read
        # (finite logits everywhere, B * ceil(V/32) * 4 extra bytes read)
        # (cold like the timed region: the logit and mask buffers rotate too)
        xm_host = workloads.unmasked_logits(w)
        bits_host = workloads.make_allowed(w).view(np.int32)
        xms = [torch.from_numpy(xm_host).to(dev) for _ in range(nsets)]
        bitss = [torch.from_numpy(bits_host.copy()).to(dev) for _ in range(nsets)]

        def masked(i):
            j = i % nsets
            tsv.ts_softmax_masked(xms[j], ts[j], bitss[j], out=ys[j])
        leg("bitmask")
        extras["masked_bitmask_us_per_call"] = round(_side_us(torch, masked), 3)
        del xms, bitss
        # every workload, graph replay (the small ones are launch-bound)
        leg("workloads by graph replay")
        extras["configs_graph_us_per_call"] = configs_graph_us(torch, tsv, workloads, dev)
        # the draws on every workload (64 uniforms per row), graph replay
        leg("draws on every workload by graph replay")
        extras["configs_graph_draw_us_per_call"] = {
            name: {op: graph_cold_us(torch, tsv, dev, workloads.make_config(name), op)
                   for op in ("sample", "ids", "probs")}
            for name in workloads.CONFIG_ORDER}
        dp = torch.cuda.get_device_properties(dev)
        clock_khz, bus_bits = tsv.ts_device_memory_params(dev)
        extras["device"] = {"name": dp.name, "cus": dp.multi_processor_count,
                            "gcn_arch": getattr(dp, "gcnArchName", ""),
                            # the peak recomputed from what HIP reports. HBM3E pins move
                            # 4 bits per reported memory clock (8 Gb/s at 2 GHz); 2 would
                            # put the peak below the rate the kernels sustain
                            "mem_clock_khz": clock_khz, "mem_bus_bits": bus_bits,
                            "hbm_peak_from_props_GBps": round(clock_khz * 1e3 * 4 * bus_bits / 8 / 1e9, 1)}
    if extras:
        extras["kernel_source_sha256"] = kernel_source_hash(ktag)
        result["extras"] = extras

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def _kernel_names(tsv, plan):
    """(kernel-name substring as rocprofv3 prints it, file tag) for a plan."""
    v, c = plan
    if v == tsv.TS_VARIANT_FUSED:
        return f"ts_fused<{c // 1024}, true, 0>", f"ts_fused_c{c}"
    if v == tsv.TS_VARIANT_SPLIT:
        return f"ts_split_finalize_write<{c // 1024}, true>", f"ts_split_c{c}"
    return "ts_rowwise", "ts_rowwise"


if __name__ == "__main__":
    sys.exit(main())
