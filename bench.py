#!/usr/bin/env python3
"""Benchmark of the low-M split-K bf16 GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the whole hot path (lowm_gemm_splitk: W stream, MFMA,
wavefront reduction, split-K publish/fold, bf16 store) on one set of inputs.
The workload is the headline shape of the TensorRT-LLM PR "Fix two
synchronization gaps in the MiniMax M3 low-M split-K GEMM" (Hardware
verification): M 4, N 6144, K 4096, split_k 2, with synthetic N(0,1)
activations and N(0,0.02) weights.  Inputs are resident in HBM before timing;
the calls rotate through a pool of input sets larger than twice the 256 MB
MALL so the weights stream from HBM rather than the Infinity Cache.

Prints one JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
MALL_BYTES = 256 << 20          # Infinity Cache
KERNEL_SOURCES = ROOT / "split_bf16_gemm_amd" / "csrc"
PMC_FILE = ROOT / "profiles" / "pmc_traffic.json"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def rnd(x, nd):
    return None if x is None else round(x, nd)


def algorithmic_bytes(M: int, N: int, K: int, S: int) -> int:
    """2KN (W once) + 2MK (A once) + 2MN (bf16 C) + 4MN(2S-1) workspace
    (every rank writes its fp32 partial, the owner reads the other S-1)."""
    ws = 4 * M * N * (2 * S - 1) if S > 1 else 0
    return 2 * K * N + 2 * M * K + 2 * M * N + ws


def source_hash() -> str:
    """Hash of the GEMM library's sources (the kernels and the host side)."""
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES.glob("lowm_*")) + [ROOT / "include" / "lowm.h"]:
        h.update(f.name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def parse_tactic(text):
    from split_bf16_gemm_amd import binding
    if not text:
        return None
    stage, rows, unroll, stages = text.split(":")
    return binding.tactic(stage, int(rows), int(unroll), int(stages))


class Pool:
    """Input sets (A, W, C, workspace) on the device, rotated call by call."""

    def __init__(self, lib, wl, sets: int, dev):
        import torch
        import workloads
        self.wl = wl
        M, N, K, S = wl.M, wl.N, wl.K, wl.split_k
        A0, W0 = workloads.make_inputs(wl)
        g = torch.Generator(device=dev)
        g.manual_seed(wl.seed_w + 7919)
        self.sets = []
        for i in range(sets):
            if i == 0:
                A, W = A0.to(dev), W0.to(dev)
            else:
                A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
                W = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = lib.make_workspace(M, N, K, S, dev)
            self.sets.append((A, W, C, ws))
        torch.cuda.synchronize()
        self.ptrs = [(A.data_ptr(), W.data_ptr(), C.data_ptr(), ws.data_ptr() if ws is not None else 0)
                     for (A, W, C, ws) in self.sets]


def make_caller(lib, wl, tactic, stream_handle):
    raw = lib.call_raw
    M, N, K, S = wl.M, wl.N, wl.K, wl.split_k

    def call(p):
        rc = raw(p[0], p[1], p[2], M, N, K, S, p[3], stream_handle, False, tactic)
        if rc:
            lib.check(rc)
    return call


def time_loop(call, ptrs, steps):
    """Elapsed time of `steps` back-to-back calls between two events (us/call)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        call(ptrs[i % len(ptrs)])
    end.record()
    end.synchronize()
    return start.elapsed_time(end) * 1e3 / steps


def time_each(call, ptrs, steps):
    """Average duration of one launch, from an event pair around each launch."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record()
        call(ptrs[i % len(ptrs)])
        evs[i][1].record()
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) * 1e3 for a, b in evs]
    return statistics.mean(d), statistics.median(d)


def time_graph(make_call, ptrs, steps, dev):
    """The same loop captured once in a HIP graph and replayed (us/call)."""
    import torch
    s = torch.cuda.Stream(device=dev)
    call = make_call(s.cuda_stream)       # launches must go to the capturing stream
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            call(ptrs[i % len(ptrs)])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) * 1e3 / steps


def hbm_read_ceiling(pool, dev, reps=5):
    """GB/s of a plain streaming read of each set's W, rotating like the GEMM."""
    import torch
    from split_bf16_gemm_amd import BwProbe
    bw = BwProbe()
    blocks = 1024
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    Ws = [s[1] for s in pool.sets]
    for W in Ws:
        bw.read(W, sink, blocks)
    res = []
    for _ in range(reps):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        n = 0
        for _ in range(4):
            for W in Ws:
                bw.read(W, sink, blocks)
                n += 1
        end.record()
        end.synchronize()
        us = start.elapsed_time(end) * 1e3 / n
        res.append(Ws[0].numel() * 2 / us / 1e3)
    return statistics.median(res)


def read_mall_warm(W, dev, steps, reps=5):
    """us per launch of the plain streaming read over one W again and again
    (the Infinity Cache holds it: not an HBM figure)."""
    import torch
    from split_bf16_gemm_amd import BwProbe
    bw = BwProbe()
    blocks = 1024
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    for _ in range(20):
        bw.read(W, sink, blocks)
    res = []
    for _ in range(reps):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            bw.read(W, sink, blocks)
        end.record()
        end.synchronize()
        res.append(start.elapsed_time(end) * 1e3 / steps)
    return statistics.median(res)


def launch_floor(blocks, steps, dev, reps=5):
    """us per launch of `steps` empty kernels with `blocks` workgroups of 256
    threads, captured in one graph and replayed: the GPU's fixed cost of a
    launch of the GEMM's grid.  (Issued one by one from Python, each launch
    costs the host more than the GPU, so a plain loop would time the host.)"""
    import torch
    from split_bf16_gemm_amd import BwProbe
    bw = BwProbe()
    s = torch.cuda.Stream(device=dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for _ in range(steps):
            rc = bw.lib.bwprobe_empty(blocks, s.cuda_stream)
            if rc:
                raise RuntimeError(f"bwprobe_empty failed: hipError {rc}")
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(reps):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        end.synchronize()
        res.append(start.elapsed_time(end) * 1e3 / steps)
    return statistics.median(res)


def pmc_traffic(wl, tactic_dict, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    if not PMC_FILE.exists():
        return None
    try:
        rec = json.loads(PMC_FILE.read_text())
    except ValueError:
        return None
    if rec.get("source_sha") != source_hash() or rec.get("workload") != wl.name:
        return None
    if rec.get("tactic") != tactic_dict:
        return None
    return rec.get("traffic_bytes_per_launch")


COPY_BYTES = 6144 * 4096 * 2


def calibrate_copy(dev, launches):
    """Copy COPY_BYTES between buffers `launches` times (source rotating over a
    pool larger than the MALL), for counter calibration under rocprofv3."""
    import torch
    from split_bf16_gemm_amd import BwProbe
    bw = BwProbe()
    srcs = [torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev) for _ in range(12)]
    dst = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    for i in range(launches):
        bw.copy(srcs[i % len(srcs)], dst, 2048)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "launches": launches}), flush=True)


def _counter_medians(run_dir: Path, counter: str) -> dict:
    """Median per-dispatch value of `counter` for every kernel in the
    rocprofv3 counter-collection CSVs under run_dir: {name: (median, n)}."""
    import csv
    vals: dict = {}
    for f in sorted(run_dir.rglob("*counter_collection.csv")):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: (statistics.median(v), len(v)) for k, v in vals.items()}


def summarize_pmc(wl_name: str, tactic_text, fetch: Path, write: Path, cfetch: Path,
                  cwrite: Path, out: Path = PMC_FILE) -> dict:
    """HBM bytes per launch of the GEMM kernel from four rocprofv3 --pmc runs
    (FETCH_SIZE and WRITE_SIZE of bench.py, then of --calibrate-copy), each
    scaled by what the counter reads for the copy of COPY_BYTES; written to
    `out` (PMC_FILE, the one roofline.traffic reads, unless another is named)
    with the kernel source hash, workload and tactic it belongs to."""
    import split_bf16_gemm_amd as sbg
    import workloads
    wl = workloads.by_name(wl_name)
    lib = sbg.load()
    tactic = parse_tactic(tactic_text)
    tac = tactic if tactic is not None else lib.pick_tactic(wl.M, wl.N, wl.K, wl.split_k)

    def gemm_value(d, counter):
        med = {k: v for k, v in _counter_medians(d, counter).items() if "lowm_" in k}
        name = max(med, key=lambda k: med[k][1])      # the kernel launched most often
        return name, med[name][0]

    def copy_value(d, counter):
        med = {k: v for k, v in _counter_medians(d, counter).items() if "copy_kernel" in k}
        return next(iter(med.values()))[0]

    kernel, f_kib = gemm_value(fetch, "FETCH_SIZE")
    _, w_kib = gemm_value(write, "WRITE_SIZE")
    cf_kib, cw_kib = copy_value(cfetch, "FETCH_SIZE"), copy_value(cwrite, "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / (cf_kib * 1024), COPY_BYTES / (cw_kib * 1024)
    traffic = round(f_kib * 1024 * f_scale + w_kib * 1024 * w_scale)
    rec = {"source_sha": source_hash(), "workload": wl.name, "tactic": tac.as_dict(),
           "kernel": kernel, "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
           "copy_fetch_kib_per_dispatch": cf_kib, "copy_write_kib_per_dispatch": cw_kib,
           "copy_bytes": COPY_BYTES, "fetch_scale": round(f_scale, 5),
           "write_scale": round(w_scale, 5), "traffic_bytes_per_launch": traffic,
           "algorithmic_bytes_per_launch": algorithmic_bytes(wl.M, wl.N, wl.K, wl.split_k)}
    out.write_text(json.dumps(rec, indent=1) + "\n")
    return rec


def counter_summary(dirs, kernel_filter="lowm_"):
    """Markdown table of the median per-dispatch value of every counter in
    rocprofv3 --pmc output directories, per kernel whose name contains
    kernel_filter (no GPU needed)."""
    import csv
    rows: dict = {}
    for d in dirs:
        for f in sorted(Path(d).rglob("*counter_collection.csv")):
            with open(f, newline="") as fh:
                for row in csv.DictReader(fh):
                    k = row.get("Kernel_Name", "")
                    if kernel_filter not in k:
                        continue
                    k = k.split("(")[0]
                    rows.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(
                        float(row["Counter_Value"]))
    for k, counters in rows.items():
        print(f"\n**{k}**\n")
        print("| counter | median per dispatch | dispatches |")
        print("|---|---|---|")
        for c in sorted(counters):
            v = counters[c]
            print(f"| {c} | {statistics.median(v):,.0f} | {len(v)} |")


def trace_breakdown(dev, wl, tactic, launches=4):
    """Where a launch's time goes, from the stress build's per-workgroup
    timestamps (s_memrealtime, 100 MHz): dispatch (first entry to this
    workgroup's entry), first data (entry to its first stage or line pair in
    LDS), stream (to the end of its main loop), reduction (wavefront sums
    through LDS), tail (publish / exchange / fold / store, to its end).
    Medians over all workgroups and over the last 5 % to end, per traced
    launch; traced launches alternate with untraced ones through the same
    rotated pool.  The timestamp stores share the vector-memory counter with
    the loads, so the traced kernel waits a little more than the product
    kernel: a picture of the timeline, not a timing."""
    import numpy as np
    import torch
    import split_bf16_gemm_amd as sbg
    stress = sbg.load("stress")
    M, N, K, S = wl.M, wl.N, wl.K, wl.split_k
    tac = tactic if tactic is not None else stress.pick_tactic(M, N, K, S)
    from split_bf16_gemm_amd import binding
    tiles = -(-N // tac.rows)
    # quarter-rows tiles: one workgroup per block of 16*unroll activation rows
    blocks = -(-M // (16 * tac.unroll)) if tac.stage == binding.LOWM_STAGE_QUARTER_ROWS else 1
    grid = (tiles + 7) // 8 * 8 * S * blocks
    T = stress.TRACE_SLOTS
    per_set = 2 * K * N + 2 * M * K + 2 * M * N + stress.workspace_bytes(M, N, K, S)
    sets = max(2, math.ceil(2 * MALL_BYTES / per_set) + 1)
    pool = Pool(stress, wl, sets, dev)
    call = make_caller(stress, wl, tactic, torch.cuda.current_stream(dev).cuda_stream)
    for i in range(2 * sets):
        call(pool.ptrs[i % sets])
    torch.cuda.synchronize()
    buf = torch.zeros(grid * T, dtype=torch.int64, device=dev)
    print(f"{wl.name}, tactic {tactic_text(tac)}, {grid} workgroups ({tiles} tiles x "
          f"split_k {S}" + (f" x {blocks} row blocks" if blocks > 1 else "") +
          "); microseconds from the first workgroup's entry")
    print("| launch | span | WGs | dispatch | first data | stream | reduction | tail | "
          "last 5 %: dispatch | first data | stream | reduction | tail | end | early owners |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    ends = []
    for it in range(launches):
        buf.zero_()
        torch.cuda.synchronize()
        stress.trace(buf)
        try:
            call(pool.ptrs[it % sets])
            torch.cuda.synchronize()
        finally:
            stress.trace(None)
        call(pool.ptrs[(it + 1) % sets])
        torch.cuda.synchronize()
        tr = buf.view(grid, T).cpu().numpy().astype(np.int64)
        valid = (tr[:, 8] < tiles) & (tr[:, 5] > 0)
        t = tr[valid]
        t0 = t[:, 0].min()
        us = (t[:, :6] - t0) / 100.0
        entry, first, lend, red, arr, end = (us[:, c] for c in range(6))
        red = np.where(t[:, 3] > 0, red, lend)
        segs = [entry, first - entry, lend - first, red - lend, end - red]
        last = end >= np.percentile(end, 95)
        early = int(((t[:, 4] == 0) & (t[:, 9] == S - 1)).sum()) if S > 1 else 0
        cells = [f"{np.median(x):.2f}" for x in segs] + \
                [f"{np.median(x[last]):.2f}" for x in segs] + [f"{np.median(end[last]):.2f}"]
        print(f"| {it} | {end.max():.2f} | {int(valid.sum())} | " + " | ".join(cells) +
              f" | {early} |", flush=True)
        ends.append((end, t[:, 9], t[:, 7], first))
    # per rank and per XCD: when workgroups end, and when their first data came
    end = np.concatenate([e[0] for e in ends])
    rank = np.concatenate([e[1] for e in ends])
    xcd = np.concatenate([e[2] for e in ends])
    first = np.concatenate([e[3] for e in ends])
    print()
    print("| group | WGs | first data median / p95 | end median / p95 / max |")
    print("|---|---|---|---|")
    for label, key, values in (("rank", rank, range(S)), ("XCD", xcd, sorted(set(xcd.tolist())))):
        for v in values:
            sel = key == v
            if sel.any():
                print(f"| {label} {v} | {int(sel.sum()) // launches} | "
                      f"{np.median(first[sel]):.2f} / {np.percentile(first[sel], 95):.2f} | "
                      f"{np.median(end[sel]):.2f} / {np.percentile(end[sel], 95):.2f} / "
                      f"{end[sel].max():.2f} |")


def host_threads() -> int:
    """Worker threads for the oracle: the CPUs this process may run on, at
    most 16 (one GPU's share of the box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_product(orc, a, w, threads: int):
    """The whole product C = A W^T from the oracle's column-range entry,
    split over `threads` Python threads by columns (each ctypes call releases
    the GIL, so the ranges run in parallel; the arithmetic per column is the
    oracle's own)."""
    from concurrent.futures import ThreadPoolExecutor
    N = w.shape[0]
    if threads == 1:
        return orc.gemm_cols(a, w, 0, N)
    bounds = [N * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda i: orc.gemm_cols(a, w, bounds[i], bounds[i + 1]),
                            range(threads)))
    import numpy as np
    return np.concatenate([c for c, _ in parts], axis=1), np.concatenate([s for _, s in parts],
                                                                         axis=1)


def time_oracle(wl, threads: int, min_runs: int = 3, budget_s: float = 5.0):
    """Median ms per whole product of the fp64 oracle on `threads` host
    threads: at least min_runs products, more while within budget_s."""
    import oracle
    import workloads
    A, W = workloads.make_inputs(wl)
    a, w = workloads.bits(A), workloads.bits(W)
    orc = oracle.default()
    times = []
    t_start = time.perf_counter()
    while len(times) < min_runs or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        oracle_product(orc, a, w, threads)
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    return statistics.median(times) * 1e3, len(times)


def cpu_baseline(wl):
    """The fp64 oracle on the host cores, for the benchmark's JSON line: whole
    products of the workload, on one thread and on T threads (columns split
    between them), median of at least 3 each, about 10 s of CPU time in all.
    `value` is the T-thread rate in the metric's unit."""
    T = host_threads()
    ms1, n1 = time_oracle(wl, 1)
    msT, nT = time_oracle(wl, T)
    b = algorithmic_bytes(wl.M, wl.N, wl.K, wl.split_k)
    return {"value": round(b / (msT * 1e-3) / 1e9, 4), "unit": "GB/s", "cores": T,
            "kind": "oracle",
            "sample": f"whole {wl.name} products (fp64, columns split over {T} threads): "
                      f"median of {nT}; single thread: median of {n1}",
            "ms_per_call": round(msT, 2), "ms_per_call_1_thread": round(ms1, 2),
            "value_1_thread": round(b / (ms1 * 1e-3) / 1e9, 4),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_table():
    """Markdown table: the fp64 oracle's ms per whole product, 1 thread and
    T threads, for the pages' shapes and the ends of the M sweep (the oracle
    does not depend on split_k)."""
    import workloads
    T = host_threads()
    model = cpu_model()
    names = ["int_closed_form_m4_n512_k1024_s2", "m4_n6144_k4096_s2", "m4_n2304_k12288_s4",
             "m4_n49152_k4096_s2", "sweep_m1_n6144_k4096_s1", "sweep_m64_n6144_k4096_s1"]
    print(f"host: {os.cpu_count()} CPUs visible, {T} used; {model}")
    print("| workload | oracle ms, 1 thread | oracle ms, T threads | T | CPU model |")
    print("|---|---|---|---|---|")
    for name in names:
        wl = workloads.by_name(name)
        ms1, _ = time_oracle(wl, 1, budget_s=0)
        msT, _ = time_oracle(wl, T, budget_s=0)
        print(f"| {name} | {ms1:.1f} | {msT:.1f} | {T} | {model} |", flush=True)


def config_table(lib, dev, steps, reps):
    """One markdown row per configuration: us/call back-to-back and replayed
    from a graph, GB/s and % of peak, each W streamed from HBM (rotated pool),
    and the plain streaming read of the same weights through the same pool
    (the read kernel of the bandwidth probe: its us per W, and the GEMM's
    excess over it)."""
    import torch
    import workloads
    from split_bf16_gemm_amd import BwProbe
    bw = BwProbe()
    print("| workload | tactic | bytes/call | us/call (plain) | us/call (graph) | GB/s | "
          "% of 8 TB/s | plain read of W (us) | GEMM - read (us) |")
    print("|---|---|---|---|---|---|---|---|---|")
    for wl in workloads.ALL:
        M, N, K, S = wl.M, wl.N, wl.K, wl.split_k
        tac = lib.pick_tactic(M, N, K, S)
        per_set = 2 * K * N + 2 * M * K + 2 * M * N + lib.workspace_bytes(M, N, K, S)
        sets = max(2, math.ceil(2 * MALL_BYTES / per_set) + 1)
        pool = Pool(lib, wl, sets, dev)
        call = make_caller(lib, wl, None, torch.cuda.current_stream(dev).cuda_stream)
        for i in range(20):
            call(pool.ptrs[i % sets])
        torch.cuda.synchronize()
        us = statistics.median(time_loop(call, pool.ptrs, steps) for _ in range(reps))
        try:
            ug = statistics.median(
                time_graph(lambda h: make_caller(lib, wl, None, h), pool.ptrs, steps, dev)
                for _ in range(reps))
        except Exception:  # graph capture is an extra figure
            ug = float("nan")
        sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
        # the read of each set's W, rotating like the GEMM
        reads = [lambda W=st[1]: bw.read(W, sink, 1024) for st in pool.sets]
        for r in reads:
            r()
        torch.cuda.synchronize()
        ur = statistics.median(time_loop(lambda f: f(), reads, steps) for _ in range(reps))
        nbytes = algorithmic_bytes(M, N, K, S)
        gbps = nbytes / us / 1e3
        print(f"| {wl.name} | {tactic_text(tac)} | {nbytes:,} | "
              f"{us:.2f} | {ug:.2f} | {gbps:.0f} | {100 * gbps / PEAK_HBM_GBPS:.1f} | "
              f"{ur:.2f} | {us - ur:+.2f} |", flush=True)
        del pool
        torch.cuda.empty_cache()


BATCH_CASES = [  # (label, M, [N...], K, split_k)
    ("Q/K/V: N 6144 + 1024 + 1024, K 4096, split_k 2", 4, [6144, 1024, 1024], 4096, 2),
    ("gate/up: 2 x N 6144, K 4096, split_k 2", 4, [6144, 6144], 4096, 2),
    ("8 x N 512, K 4096, split_k 2", 4, [512] * 8, 4096, 2),
    ("3 x N 2304, K 12288, split_k 4", 4, [2304] * 3, 12288, 4),
    ("1 x N 6144, K 4096, split_k 2", 4, [6144], 4096, 2),
]


def batched_table(lib, dev, steps, reps):
    """One markdown row per batch of GEMMs: us per step for one batched launch
    and for one launch per GEMM, each back-to-back and as `steps` steps
    captured in one graph and replayed; W from HBM through a rotated pool."""
    import torch
    from split_bf16_gemm_amd import binding
    print("| batch (M 4) | bytes/step | batched | separate | graph, batched | graph, separate | "
          "GB/s batched (% of 8 TB/s) |")
    print("|---|---|---|---|---|---|---|")
    for label, M, Ns, K, S in BATCH_CASES:
        per_set = sum(2 * K * N + 2 * M * K + 2 * M * N for N in Ns) + \
            lib.batched_workspace_bytes(M, Ns, K, S)
        sets = max(2, math.ceil(2 * MALL_BYTES / per_set) + 1)
        g = torch.Generator(device=dev)
        g.manual_seed(9000 + len(Ns))
        pool = []
        for _ in range(sets):
            As = [torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16) for _ in Ns]
            Ws = [(torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
                  for N in Ns]
            Cs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for N in Ns]
            ws_b = torch.zeros(max(1, lib.batched_workspace_bytes(M, Ns, K, S)), dtype=torch.uint8,
                               device=dev)
            ws_s = [lib.make_workspace(M, N, K, S, dev) for N in Ns]
            pool.append((lib.descs(As, Ws, Cs), ws_b, [(A.data_ptr(), W.data_ptr(), C.data_ptr(),
                                                        0 if w is None else w.data_ptr(), N)
                                                       for A, W, C, w, N in zip(As, Ws, Cs, ws_s, Ns)],
                         (As, Ws, Cs, ws_s)))
        torch.cuda.synchronize()

        def batched(h):
            def call(item):
                rc = lib.lib.lowm_gemm_splitk_batched(item[0], len(Ns), M, K, S,
                                                      item[1].data_ptr() if S > 1 else None, h)
                if rc:
                    lib.check(rc)
            return call

        def separate(h):
            def call(item):
                for a, w, c, ws, N in item[2]:
                    rc = lib.call_raw(a, w, c, M, N, K, S, ws, h)
                    if rc:
                        lib.check(rc)
            return call

        cur = torch.cuda.current_stream(dev).cuda_stream
        for f in (batched(cur), separate(cur)):
            for i in range(sets):
                f(pool[i])
        torch.cuda.synchronize()
        ub = statistics.median(time_loop(batched(cur), pool, steps) for _ in range(reps))
        us_ = statistics.median(time_loop(separate(cur), pool, steps) for _ in range(reps))
        gb = statistics.median(time_graph(batched, pool, steps, dev) for _ in range(reps))
        gs = statistics.median(time_graph(separate, pool, steps, dev) for _ in range(reps))
        nbytes = sum(algorithmic_bytes(M, N, K, S) for N in Ns)
        gbps = nbytes / ub / 1e3
        print(f"| {label} | {nbytes:,} | {ub:.2f} | {us_:.2f} | {gb:.2f} | {gs:.2f} | "
              f"{gbps:.0f} ({100 * gbps / PEAK_HBM_GBPS:.1f} %) |", flush=True)
        del pool
        torch.cuda.empty_cache()


def time_shape(lib, dev, M, N, K, S, tactic, steps, reps, seed=0):
    """us/call of back-to-back launches of one shape and tactic (None: the
    default), W streamed from HBM through a rotated pool of synthetic input
    sets larger than twice the MALL; median of `reps` timed loops.  Returns
    None when the build has no such tactic for the shape."""
    import torch
    import workloads
    from split_bf16_gemm_amd import binding
    if lib.check_launch(M, N, K, S, tactic=tactic) != binding.LOWM_OK:
        return None
    wl = workloads.Workload(f"shape_m{M}_n{N}_k{K}_s{S}", M, N, K, S,
                            seed_a=3000 + seed, seed_w=4000 + seed)
    per_set = 2 * K * N + 2 * M * K + 2 * M * N + lib.workspace_bytes(M, N, K, S)
    sets = max(2, math.ceil(2 * MALL_BYTES / per_set) + 1)
    pool = Pool(lib, wl, sets, dev)
    call = make_caller(lib, wl, tactic, torch.cuda.current_stream(dev).cuda_stream)
    for i in range(max(10, sets)):
        call(pool.ptrs[i % sets])
    torch.cuda.synchronize()
    us = statistics.median(time_loop(call, pool.ptrs, steps) for _ in range(reps))
    del pool
    torch.cuda.empty_cache()
    return us


FENCE_WORKLOADS = ["m4_n6144_k4096_s2", "m4_n2304_k12288_s4", "sweep_m1_n6144_k4096_s8",
                   "sweep_m8_n6144_k4096_s8", "sweep_m16_n6144_k4096_s4",
                   "sweep_m32_n6144_k4096_s2", "sweep_m64_n6144_k4096_s2"]


def fence_ab(dev, steps, reps):
    """Markdown table: us/call of the default build against the fenced build
    (release arrival, acquire fence in the owner), default tactic, same
    pool, alternating the two libraries twice per workload."""
    import split_bf16_gemm_amd as sbg
    import workloads
    libs = {"default": sbg.load(), "fenced": sbg.load("fenced")}
    print("| workload | tactic | default build (us) | fenced build (us) | fenced / default |")
    print("|---|---|---|---|---|")
    for name in FENCE_WORKLOADS:
        wl = workloads.by_name(name)
        res = {k: [] for k in libs}
        for r in range(2):
            for k, lib in libs.items():
                res[k].append(time_shape(lib, dev, wl.M, wl.N, wl.K, wl.split_k, None, steps,
                                         reps, seed=r))
        d, f = statistics.median(res["default"]), statistics.median(res["fenced"])
        t = tactic_text(libs["default"].pick_tactic(wl.M, wl.N, wl.K, wl.split_k))
        print(f"| {name} | {t} | {d:.2f} | {f:.2f} | {f / d:.2f} |", flush=True)


PUSH_WORKLOADS = ["m4_n6144_k4096_s2", "m4_n2304_k12288_s4", "sweep_m1_n6144_k4096_s1",
                  "sweep_m16_n6144_k4096_s2", "sweep_m64_n6144_k4096_s2"]


def push_ab(lib, dev, steps, reps):
    """Markdown table: us/call of lowm_gemm_splitk against lowm_gemm_splitk_push
    (the owner also writes its tile to an exchange buffer and raises one flag
    per 16 columns), default tactic, the same rotated pool."""
    import torch
    import workloads
    print("| workload | tactic | plain (us) | push (us) | push - plain (us) |")
    print("|---|---|---|---|---|")
    stream = torch.cuda.current_stream(dev).cuda_stream
    for name in PUSH_WORKLOADS:
        wl = workloads.by_name(name)
        M, N, K, S = wl.M, wl.N, wl.K, wl.split_k
        per_set = 2 * K * N + 2 * M * K + 4 * M * N + lib.workspace_bytes(M, N, K, S)
        sets = max(2, math.ceil(2 * MALL_BYTES / per_set) + 1)
        pool = Pool(lib, wl, sets, dev)
        bufs = [(torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 torch.zeros((N + 15) // 16, dtype=torch.int32, device=dev)) for _ in range(sets)]
        ptrs = [p + (b.data_ptr(), f.data_ptr()) for p, (b, f) in zip(pool.ptrs, bufs)]
        plain = make_caller(lib, wl, None, stream)
        fn = lib.lib.lowm_gemm_splitk_push

        def push(p):
            rc = fn(p[0], p[1], p[2], M, N, K, S, p[3], p[4], N, p[5], 1, stream, None)
            if rc:
                lib.check(rc)
        for i in range(max(10, sets)):
            plain(ptrs[i % sets])
            push(ptrs[i % sets])
        torch.cuda.synchronize()
        res = {"plain": [], "push": []}
        for _ in range(reps):
            res["plain"].append(time_loop(plain, ptrs, steps))
            res["push"].append(time_loop(push, ptrs, steps))
        a, b = statistics.median(res["plain"]), statistics.median(res["push"])
        t = tactic_text(lib.pick_tactic(M, N, K, S))
        print(f"| {name} | {t} | {a:.2f} | {b:.2f} | {b - a:+.2f} |", flush=True)
        del pool, bufs
        torch.cuda.empty_cache()


def tactic_text(t) -> str:
    stage = repr(t).split("(")[1].split(",")[0]
    return f"{stage}:{t.rows}:{t.unroll}:{t.stages}"


def tactic_matrix(lib, dev, workload_names, tactic_texts, steps, reps):
    """Markdown table: us/call (and % of 8 TB/s) of every listed tactic on
    every listed workload ('default' is the tactic lowm_pick_tactic gives)."""
    import workloads
    print("| workload | " + " | ".join(tactic_texts) + " | best |")
    print("|---|" + "---|" * (len(tactic_texts) + 1))
    for name in workload_names:
        wl = workloads.by_name(name)
        M, N, K, S = wl.M, wl.N, wl.K, wl.split_k
        nbytes = algorithmic_bytes(M, N, K, S)
        cells, best = [], None
        for text in tactic_texts:
            t = None if text == "default" else parse_tactic(text)
            us = time_shape(lib, dev, M, N, K, S, t, steps, reps)
            if us is None:
                cells.append("—")
                continue
            label = text if t is not None else f"default ({tactic_text(lib.pick_tactic(M, N, K, S))})"
            if best is None or us < best[0]:
                best = (us, label)
            cells.append(f"{us:.2f} ({100 * nbytes / us / 1e3 / PEAK_HBM_GBPS:.1f} %)")
        print(f"| {name} | " + " | ".join(cells) + f" | {best[1] if best else '—'} |", flush=True)


SPLIT_GRID = {"M": (4, 16, 32, 64), "N": (768, 1536, 3072, 6144, 12288, 24576),
              "K": (2048, 4096, 8192, 16384), "S": (1, 2, 4, 8)}


def split_sweep(lib, dev, Ms, steps, reps):
    """For each (M, N, K) of the grid: us/call with the default tactic at
    split_k 1, 2, 4, 8, the fastest split_k, and what lowm_pick_split_k says."""
    print("| M | N | K | " + " | ".join(f"split_k {s}" for s in SPLIT_GRID["S"]) +
          " | fastest | picked |")
    print("|---|---|---|" + "---|" * (len(SPLIT_GRID["S"]) + 2))
    for M in Ms:
        for N in SPLIT_GRID["N"]:
            for K in SPLIT_GRID["K"]:
                times = {}
                for S in SPLIT_GRID["S"]:
                    us = time_shape(lib, dev, M, N, K, S, None, steps, reps, seed=S)
                    if us is not None:
                        times[S] = us
                best = min(times, key=times.get)
                cells = [f"{times[S]:.2f}" if S in times else "—" for S in SPLIT_GRID["S"]]
                print(f"| {M} | {N} | {K} | " + " | ".join(cells) +
                      f" | {best} | {lib.pick_split_k(M, N, K)} |", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="m4_n6144_k4096_s2")
    ap.add_argument("--tactic", default=None, help="stage:rows:unroll:stages, e.g. reg:16:4:3")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--only-gemm", action="store_true",
                    help="time only the GEMM loop (for profiler runs): no event pairs, graph, "
                         "MALL-warm, read ceiling or launch floor figures")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="no GPU: write the HBM traffic record from four rocprofv3 --pmc "
                         "output directories (FETCH_SIZE, WRITE_SIZE of this bench, then of "
                         "--calibrate-copy)")
    ap.add_argument("--pmc-file", default=str(PMC_FILE),
                    help="where --summarize-pmc writes its record (default: the one "
                         "roofline.traffic reads)")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="no GPU: print the median per-dispatch value of every counter in "
                         "these rocprofv3 --pmc output directories, per GEMM kernel")
    ap.add_argument("--table", action="store_true",
                    help="time every configuration (plain loop and graph replay, weights "
                         "from HBM) and print a markdown table instead of the JSON line")
    ap.add_argument("--tactic-matrix", nargs=2, metavar=("WORKLOADS", "TACTICS"),
                    help="comma-separated workload names and tactics (stage:rows:unroll:stages "
                         "or 'default'): print a markdown table of us/call, W from HBM")
    ap.add_argument("--split-sweep", metavar="MS",
                    help="comma-separated M values: time split_k 1/2/4/8 with the default "
                         "tactic over the N x K grid and print the fastest per shape")
    ap.add_argument("--trace", action="store_true",
                    help="timeline of --workload (and --tactic) from the stress build's "
                         "per-workgroup timestamps; print a markdown table")
    ap.add_argument("--batched", action="store_true",
                    help="time batched launches against one launch per GEMM (plain loop and "
                         "one captured graph of all steps); print a markdown table")
    ap.add_argument("--fence-ab", action="store_true",
                    help="time the default build against the fenced comparison build "
                         "(python -m split_bf16_gemm_amd.build liblowm_fenced.so first); print "
                         "a markdown table")
    ap.add_argument("--push-ab", action="store_true",
                    help="time the push epilogue entry point against the plain one; print a "
                         "markdown table")
    ap.add_argument("--cpu-table", action="store_true",
                    help="no GPU: time the fp64 oracle (1 and T threads) on the pages' "
                         "shapes and the M-sweep ends; print a markdown table")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only the plain copy kernel (50,331,648 bytes per launch) so "
                         "profiler byte counters can be scaled against a known size")
    args = ap.parse_args()

    if args.summarize_pmc:
        rec = summarize_pmc(args.workload, args.tactic, *(Path(d) for d in args.summarize_pmc),
                            out=Path(args.pmc_file))
        print(json.dumps(rec), flush=True)
        return

    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.cpu_table:
        cpu_table()
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import split_bf16_gemm_amd as sbg
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(dev, args.steps)
        return
    lib = sbg.load()
    if args.table:
        config_table(lib, dev, args.steps, args.reps)
        return
    if args.batched:
        batched_table(lib, dev, args.steps, args.reps)
        return
    if args.trace:
        trace_breakdown(dev, workloads.by_name(args.workload), parse_tactic(args.tactic))
        return
    if args.tactic_matrix:
        names, tacs = (x.split(",") for x in args.tactic_matrix)
        tactic_matrix(lib, dev, names, tacs, args.steps, args.reps)
        return
    if args.push_ab:
        push_ab(lib, dev, args.steps, args.reps)
        return
    if args.fence_ab:
        fence_ab(dev, args.steps, args.reps)
        return
    if args.split_sweep:
        split_sweep(lib, dev, [int(m) for m in args.split_sweep.split(",")], args.steps, args.reps)
        return
    wl = workloads.by_name(args.workload)
    M, N, K, S = wl.M, wl.N, wl.K, wl.split_k
    tactic = parse_tactic(args.tactic)
    tac = tactic if tactic is not None else lib.pick_tactic(M, N, K, S)
    per_set = 2 * K * N + 2 * M * K + 2 * M * N + lib.workspace_bytes(M, N, K, S)
    sets = max(2, math.ceil(2 * MALL_BYTES / per_set) + 1)
    log(f"workload {wl.name}: tactic {tac!r}, pool {sets} sets x {per_set / 1e6:.1f} MB")
    pool = Pool(lib, wl, sets, dev)
    stream = torch.cuda.current_stream(dev)
    call = make_caller(lib, wl, tactic, stream.cuda_stream)

    for i in range(args.warmup):
        call(pool.ptrs[i % sets])
    torch.cuda.synchronize()

    us_loop = statistics.median(time_loop(call, pool.ptrs, args.steps) for _ in range(args.reps))
    grid = (-(-N // tac.rows) + 7) // 8 * 8 * S      # the GEMM's workgroups
    us_kernel = us_kernel_med = us_warm = us_graph = ceiling = floor_us = read_warm_us = None
    if not args.only_gemm:
        each = [time_each(call, pool.ptrs, args.steps) for _ in range(args.reps)]
        us_kernel = statistics.median(e[0] for e in each)
        us_kernel_med = statistics.median(e[1] for e in each)
        us_warm = statistics.median(time_loop(call, pool.ptrs[:1], args.steps)
                                    for _ in range(args.reps))
        if not args.no_graph:
            try:
                us_graph = statistics.median(
                    time_graph(lambda h: make_caller(lib, wl, tactic, h), pool.ptrs, args.steps,
                               dev)
                    for _ in range(args.reps))
            except Exception as e:  # graph capture is an extra figure, not the metric
                log(f"graph timing skipped: {e}")
        ceiling = hbm_read_ceiling(pool, dev)
        floor_us = launch_floor(grid, args.steps, dev)
        read_warm_us = read_mall_warm(pool.sets[0][1], dev, args.steps)

    nbytes = algorithmic_bytes(M, N, K, S)
    gbps = nbytes / us_loop / 1e3
    # Average duration per launch from the events around the timed region
    # (the profiler's per-kernel average agrees within the launch gap); event
    # pairs around every launch add several microseconds of their own.
    achieved = gbps
    log(f"us/call {us_loop:.3f} (plain loop), kernel {us_kernel} avg / {us_kernel_med} "
        f"median (event pairs), graph {us_graph}, MALL-warm {us_warm}; "
        f"HBM read ceiling {ceiling} GB/s; empty kernel, {grid} workgroups: {floor_us} us")

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)
    out = {
        "metric": "µs/call + achieved HBM GB/s (% of peak), M=4 N=6144 K=4096 split_k=2",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_loop / 1e3, 6),
        "us_per_call": round(us_loop, 3),
        "pct_of_peak_hbm": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "M": M, "N": N, "K": K, "split_k": S,
            "tactic": tac.as_dict(), "bytes_per_call": nbytes, "pool_sets": sets,
            "seeds": {"a": wl.seed_a, "w": wl.seed_w},
        },
        "timings_us": {
            "plain_loop_per_call": round(us_loop, 3),
            "kernel_avg_event_pairs": rnd(us_kernel, 3),
            "kernel_median_event_pairs": rnd(us_kernel_med, 3),
            "graph_replay_per_call": rnd(us_graph, 3),
            "mall_warm_single_set_not_hbm": rnd(us_warm, 3),
            "empty_kernel_same_grid_graph": rnd(floor_us, 3),
            "plain_read_mall_warm_not_hbm": rnd(read_warm_us, 3),
        },
        "hbm_read_ceiling_gbps": rnd(ceiling, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": pmc_traffic(wl, tac.as_dict(), nbytes),
        },
        "cpu_baseline": cpu,
        "kernel_source_sha": source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
