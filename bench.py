#!/usr/bin/env python3
"""Benchmark of the few-row quantized verify GEMM on one MI355X.

Headline workload: 2-bit affine g64 weights, MLP up-projection shape K=5120, N=17408,
fp16 activations, verify calls at every row count M = 1..8.  A "step" is one verify call
at each M (8 calls).  The timed region runs exactly `--steps` steps, split into `--trials`
trials; each trial runs one block of calls per row count with a HIP event pair around it
(events on the stream the kernels run on), and the calls cycle through a pool of >= 1 GiB of
distinct weight copies so the 256 MB Infinity Cache cannot serve repeated calls.  Inputs
are resident in HBM before timing starts.

Before each block a gate (the library's streaming read over a 1 GiB buffer) holds the GPU
while the host enqueues the block, so the block's event pair times the calls running back
to back on the device rather than the host's submission rate; host_us_per_call reports
the latter.  Before anything is timed the GPU runs 50 ms of streaming reads (clock
settle: the first ~10 ms of back-to-back work run up to 10% slower, measured on MI355X),
then the `--warmup` untimed steps.  Per-M figures are the median over the trials (the min
is given too).

stream_ceiling times the library's plain streaming-read kernel over the same bytes and
pool size the same way, swept over loads in flight per thread and workgroups per CU; the
best configuration is what reading those bytes in one launch reaches here.

per_workload: the same measurement of the other named workloads (1-bit MLP up and down,
rotated attention, output head, 1-bit affine), summarised: per-M us/call, t8/t1, stream
ceiling, roofline fraction.  For the output head a call is the verify GEMM with the argmax
of every row in one call (`verify_gemm_argmax`, the argmax fused into the GEMM's epilogue
on this shape), at M = 1 and the ragged M = 5..8.

For a routed-expert workload (synthetic.inputs.EXPERT_WORKLOADS) a call is one grouped
expert verify of M rows, each routed to topk of the E experts; the calls cycle through 64
seeded routings and the weight pool.  value counts the packed bytes of the distinct experts
each call routes to (each read once), and the line also gives the time of the same work as
one plain verify call per (row, slot), which reads an expert once per row routed to it.

Prints one JSON line: value = packed-weight bytes (codes + fp16 scales + fp16 biases)
moved per second over all timed calls (GB/s, 1e9), plus per-M microseconds per call,
t(M=8)/t(M=1), a roofline object for the dominant kernel and the CPU oracle baseline.

The affine formats' scales and biases are passed interleaved (each group's scale and bias
side by side, built once before timing with vg_pack_scale_bias, as a weight load would):
the same bytes in the library's faster layout.  --scale-bias separate times the two
separate arrays instead; config.scale_bias names the layout.

Options:
  --workload NAME    another named workload as the headline (see synthetic.inputs.WORKLOADS)
  --m LIST           only these row counts, e.g. "8" (for profiling one kernel; no
                     per-workload entries)
  --warmup W         untimed warm-up steps before the timed ones (default 200)
  --trials T         split the timed steps into T trials (default 7); per-M figures are
                     the median over the trials (and the min)
  --force-variant V  run every call on kernel variant V (see vg_variant_name) instead of the
                     per-shape dispatch, for A/B timing
  --scale-bias L     "interleaved" (default) or "separate" scales and biases
  --table            one JSON line per workload (instead of per_workload entries)
  --no-per-workload  the headline workload only
  --stream-sweep     print the streaming-read sweep at every workload's byte count, then exit
  --no-cpu           skip the CPU oracle baseline leg
  --copy-calibration run only a device-to-device copy of known size (for HBM counters)
  --host-overhead    run the native harness (vg_host_overhead, built by build()) that times
                     the C ABI's host cost per call beside a bare kernel launch
  --ingest-counters FETCH WRITE CFETCH CWRITE
                     write profiles/hbm_traffic.json from four rocprofv3 --pmc output
                     directories: FETCH_SIZE and WRITE_SIZE of a `--m 8 --no-cpu` run,
                     and of a `--copy-calibration` run (no GPU needed)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import re
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synthetic import EXPERT_WORKLOADS, WORKLOADS, draw_experts, draw_route, workload_case  # noqa: E402

HBM_PEAK_GBS = 8000.0
POOL_BYTES = 1 << 30
METRIC = "µs/call and packed-weight GB/s (% of HBM peak) at M=1..8; t(M=8)/t(M=1)"
KERNEL_SOURCES = ["few_row_quantized_verify_amd/csrc/vg_kernels.hip",
                  "few_row_quantized_verify_amd/csrc/vg_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_digest() -> str:
    """Hash of the kernel sources' code: comments and whitespace are dropped, so a comment
    edit does not mark the stored HBM counters as stale; any change to the code does."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)   # block comments
        src = re.sub(r"//[^\n]*", " ", src)                # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def packed_bytes(case) -> int:
    n = case.words.nbytes + case.scales.nbytes
    return n + (case.biases.nbytes if case.biases is not None else 0)


def x_bytes(case, M):
    return M * case.K * (4 if case.x_dtype == "f32" else 2)


def host_cpu() -> dict:
    """Host CPU model and logical core count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for l in f:
                if l.startswith("model name"):
                    model = l.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "os_cpu_count": os.cpu_count()}


def cpu_baseline(case) -> dict:
    """The oracle (fp64 numpy, untuned) on the host: the whole call (every output column)
    at M = 8, median of 3 runs with BLAS on every thread it uses, and one run on one
    thread."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count() or 1
    M = 8

    def run():
        t0 = time.perf_counter()
        oracle.verify(case.fmt, case.x(M), case.x_dtype, case.words, case.scales, case.biases)
        return time.perf_counter() - t0

    runs = [run() for _ in range(3)]
    dt = float(np.median(runs))
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            dt1 = run()
        one = {"value": packed_bytes(case) / dt1 / 1e9, "s_per_call": round(dt1, 3)}
    return {"value": packed_bytes(case) / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"whole call, M=8, {case.fmt} K={case.K} N={case.N}: median of 3 runs "
                      f"({', '.join(f'{r * 1e3:.0f}' for r in runs)} ms)",
            "us_per_call": round(dt * 1e6), "one_thread": one, "host": host_cpu()}


def cpu_baseline_experts(ec, routes) -> dict:
    """The oracle's routed-expert verify on the host, on a bounded sample of columns."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    M = routes[0].shape[0]
    ncols = min(ec.N, 128)
    cols = np.arange(ncols)
    per_expert = (ec.words[0].nbytes + ec.scales[0].nbytes +
                  (ec.biases[0].nbytes if ec.biases is not None else 0))
    t0 = time.perf_counter()
    reps = 0
    nbytes = 0.0
    while True:
        r = routes[reps % len(routes)]
        oracle.verify_experts(ec.fmt, ec.x(M), ec.x_dtype, r, ec.words, ec.scales, ec.biases, rows=cols)
        nbytes += len(np.unique(r)) * per_expert * ncols / ec.N
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 20:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"M={M}, first {ncols} of {ec.N} output columns of every routed slot, "
                      f"{reps} routings, {dt / reps * 1e3:.1f} ms/routing"}


def bench_experts(args, vg, torch, dev) -> dict:
    from synthetic.torch_io import case_tensors, f16_tensor, words_tensor
    name = args.workload
    fmt, K, N, E, topk, x_dtype = EXPERT_WORKLOADS[name]
    Ms = tuple(int(v) for v in args.m.split(",")) if args.m else (1, 2, 4, 8)
    ec = draw_experts(fmt, K, N, E, x_dtype, seed=0)
    per_expert = (ec.words[0].nbytes + ec.scales[0].nbytes +
                  (ec.biases[0].nbytes if ec.biases is not None else 0))
    ncopy = max(2, -(-POOL_BYTES // (per_expert * E)))
    w0, s0 = words_tensor(ec.words, dev), f16_tensor(ec.scales, dev)
    b0 = f16_tensor(ec.biases, dev) if ec.biases is not None else None
    s0, b0, layout = scale_bias_layout(args, vg, s0, b0)
    pool = [(w0.clone(), s0.clone(), None if b0 is None else b0.clone()) for _ in range(ncopy)]
    NR = 64
    routes = {M: [draw_route(M, topk, E, seed=1000 * M + r) for r in range(NR)] for M in Ms}
    rdev = {M: [torch.from_numpy(r).to(dev) for r in routes[M]] for M in Ms}
    uniq = {M: [len(np.unique(r)) for r in routes[M]] for M in Ms}
    x_all = {M: case_tensors(ec, M, dev)[0] for M in Ms}
    ys = {M: torch.empty((M, topk, N), dtype=torch.float32, device=dev) for M in Ms}

    def call(M, j):
        w, s, b = pool[j % ncopy]
        vg.verify_gemm_experts(fmt, x_all[M], rdev[M][j % NR], w, s, b, y=ys[M])

    for M in Ms:
        for j in range(args.warmup):
            call(M, j)
    torch.cuda.synchronize()
    # the same protocol as the plain workloads: a gate holds the GPU while the host enqueues
    # each (trial, M) block, so the event pair times the calls back to back on the device
    gate = Gate(vg, torch, dev, torch.cuda.current_stream().cuda_stream)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CLOCK_SETTLE_S:
        gate.hold(4)
        torch.cuda.synchronize()
    gate.calibrate(torch)
    t_wall = time.perf_counter()
    calls = {M: [] for M in Ms}

    def timed_call(M, j):
        call(M, j)
        calls[M].append(j)

    trial_us, _, _ = timed_blocks(torch, timed_call, Ms, trial_sizes(args.steps, args.trials), gate)
    wall = time.perf_counter() - t_wall
    us = {M: float(np.median(trial_us[M])) for M in Ms}
    # routed packed bytes per call at M, over the routings the timed calls used
    nbytes = {M: args.steps * float(np.mean([uniq[M][j % NR] for j in calls[M]])) * per_expert for M in Ms}

    # the same routed products as one plain verify call per (row, slot), on routing 0
    Mtop = max(Ms)
    rt0 = routes[Mtop][0]
    xs = [x_all[Mtop][m:m + 1].contiguous() for m in range(Mtop)]
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)

    def per_slot(j):
        w, s, b = pool[j % ncopy]
        for m in range(Mtop):
            for sl in range(topk):
                e = int(rt0[m, sl])
                vg.verify_gemm(fmt, xs[m], w[e], s[e], None if b is None else b[e], y=y1)

    for j in range(3):
        per_slot(j)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(5, args.steps // 10)
    e0.record()
    for j in range(reps):
        per_slot(j)
    e1.record()
    torch.cuda.synchronize()
    per_slot_us = e0.elapsed_time(e1) * 1e3 / reps

    total_s = sum(us.values()) * args.steps * 1e-6
    value = sum(nbytes.values()) / total_s / 1e9
    per_m = {str(M): {"us_per_call": round(us[M], 3),
                      "distinct_experts_mean": round(float(np.mean(uniq[M])), 2),
                      "gbs": round(nbytes[M] / args.steps / (us[M] * 1e-6) / 1e9, 1),
                      "pct_hbm_peak": round(100 * nbytes[M] / args.steps / (us[M] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
             for M in Ms}
    algo = nbytes[Mtop] / args.steps + x_bytes(ec, Mtop) + Mtop * topk * N * 4
    achieved = algo / (us[Mtop] * 1e-6) / 1e9
    kern = vg.variant_name(0 if Mtop <= 4 else 1)
    line = {
        "metric": "µs/call and routed packed-weight GB/s (% of HBM peak) of the grouped expert verify",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sum(us.values()) * 1e-3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if x_dtype != "f32" else "f32", "data": "synthetic",
        "config": {"workload": name, "format": fmt, "K": K, "N": N, "E": E, "topk": topk,
                   "x_dtype": x_dtype, "M": list(Ms), "packed_bytes_per_expert": per_expert,
                   "scale_bias": layout,
                   "routings": NR, "weight_pool_copies": ncopy},
        "per_m": per_m,
        "per_slot_calls_us": {"M": Mtop, "us": round(per_slot_us, 2),
                              "grouped_speedup": round(per_slot_us / us[Mtop], 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": kern, "M": Mtop, "algorithmic_bytes_per_launch": round(algo)},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_experts(ec, routes[Mtop])
    return line


def trial_sizes(steps: int, trials: int):
    """Split `steps` timed steps into `trials` trials of near-equal size (all of them run)."""
    trials = max(1, min(trials, steps))
    return [steps // trials + (1 if t < steps % trials else 0) for t in range(trials)]


class Gate:
    """Holds the GPU busy while the host enqueues a block of calls, so the block then runs
    back to back and its event pair times the device, not the host's submission rate (a
    call through the binding costs the host ~5 us, about what the smaller calls cost the
    GPU).  The gate is the library's streaming read over a 1 GiB buffer, enqueued before
    the block's start event; passes over it are added as the block grows."""

    HOST_US_PER_CALL = 8.0   # generous: measured 4-6 us on the boxes

    def __init__(self, vg, torch, dev, sh):
        self.vg, self.sh = vg, sh
        self.buf = torch.empty((POOL_BYTES // 4,), dtype=torch.int32, device=dev).fill_(1)
        self.sink = torch.zeros((vg.lib().vg_stream_read_blocks(),), dtype=torch.int32, device=dev)
        self.us_per_pass = 180.0   # ~1 GiB at ~6 TB/s; refined by calibrate()

    def calibrate(self, torch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.hold(1)
        e0.record()
        for _ in range(4):
            self.hold(1)
        e1.record()
        torch.cuda.synchronize()
        self.us_per_pass = e0.elapsed_time(e1) * 1e3 / 4

    def hold(self, passes):
        for _ in range(passes):
            self.vg.stream_read(self.buf, POOL_BYTES, self.sink, stream=self.sh, loads_in_flight=4, wgs_per_cu=8)

    def before(self, ncalls):
        self.hold(max(1, int(np.ceil(ncalls * self.HOST_US_PER_CALL / self.us_per_pass))))


def timed_blocks(torch, call, Ms, sizes, gate, j0=0):
    """Per (trial, M): a gate, then an event pair around that trial's block of calls on the
    kernels' stream.  Returns (per-M list of trial us/call, per-M host s, next call index)."""
    ev = [{M: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for M in Ms}
          for _ in sizes]
    host_s = {M: 0.0 for M in Ms}
    j = j0
    for t, n in enumerate(sizes):
        for M in Ms:
            gate.before(n)
            ev[t][M][0].record()
            h0 = time.perf_counter()
            for _ in range(n):
                call(M, j)
                j += 1
            host_s[M] += time.perf_counter() - h0
            ev[t][M][1].record()
    torch.cuda.synchronize()
    trial_us = {M: [ev[t][M][0].elapsed_time(ev[t][M][1]) * 1e3 / n for t, n in enumerate(sizes)] for M in Ms}
    return trial_us, host_s, j


STREAM_SWEEP = [(lif, wgs) for lif in (1, 2, 4, 8, 16) for wgs in (1, 2, 4, 8, 16)]


def stream_ceiling(vg, torch, dev, nbytes: int, ncopy: int, warmup: int, sizes, gate, sweep=STREAM_SWEEP,
                   full=False) -> dict:
    """The library's streaming-read kernel over a pool of `ncopy` distinct buffers of one
    call's packed bytes, timed like the calls (gate, then an event pair per block; median
    over the trials), in every configuration of `sweep` (16-byte loads in flight per
    thread, workgroups of 256 threads per CU): the best is what reading those bytes in one
    launch reaches here."""
    n16 = (nbytes + 15) // 16 * 16
    pool = [torch.empty((n16 // 4,), dtype=torch.int32, device=dev).fill_(1) for _ in range(ncopy)]
    sink = torch.zeros((vg.lib().vg_stream_read_blocks(),), dtype=torch.int32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    table = []
    for lif, wgs in sweep:
        def call(_, j):
            vg.stream_read(pool[j % ncopy], n16, sink, stream=sh, loads_in_flight=lif, wgs_per_cu=wgs)
        for j in range(max(3, warmup)):
            call(0, j)
        trial_us, _, _ = timed_blocks(torch, call, (0,), sizes, gate)
        us = float(np.median(trial_us[0]))
        table.append({"loads_in_flight": lif, "wgs_per_cu": wgs, "us_per_call": round(us, 3),
                      "pct_hbm_peak": round(100 * n16 / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)})
    del pool
    best = min(table, key=lambda r: r["us_per_call"])
    us = best["us_per_call"]
    out = {"us_per_call": us, "gbs": round(n16 / (us * 1e-6) / 1e9, 1),
           "pct_hbm_peak": round(100 * n16 / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1), "bytes": n16,
           "loads_in_flight": best["loads_in_flight"], "wgs_per_cu": best["wgs_per_cu"],
           "configs_swept": len(table)}
    if full:
        out["sweep"] = table
    return out


def load_traffic(kernel: str, digest: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    ent = t.get("kernels", {}).get(kernel)
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent.get("hbm_bytes_per_launch")


def _counter_rows(d: str):
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _mean_counter(d: str, counter: str, kernel_prefix: str):
    vals = [float(r["Counter_Value"]) for r in _counter_rows(d)
            if r["Counter_Name"] == counter and kernel_prefix in r["Kernel_Name"]]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def ingest_counters(fetch_dir, write_dir, cfetch_dir, cwrite_dir, workload, M) -> int:
    """HBM bytes per launch of the row count's kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a copy of known size."""
    # The verify kernel is the one GEMM variant the counter run dispatched (a `--m M` run
    # launches exactly one); the dispatch query itself needs a GPU, which this step does not.
    names = {r["Kernel_Name"].split("vg::", 1)[1].split("<", 1)[0] for r in _counter_rows(fetch_dir)
             if r["Kernel_Name"].startswith("void vg::vg_") and "stream_read" not in r["Kernel_Name"]}
    if len(names) != 1:
        print(f"expected one verify kernel in the counter output, found {sorted(names)}", file=sys.stderr)
        return 1
    kern = names.pop()
    cf, _ = _mean_counter(cfetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _ = _mean_counter(cwrite_dir, "WRITE_SIZE", "copyBuffer")
    if cf is None:
        cf, _ = _mean_counter(cfetch_dir, "FETCH_SIZE", "")
    if cw is None:
        cw, _ = _mean_counter(cwrite_dir, "WRITE_SIZE", "")
    nbytes = 256 << 20
    fetch_factor = nbytes / (cf * 1024.0)
    write_factor = nbytes / (cw * 1024.0)
    kf, nf = _mean_counter(fetch_dir, "FETCH_SIZE", "vg::" + kern + "<")
    kw, nw = _mean_counter(write_dir, "WRITE_SIZE", "vg::" + kern + "<")
    if kf is None or kw is None:
        print(f"no {kern} dispatches in the counter output", file=sys.stderr)
        return 1
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        t = {}
    t["note"] = ("HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per "
                 "dispatch), each scaled by the factor the same counter shows for a 256 MiB device "
                 "copy (bench.py --copy-calibration).  Keyed by variant/workload/M; valid only while "
                 "the kernel sources hash to source_digest.")
    t["calibration"] = {"copy_bytes": nbytes, "fetch_factor": fetch_factor, "write_factor": write_factor}
    fb = kf * 1024.0 * fetch_factor
    wb = kw * 1024.0 * write_factor
    t.setdefault("kernels", {})[f"{kern}/{workload}/M{M}"] = {
        "source_digest": kernel_source_digest(), "dispatches": [nf, nw],
        "fetch_bytes": round(fb), "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t["kernels"][f"{kern}/{workload}/M{M}"]))
    return 0


def scale_bias_layout(args, vg, s0, b0):
    """The affine formats' scales and biases in the layout the run asks for: interleaved
    (scale, bias) pairs, built once on the device like a weight load would (the library's
    faster layout; the same bytes), or the two separate arrays.  Returns (scales, biases,
    layout name)."""
    if b0 is None:
        return s0, None, "none"
    if getattr(args, "scale_bias", "interleaved") == "separate":
        return s0, b0, "separate"
    sb = vg.pack_scale_bias(s0, b0)
    return sb, None, "interleaved"


def raw_caller(vg, fmt, x, w, s, b, y, sh, idx=None):
    """The C ABI entry point of one verify call with its arguments marshalled once (the
    binding's checked wrapper has already run the same call once): the timed loop then
    costs the host the ctypes call only."""
    import ctypes
    from few_row_quantized_verify_amd import binding as B
    L = B.lib()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    M, K = x.shape
    N = w.shape[0]
    xt = B._xdtype(x)
    st = ctypes.c_void_p(sh)
    if idx is not None:
        args = (B.FORMATS[fmt], P(x), xt, M, K, P(w), P(s), P(b), N, P(y), P(idx),
                None, None, st)
        fn = L.verify_gemm_argmax
    elif fmt == "sign1":
        args, fn = (P(x), xt, M, K, P(w), P(s), N, P(y), st), L.verify_gemm_sign1
    elif fmt == "had2":
        args, fn = (P(x), xt, M, K, P(w), P(s), P(b), N, 128, P(y), st), L.verify_gemm_had2
    else:
        fn = L.verify_gemm_affine2 if fmt == "affine2" else L.verify_gemm_affine1
        args = (P(x), xt, M, K, P(w), P(s), P(b), N, P(y), st)

    def call():
        st_ = fn(*args)
        if st_ != 0:
            raise B.VerifyGemmError(st_, L.vg_last_error().decode())
    return call


def bench_workload(args, vg, torch, dev, name, Ms, gate, sh, full_sweep=False) -> dict:
    """One workload at each row count in Ms: warm-up, then the timed steps as trials of
    gated blocks of calls cycling through a >= 1 GiB pool of weight copies."""
    from synthetic.torch_io import case_tensors, f16_tensor, words_tensor
    fmt, K, N, x_dtype, _ = WORKLOADS[name]
    case = workload_case(name, seed=0)
    pb = packed_bytes(case)
    ncopy = max(2, -(-POOL_BYTES // pb))
    x_all = {M: case_tensors(case, M, dev)[0] for M in Ms}
    w0 = words_tensor(case.words, dev)
    s0 = f16_tensor(case.scales, dev)
    b0 = f16_tensor(case.biases, dev) if case.biases is not None else None
    s0, b0, layout = scale_bias_layout(args, vg, s0, b0)
    pool = [(w0.clone(), s0.clone(), None if b0 is None else b0.clone()) for _ in range(ncopy)]
    del w0, s0, b0
    ys = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    head = name.startswith("head_")
    idx = {M: torch.empty((M,), dtype=torch.int32, device=dev) for M in Ms}
    # one checked call per (M, copy) through the binding, then the raw C ABI calls
    calls = {}
    for M in Ms:
        for c, (w, s, b) in enumerate(pool):
            if head:
                vg.verify_gemm_argmax(fmt, x_all[M], w, s, b, y=ys[M], idx=idx[M], stream=sh)
            else:
                vg.verify_gemm(fmt, x_all[M], w, s, b, y=ys[M], stream=sh)
            calls[M, c] = raw_caller(vg, fmt, x_all[M], w, s, b, ys[M], sh, idx[M] if head else None)

    def call(M, j):
        calls[M, j % ncopy]()

    for M in Ms:
        for j in range(args.warmup):
            call(M, j)
    torch.cuda.synchronize()
    sizes = trial_sizes(args.steps, args.trials)
    t_wall = time.perf_counter()
    trial_us, host_s, _ = timed_blocks(torch, call, Ms, sizes, gate)
    wall = time.perf_counter() - t_wall
    us = {M: float(np.median(trial_us[M])) for M in Ms}
    total_s = sum(us.values()) * args.steps * 1e-6
    value = pb * len(Ms) * args.steps / total_s / 1e9
    per_m = {str(M): {"us_per_call": round(us[M], 3),
                      "us_per_call_min": round(min(trial_us[M]), 3),
                      "host_us_per_call": round(host_s[M] / args.steps * 1e6, 2),
                      "gbs": round(pb / (us[M] * 1e-6) / 1e9, 1),
                      "pct_hbm_peak": round(100 * pb / (us[M] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                      "variant": vg.variant_name(vg.plan_variant(fmt, x_dtype, M, N, K)),
                      "k_slices": vg.plan_ksplit(fmt, x_dtype, M, N, K)}
             for M in Ms}
    del pool, calls
    torch.cuda.empty_cache()
    ceiling = stream_ceiling(vg, torch, dev, pb, ncopy, min(args.warmup, 20), sizes, gate, full=full_sweep)
    Mtop = max(Ms)
    kern = per_m[str(Mtop)]["variant"]
    algo = pb + x_bytes(case, Mtop) + Mtop * N * 4
    achieved = algo / (us[Mtop] * 1e-6) / 1e9
    traffic = load_traffic(f"{kern}/{name}/M{Mtop}", kernel_source_digest())
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sum(us.values()) * 1e-3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if x_dtype != "f32" else "f32", "data": "synthetic",
        "config": {"workload": name, "format": fmt, "K": K, "N": N, "x_dtype": x_dtype,
                   "M": list(Ms), "packed_bytes_per_call": pb, "weight_pool_copies": ncopy,
                   "scale_bias": layout},
        "per_m": per_m,
        "t8_over_t1": round(us[Mtop] / us[min(Ms)], 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kern, "M": Mtop,
                     "algorithmic_bytes_per_launch": algo},
        "stream_ceiling": ceiling,
        "trials": len(sizes),
        "wall_s_timed": round(wall, 4),
    }
    return line


def summary(line) -> dict:
    """The compact per-workload entry of the headline line."""
    pm = line["per_m"]
    return {"config": {k: line["config"][k] for k in ("format", "K", "N", "x_dtype", "packed_bytes_per_call",
                                                        "scale_bias")},
            "us_per_call": {m: v["us_per_call"] for m, v in pm.items()},
            "pct_hbm_peak": {m: v["pct_hbm_peak"] for m, v in pm.items()},
            "variant": {m: v["variant"] for m, v in pm.items()},
            "gbs_all_m": line["value"], "t8_over_t1": line["t8_over_t1"],
            "stream_ceiling_us": line["stream_ceiling"]["us_per_call"],
            "stream_ceiling_pct": line["stream_ceiling"]["pct_hbm_peak"],
            "roofline_frac": line["roofline"]["frac"]}


# The workloads measured beside the headline on every default run (the headline is the
# 2-bit MLP up-projection; see the module docstring).
PER_WORKLOAD = ["mlp_up_sign1_k5120_n17408", "mlp_down_sign1_k17408_n5120", "attn_had2_k5120_n6144",
                "head_affine2_k5120_n151936", "mlp_up_affine1_k5120_n17408"]
CLOCK_SETTLE_S = 0.05


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--trials", type=int, default=7)
    ap.add_argument("--workload", default="mlp_up_affine2_k5120_n17408")
    ap.add_argument("--table", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-per-workload", action="store_true")
    ap.add_argument("--stream-sweep", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--m", default=None)
    ap.add_argument("--force-variant", default=None)
    ap.add_argument("--scale-bias", choices=("interleaved", "separate"), default="interleaved",
                    help="layout of the affine formats' scales and biases (same bytes)")
    ap.add_argument("--host-overhead", action="store_true",
                    help="run the native harness timing the C ABI's host cost per call, then exit")
    ap.add_argument("--ingest-counters", nargs=4, metavar="DIR", default=None)
    args = ap.parse_args()
    if args.ingest_counters:
        return ingest_counters(*args.ingest_counters, args.workload,
                               int(args.m) if args.m else 8)
    if args.host_overhead:
        # a child process of its own (this one has not touched the GPU)
        exe = os.path.join(ROOT, "few_row_quantized_verify_amd", "vg_host_overhead")
        if not os.path.exists(exe):
            print(f"{exe} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`",
                  file=sys.stderr)
            return 2
        return subprocess.run([exe]).returncode
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify GEMM runs on one device here; "
              "run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import few_row_quantized_verify_amd as vg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.force_variant:
        names_v = [vg.variant_name(i) for i in range(vg.variant_count())]
        if args.force_variant not in names_v:
            print(f"unknown variant {args.force_variant!r}; one of {names_v}", file=sys.stderr)
            return 2
        vg.force_variant(names_v.index(args.force_variant))

    if args.copy_calibration:
        nbytes = 256 << 20
        a = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}))
        return 0

    if args.workload in EXPERT_WORKLOADS:
        print(json.dumps(bench_experts(args, vg, torch, dev)))
        return 0

    sh = torch.cuda.current_stream().cuda_stream   # the raw handle: no lookup per call
    gate = Gate(vg, torch, dev, sh)
    # clock settle: the GPU runs back-to-back work for a while before anything is timed
    # (measured on MI355X: the first ~10 ms of calls run up to 10% slower)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CLOCK_SETTLE_S:
        gate.hold(4)
        torch.cuda.synchronize()
    gate.calibrate(torch)

    if args.stream_sweep:
        # the streaming-read ceiling swept at the byte counts of the workloads
        sizes = trial_sizes(args.steps, args.trials)
        for name in WORKLOADS:
            if name.startswith("tiny_"):
                continue
            pb = packed_bytes(workload_case(name, seed=0, N=1)) // 1 * WORKLOADS[name][2]
            ncopy = max(2, -(-POOL_BYTES // pb))
            c = stream_ceiling(vg, torch, dev, pb, ncopy, min(args.warmup, 20), sizes, gate, full=True)
            print(json.dumps({"stream_sweep": name, "bytes": pb, **c}), flush=True)
        return 0

    names = list(WORKLOADS) if args.table else [args.workload]
    Ms_arg = tuple(int(v) for v in args.m.split(",")) if args.m else None
    lines = []
    headline = None
    for name in names:
        Ms = Ms_arg or WORKLOADS[name][4]
        line = bench_workload(args, vg, torch, dev, name, Ms, gate, sh)
        if name == args.workload:
            headline = line
        lines.append(line)
    if headline is None:
        headline = lines[0]
    if not args.no_per_workload and not args.table and Ms_arg is None:
        per = {}
        for name in PER_WORKLOAD:
            if name == args.workload:
                continue
            per[name] = summary(bench_workload(args, vg, torch, dev, name, WORKLOADS[name][4], gate, sh))
        headline["per_workload"] = per
    headline["clock_settle_s"] = CLOCK_SETTLE_S
    headline["gate"] = {"kind": "streaming read of 1 GiB before each block of calls", "us_per_pass":
                        round(gate.us_per_pass, 1)}
    if not args.no_cpu:
        headline["cpu_baseline"] = cpu_baseline(workload_case(headline["config"]["workload"], seed=0))
    if args.table:
        for l in lines:
            if l is not headline:
                print(json.dumps(l))
    print(json.dumps(headline))
    return 0


if __name__ == "__main__":
    sys.exit(main())
