#!/usr/bin/env python3
"""Cold-cache benchmark of the five decode projections on one MI355X.

Metric: cold-cache microseconds per load (the sum of its five layers' times)
plus achieved HBM bandwidth against the roofline, over the six loads m = 1 to
256. Loads, layers and the cold-cache rule follow guide ch. 1 "The problem,
the judge and the speed of light" (§1.2 the loads, §1.3 a load's time is the
sum of its five shapes, §1.4 a buffer larger than the cache is read before
every timed call, and calls are replayed from a graph).

One step runs every load once: 6 loads x 5 layers = 30 cold calls. Each call
is a flush (a read of FLUSH_BYTES, more than the 32 MB of L2 plus the 256 MB
Infinity Cache; the flush study below picks its kind) followed by the
projection kernel, launched with a pair of HIP events that the runtime stamps
at the start and end of that kernel's own execution (hipExtLaunchKernel), on
the stream the kernel runs on. The headline `value` is the median over the
timed steps of the step's sum of 30 kernel durations, i.e. the sum of the six
per-load times. Inputs are seeded synthetic tensors resident in device memory
before timing starts; weights are prepared (repacked) before timing.

Also reported, each from the same process:
* per load and layer: median kernel time, achieved TB/s of the bytes the
  kernel reads, the BF16-equivalent rate, and the fraction of a measured
  cold read floor over the same bytes (the hand-written read kernel, best
  of plain and non-temporal loads over several grid shapes, the GEMV's own
  among them);
* graph replay (the pages' method, guide ch. 10 "Measure, experiment, and
  try your own changes" §10.1): each load captured as ONE graph of its five
  kernels between two GPU wall-clock stamps, replayed cold, paired and
  alternated with a graph of five read-floor kernels over the same bytes;
  reported raw (host events around the replay) and as the stamped span;
* the flush study: the 67 MB read floor and the pooler decode-1 kernel
  with no flush, a 1 GiB non-temporal flush, a 1 GiB plain flush and a
  2 GiB plain flush;
* the awkward token counts (guide ch. 1 §1.2), timed like the loads;
* the roofline of the dominant kernel and the CPU oracle's own times.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --pmc-pass     (short run used under rocprofv3 --pmc)
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GIB = 1 << 30
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_TFLOPS = 2500.0   # MI355X dense BF16 matrix peak
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_loads.json")
LOAD_ORDER = ("decode-1", "decode-16", "decode-32", "verify-1", "verify-16", "verify-32")
# Pages' H200 per-load times, best reported (guide ch. 1 §1.8 table): context
# from other hardware, not a target.
H200_BEST_US = {"decode-1": 38.25, "decode-16": 54.03, "decode-32": 63.77, "verify-1": 39.98,
                "verify-16": 77.91, "verify-32": 94.80}

# The flush used before every timed call: (mode, bytes). Chosen from the flush
# study (the kind after which the kernels read coldest); 0 = non-temporal,
# 1 = plain loads.
FLUSH_MODE = 1
FLUSH_BYTES = GIB
FLUSH_BUF_BYTES = 2 * GIB
STUDY_CONDITIONS = (("none", None, 0), ("nt-1GiB", 0, GIB), ("plain-1GiB", 1, GIB), ("plain-2GiB", 1, 2 * GIB))

# Read-floor configurations tried for every byte count (grid, waves, unroll);
# each in both load modes, plus the projection kernel's own grid and waves.
FLOOR_CONFIGS = ((256, 8, 4), (256, 16, 2), (512, 8, 4), (1024, 8, 4), (2048, 4, 4), (4096, 4, 2))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Every kernel source (kernels, weight layouts, the 12-bit encoder, the
# measurement kernels that scale the counters); the dispatch choice itself is
# also checked by kernel name.
def kernel_sources():
    d = os.path.join(ROOT, "gemv_decode_projections_amd", "csrc")
    return sorted(n for n in os.listdir(d) if n.endswith((".h", ".hip")))


def source_hash():
    """Hash of the kernel sources with comments and blank space removed (a
    comment edit does not change a kernel)."""
    import re

    h = hashlib.sha256()
    for name in kernel_sources():
        with open(os.path.join(ROOT, "gemv_decode_projections_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stored_bytes(layer, m, cfg, zcr):
    """Bytes the chosen kernel must read and write for one call: the
    algorithmic bytes, except that a kernel on the 12-bit weights reads 3/4 of
    the BF16 weight bytes plus the correction table (N rows x zcr slots x 8
    bytes)."""
    from gemv_decode_projections_amd import roofline as rf
    from gemv_decode_projections_amd.layers import DIMS

    b = rf.bytes_of(layer, m)
    if cfg.kind == 0 and cfg.flags & 4:
        n = DIMS[layer][0]
        b = b - rf.weight_bytes(layer, m) // 4 + n * zcr * 8
    return b


def mfma_flops(layer, m):
    """Matrix-core FLOPs the kernels issue: 2 m N K, three times that for the
    router (its FP32 weights enter as three exact BF16 parts)."""
    from gemv_decode_projections_amd import roofline as rf

    return rf.flops_of(layer, m) * (3 if layer == "router" else 1)


class Bench:
    def __init__(self, seed=0):
        import numpy as np
        import torch

        from gemv_decode_projections_amd import binding as B
        from workload import LAYERS, LOADS, make_weight, make_x

        self.np, self.torch, self.B = np, torch, B
        self.LAYERS, self.LOADS, self.make_x = LAYERS, LOADS, make_x
        self.dev = torch.device("cuda", 0)
        self.weights = {}
        for layer in LAYERS:
            w = make_weight(layer, seed)
            self.weights[layer] = w
            wd = (torch.from_numpy(w) if w.dtype == np.float32
                  else torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)).to(self.dev)
            B.proj_prepare(layer, wd)
            del wd
        self.flush_buf = torch.ones(FLUSH_BUF_BYTES, dtype=torch.uint8, device=self.dev)
        self.sink = torch.zeros(1 << 16, dtype=torch.int32, device=self.dev)
        self.floor_buf = torch.ones(80 << 20, dtype=torch.uint8, device=self.dev)
        self.stamps = torch.zeros(64, dtype=torch.int64, device=self.dev)
        self.timer = B.KernelTimer()
        self.inputs = {}
        self.floor_cfg = {}
        torch.cuda.synchronize()

    def flush(self, mode=FLUSH_MODE, nbytes=FLUSH_BYTES, stream=None):
        if mode is not None:
            self.B.proj_bench_flush(self.flush_buf, self.sink, stream, mode=mode, nbytes=nbytes)

    def xin(self, layer, m, variant=0):
        key = (layer, m, variant)
        if key not in self.inputs:
            xs = self.make_x(layer, m, seed=1000 + variant, outliers=bool(variant % 2))
            x = self.torch.from_numpy(xs.bits.view(self.np.int16)).view(self.torch.bfloat16).to(self.dev)
            self.inputs[key] = (x, self.B.new_out(layer, m, device=self.dev))
        return self.inputs[key]

    def kernel_us(self, layer, m, variant=0, flush=(FLUSH_MODE, FLUSH_BYTES)):
        """One cold call: flush, then the projection kernel timed by its own events."""
        x, out = self.xin(layer, m, variant)
        self.flush(*flush)
        self.B.proj_run_timed(layer, x, m, out, self.timer)
        return self.timer.elapsed_us()

    def floor_once(self, nbytes, cfg, flush=(FLUSH_MODE, FLUSH_BYTES)):
        grid, waves, unroll, mode = cfg
        self.flush(*flush)
        self.B.proj_bench_read_floor(self.floor_buf, nbytes, self.sink, grid, waves, unroll,
                                     events=self.timer, mode=mode)
        return self.timer.elapsed_us()

    def floor_us(self, nbytes, reps, extra=()):
        """Cold pure-read time of `nbytes` (rounded up to 16): the best median
        over the read kernel's configurations (both load modes); the best
        configuration is kept for the graph leg."""
        nbytes = (nbytes + 15) // 16 * 16
        best = None
        cfgs = [c + (mode,) for c in tuple(FLOOR_CONFIGS) + tuple(extra) for mode in (0, 1)]
        for cfg in cfgs:
            med = statistics.median(self.floor_once(nbytes, cfg) for _ in range(reps))
            if best is None or med < best[0]:
                best = (med, cfg)
        self.floor_cfg[nbytes] = best[1]
        return best[0], best[1]

    # -------------------------------------------------------------- graphs

    def capture(self, fn):
        """A HIP graph of fn(stream), captured on a side stream."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn(s)
        torch.cuda.synchronize()
        return g, s

    def load_graph(self, name):
        """Stamp 0, the load's five projection kernels back to back, stamp 1."""
        m = self.LOADS[name]
        xs = {l: self.xin(l, m, 0) for l in self.LAYERS}

        def body(s):
            self.B.proj_bench_stamp(self.stamps, 0, s)
            for l in self.LAYERS:
                x, out = xs[l]
                self.B.proj_run(l, x, m, out, s)
            self.B.proj_bench_stamp(self.stamps, 1, s)
        return self.capture(body)

    def floor_graph(self, byte_counts):
        """Stamp 2, one read-floor kernel per layer over its bytes (best configuration), stamp 3."""
        def body(s):
            self.B.proj_bench_stamp(self.stamps, 2, s)
            for nb in byte_counts:
                nb = (nb + 15) // 16 * 16
                grid, waves, unroll, mode = self.floor_cfg[nb]
                self.B.proj_bench_read_floor(self.floor_buf, nb, self.sink, grid, waves, unroll, stream=s, mode=mode)
            self.B.proj_bench_stamp(self.stamps, 3, s)
        return self.capture(body)

    def replay(self, g, s):
        """Cold replay: flush on the replay stream, then the graph between two
        host-recorded events. Returns (event us, stamped span us)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            self.flush(stream=s)
            e0.record(s)
            g.replay()
            e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3


def cpu_baseline(layers, loads, reps_small=3):
    """The CPU oracle on every load (the same shapes, its own full outputs) on
    the host's cores: the median of `reps_small` runs per layer for m <= 32,
    one run above; decode-1 also on one thread."""
    import oracle
    from workload import make_weight, make_x

    ws = {l: make_weight(l, 0) for l in layers}
    per_load = {}
    t_all = time.perf_counter()
    for name in LOAD_ORDER:
        m = loads[name]
        lay = {}
        for l in layers:
            xs = make_x(l, m, seed=1000)
            ts = []
            for _ in range(reps_small if m <= 32 else 1):
                t0 = time.perf_counter()
                oracle.reference(l, xs.bits, ws[l])
                ts.append((time.perf_counter() - t0) * 1e6)
            lay[l] = round(statistics.median(ts), 1)
        per_load[name] = {"m": m, "us": round(sum(lay.values()), 1), "layers_us": lay}
    nt = oracle.threads()
    one = []
    try:
        oracle.set_threads(1)
        xs1 = {l: make_x(l, 1, seed=1000) for l in layers}
        for _ in range(3):
            t0 = time.perf_counter()
            for l in layers:
                oracle.reference(l, xs1[l].bits, ws[l])
            one.append((time.perf_counter() - t0) * 1e6)
    finally:
        oracle.set_threads(nt)
    total = sum(v["us"] for v in per_load.values())
    return {
        "value": round(total, 1),
        "unit": "us per six-load set (sum of the six loads' five layers)",
        "cores": nt,
        "kind": "oracle",
        "sample": "the whole workload: each load's five layers at its m, every output, FP64 oracle; median of %d "
                  "runs per layer for m <= 32, one run above; %.1f s on %s" % (
                      reps_small, time.perf_counter() - t_all, _cpu_name()),
        "loads": per_load,
        "decode1_single_thread_us": round(statistics.median(one), 1),
    }


def _cpu_name():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip() + " x%d" % os.cpu_count()
    except OSError:
        pass
    return "unknown CPU"


def traffic_for(layer, m, kernel=None):
    """HBM bytes per launch of (layer, m) from the committed counter summary.

    None when there is no summary, the kernel sources changed since the
    counters were read (the summary stores a hash of the sources), or the
    dispatch now picks a different kernel for (layer, m).
    """
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    k = d.get("launches", {}).get("%s@%d" % (layer, m))
    if not k or (kernel is not None and k.get("kernel") != kernel):
        return None
    return int(round(k["fetch_bytes"] + k["write_bytes"]))


def kernel_name(cfg, f32w):
    """Template name of the kernel a configuration launches (as profilers print it)."""
    f = "true" if f32w else "false"
    if cfg.kind == 0:   # last arguments: 12-bit weights, preloaded activation rows (0: none)
        xp = 4 if cfg.flags & 32 else 8 if cfg.flags & 64 else 0
        return "skinny_kernel<%d, %d, %d, %d, %s, %s, %d>" % (cfg.nt, cfg.rb, cfg.waves, cfg.spw, f,
                                                              "true" if cfg.flags & 4 else "false", xp)
    if cfg.kind == 1:   # <rows per wave, token blocks, waves, k-steps per super-step, depth, fp32>
        return "tiled_kernel<%d, %d, %d, %d, %d, %s>" % (cfg.rb // cfg.waves, cfg.nt, cfg.waves,
                                                         min(4, cfg.spw // 2), cfg.spw, f)
    if cfg.kind == 3:   # <rows per wave, token blocks, depth, k-steps per super-step, fp32, stream, waves, LDS DMA>
        return "wide_kernel<%d, %d, %d, %d, %s, %s, %d, %s>" % (cfg.rb // cfg.waves, cfg.nt, cfg.spw,
                                                               4 if cfg.spw >= 16 else 2, f,
                                                               "true" if cfg.flags & 8 else "false", cfg.waves,
                                                               "true" if cfg.flags & 128 else "false")
    return "rowdot_kernel<%d, %d, %d, %s>" % (cfg.nt, cfg.rb, cfg.spw, f)


PROJ_KERNELS = ("skinny_kernel", "tiled_kernel", "rowdot_kernel", "wide_kernel")


def _is_proj_kernel(name):
    return any(k in name for k in PROJ_KERNELS)


def _short(name):
    return name.split("(")[0].replace("void gdp::", "").replace("gdp::(anonymous namespace)::", "")


def _read_csv(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


# ------------------------------------------------------- launch sequence

def call_sequence(steps, warmup, study_reps, awkward_reps, graph_reps):
    """(tag, layer, m) of every projection kernel bench.py launches, in launch
    order: the event-timed steps (tag = load name, warm-up steps tagged
    'warmup:<load>'), the flush study's pooler calls ('study:<condition>'), the
    awkward token counts ('m=<m>') and the graph replays ('graph:<load>')."""
    from workload import AWKWARD_M, LAYERS, LOADS

    seq = []
    for s in range(warmup + steps):
        for name in LOAD_ORDER:
            for l in LAYERS:
                seq.append(("warmup:" + name if s < warmup else name, l, LOADS[name]))
    for _ in range(study_reps):
        for cond, _, _ in STUDY_CONDITIONS:
            seq.append(("study:" + cond, "pooler", 1))
    for m in AWKWARD_M:
        for l in LAYERS:
            seq += [("m=%d" % m, l, m)] * awkward_reps
    for name in LOAD_ORDER:
        for _ in range(graph_reps):
            seq += [("graph:" + name, l, LOADS[name]) for l in LAYERS]
    return seq


def summarize_loads_trace(trace_csv, steps, warmup, study_reps, awkward_reps, graph_reps):
    """Kernel durations of every (tag, layer) from a rocprofv3 kernel trace of
    bench.py, matching the trace's projection launches one to one with
    call_sequence() (the run's counts must be the ones given here)."""
    from gemv_decode_projections_amd import roofline as rf

    allrows = _read_csv(trace_csv)
    # proj_prepare's warm-up launches come before the bench's first flush.
    flushes = [int(r["Start_Timestamp"]) for r in allrows if "flush_kernel" in r["Kernel_Name"]]
    t_first = min(flushes) if flushes else -1
    rows = sorted((r for r in allrows if _is_proj_kernel(r["Kernel_Name"]) and int(r["Start_Timestamp"]) > t_first),
                  key=lambda r: int(r["Start_Timestamp"]))
    seq = call_sequence(steps, warmup, study_reps, awkward_reps, graph_reps)
    if len(rows) != len(seq):
        raise SystemExit("trace has %d projection launches, the bench sequence %d: counts differ"
                         % (len(rows), len(seq)))
    per = {}
    for (tag, layer, m), r in zip(seq, rows):
        e = per.setdefault((tag, layer), {"kernel": _short(r["Kernel_Name"]), "m": m,
                                          "grid": int(r["Grid_Size_X"]), "d": []})
        if e["kernel"] != _short(r["Kernel_Name"]):
            raise SystemExit("(%s, %s): launches of different kernels %s / %s" % (tag, layer, e["kernel"],
                                                                                 _short(r["Kernel_Name"])))
        e["d"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = {}
    for (tag, layer), e in per.items():
        if tag.startswith("warmup"):
            continue
        d = out.setdefault(tag, {"m": e["m"], "layers": {}})
        med = statistics.median(e["d"])
        d["layers"][layer] = {"kernel": e["kernel"], "grid": e["grid"], "n": len(e["d"]),
                              "median_us": round(med, 3), "mean_us": round(statistics.mean(e["d"]), 3),
                              "TBps": round(rf.bytes_of(layer, e["m"]) / med / 1e6, 3)}
    for d in out.values():
        d["sum_median_us"] = round(sum(v["median_us"] for v in d["layers"].values()), 2)
    return out


def summarize_graph_trace(trace_csv, graph_reps):
    """In-graph kernel durations and the gaps between kernels, from the graph
    replays of a rocprofv3 kernel trace of bench.py: each replayed graph is
    a stamp kernel, five kernels, a stamp kernel. Per load (the load graphs
    come in LOAD_ORDER, graph_reps each) and for the floor graphs: medians of
    each kernel's duration, of the six gaps (stamp -> first kernel, the four
    between kernels, last kernel -> stamp) and of the span from the first
    kernel's start to the last one's end."""
    rows = sorted(_read_csv(trace_csv), key=lambda r: int(r["Start_Timestamp"]))
    stamps = [i for i, r in enumerate(rows) if "stamp_kernel" in r["Kernel_Name"]]
    if len(stamps) % 2:
        raise SystemExit("odd number of stamp kernels in the trace")
    loads, floors = [], []
    for a, b in zip(stamps[::2], stamps[1::2]):
        inner = rows[a + 1:b]
        if len(inner) != 5:
            raise SystemExit("a stamped graph holds %d kernels, not 5" % len(inner))
        ts = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in [rows[a]] + inner + [rows[b]]]
        rec = {"kernels": [_short(r["Kernel_Name"]) for r in inner],
               "dur": [(e - s) / 1e3 for s, e in ts[1:-1]],
               "gaps": [(ts[i + 1][0] - ts[i][1]) / 1e3 for i in range(6)],
               "span": (ts[5][1] - ts[1][0]) / 1e3}
        (loads if all(_is_proj_kernel(k) for k in rec["kernels"]) else floors).append(rec)
    if len(loads) != graph_reps * len(LOAD_ORDER) or len(floors) != len(loads):
        raise SystemExit("found %d load and %d floor graph replays, expected %d each"
                         % (len(loads), len(floors), graph_reps * len(LOAD_ORDER)))

    def agg(recs):
        return {"kernels": recs[0]["kernels"],
                "kernel_median_us": [round(statistics.median(r["dur"][i] for r in recs), 3) for i in range(5)],
                "gap_median_us": [round(statistics.median(r["gaps"][i] for r in recs), 3) for i in range(6)],
                "span_median_us": round(statistics.median(r["span"] for r in recs), 3),
                "n": len(recs)}
    out = {}
    for j, name in enumerate(LOAD_ORDER):
        out[name] = {"graph": agg(loads[j * graph_reps:(j + 1) * graph_reps]),
                     "floor_graph": agg(floors[j * graph_reps:(j + 1) * graph_reps])}
    return out


# ------------------------------------------------------- profile pages

CMD_VARS = "`$REPO`: the repository root on the MI355X host; `$OUT`: the directory the runs write to"
BENCH_CMD = "python3 $REPO/bench.py > $OUT/bench.json"
PROFILE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_bench "
               "-o bench -- python3 -u $REPO/bench.py --no-cpu-baseline > $OUT/bench_prof.json")
PMC_CMDS = (
    "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o fetch "
    "-- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_fetch.log 2>&1",
    "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o write "
    "-- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_write.log 2>&1",
    "cd /tmp && rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv -d $OUT/pmc_mfma "
    "-o mfma -- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_mfma.log 2>&1",
    "cd /tmp && rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE --output-format csv -d $OUT/pmc_lds "
    "-o lds -- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_lds.log 2>&1",
)
PMC_HASH_TAG = "pmc pass kernel sources:"

# With --out-root DIR, paths under DIR are shown as $OUT/... on the profile pages.
OUT_ROOT = None


def shown(path):
    if OUT_ROOT and os.path.abspath(path).startswith(os.path.abspath(OUT_ROOT) + os.sep):
        return "$OUT/" + os.path.relpath(path, OUT_ROOT)
    return path


def md_loads_trace(lt, trace_csv, counts, bench_line=None):
    """profiles/loads_kernels_trace.md: every (load, layer) kernel's trace
    durations, and the dominant kernel's event average from the same run."""
    steps, warmup, study, awk, graph = counts
    L = ["# Every load's kernels: rocprofv3 kernel trace of bench.py (MI355X, 1 GPU)", "",
         "Commands (%s):" % CMD_VARS, "", "```", PROFILE_CMD,
         "python bench.py --summarize-loads-trace %s --steps %d --warmup %d --study-reps %d --awkward-reps %d "
         "--graph-reps %d --bench-json %s --md > profiles/loads_kernels_trace.md"
         % (shown(trace_csv), steps, warmup, study, awk, graph, shown("$OUT/bench.json")), "```", "",
         "Every launch is cold (flush before it). Launches are matched in order with the bench's launch sequence",
         "(`bench.call_sequence`); the load rows cover the %d timed steps; loads named m=<m> are the awkward token"
         % steps,
         "counts, graph:<load> the in-graph launches of the graph leg, study:<condition> the flush study's pooler",
         "decode-1 calls. TB/s uses the algorithmic bytes (guide ch. 1 §1.7 formulas).", ""]
    if bench_line:
        roof = bench_line["roofline"]
        tr = lt.get(roof["load"], {}).get("layers", {}).get(roof["layer"])
        L += ["The same bench command run without the profiler in the same session (`%s`) reports the dominant kernel"
              % BENCH_CMD,
              "(%s, %s, `%s`) at an event average of %.3f us over its timed steps; the trace's mean for the same"
              % (roof["load"], roof["layer"], roof["kernel"], roof["avg_us"]),
              "launches is %s us. (Under the profiler the events themselves read longer per call, because tracing"
              % ("%.3f" % tr["mean_us"] if tr else "n/a"),
              "adds work around each dispatch; the trace stamps do not include it.)", ""]
    L += ["| load | m | layer | kernel | grid (threads) | n | median us | mean us | TB/s |",
          "|---|---|---|---|---|---|---|---|---|"]
    for ld, d in lt.items():
        for l, e in d["layers"].items():
            L.append("| %s | %d | %s | `%s` | %d | %d | %.3f | %.3f | %.3f |" % (
                ld, d["m"], l, e["kernel"], e["grid"], e["n"], e["median_us"], e["mean_us"], e["TBps"]))
    L += ["", "Per-load sums of the trace medians (us): "
          + ", ".join("%s %.2f" % (ld, d["sum_median_us"]) for ld, d in lt.items() if ld in LOAD_ORDER) + ".", ""]
    return "\n".join(L)


def md_graph_trace(gt, trace_csv, graph_reps):
    """profiles/graph_replay_trace.md from summarize_graph_trace()."""
    L = ["# Loads replayed as graphs: in-graph kernel durations and gaps (rocprofv3 kernel trace, MI355X)", "",
         "Same profiled run as `loads_kernels_trace.md` (command there); table from",
         "`python bench.py --summarize-graph-trace %s --graph-reps %d --md`." % (shown(trace_csv), graph_reps), "",
         "Each load is one graph: a stamp kernel, the load's five projection kernels back to back (qkv_gate, o,",
         "pooler, unpooler, router), a stamp kernel; its floor graph holds five read-floor kernels over the same",
         "bytes. Every replay follows a flush; the two graphs alternate, order swapped each repetition.",
         "Gaps: stamp -> first kernel, the four between kernels, last kernel -> stamp (start of the next minus end",
         "of the previous, us). Span: first kernel start to last kernel end. Medians of %d replays." % graph_reps, "",
         "| load | graph | kernel durations (us) | sum | gaps (us) | span us |", "|---|---|---|---|---|---|"]
    for name, d in gt.items():
        for which in ("graph", "floor_graph"):
            e = d[which]
            L.append("| %s | %s | %s | %.2f | %s | %.2f |" % (
                name, "projections" if which == "graph" else "read floor",
                " / ".join("%.2f" % v for v in e["kernel_median_us"]), sum(e["kernel_median_us"]),
                " / ".join("%.2f" % v for v in e["gap_median_us"]), e["span_median_us"]))
    inner = [g for d in gt.values() for g in d["graph"]["gap_median_us"][1:5]]
    L += ["", "Between kernels of one graph the median gap is %.2f us (range %.2f-%.2f over the loads): the"
          % (statistics.median(inner), min(inner), max(inner)),
          "per-kernel fixed cost a load pays four times on top of its kernels' own durations.", ""]
    return "\n".join(L)


def md_pmc(pm, csvs, logs):
    """profiles/pmc_loads.md from summarize_pmc()'s result."""
    args = "%s --pmc-logs %s" % (" ".join(shown(c) for c in csvs), " ".join(shown(g) for g in logs))
    L = ["# HBM traffic, MFMA use and LDS bank conflicts per launch, every load: rocprofv3 --pmc (MI355X, 1 GPU)", "",
         "Commands (%s; one counter set per run):" % CMD_VARS, "", "```"] + list(PMC_CMDS) + [
         "python bench.py --summarize-pmc %s > profiles/pmc_loads.json" % args,
         "python bench.py --summarize-pmc %s --md > profiles/pmc_loads.md" % args, "```", "",
         "The pass runs every load's five kernels cold (flush before each), %d times, then copies 64 MiB three"
         % PMC_REPS,
         "times. FETCH_SIZE reads %.4f x fewer KiB than that copy moves and WRITE_SIZE reads it with scale %.4f; both"
         % (pm["fetch_scale"], pm["write_scale"]),
         "are multiplied by their scale. Medians of the %d passes. MFMA util = MFMA-busy cycles over all SIMD cycles"
         % PMC_REPS,
         "of the dispatch (rocprofv3's MfmaUtil); MOPS = SQ_INSTS_VALU_MFMA_MOPS_BF16 as counted. LDS conflict % =",
         "SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE: the share of the LDS's indexed-access cycles lost to bank",
         "conflicts (0 when every access is conflict-free; 50 when each one takes twice its cycles). Kernels whose last",
         "template argument is `true` read 12-bit lossless weights (3/4 of the BF16 bytes plus a correction table).",
         "FETCH_SIZE counts what the L2 caches fetch from memory (HBM or the Infinity Cache behind them); each XCD's",
         "L2 fetches its own copy of data that workgroups on several XCDs read (x at large m).", "",
         "| load | layer | kernel | fetched by L2 (FETCH_SIZE, bytes) | written (WRITE_SIZE, bytes) | algorithmic bytes "
         "| traffic / algorithmic | MFMA util % | MFMA MOPS (bf16) | LDS conflict % |",
         "|---|---|---|---|---|---|---|---|---|---|"]
    for key, e in pm["launches"].items():
        L.append("| %s | %s | `%s` | %d | %d | %d | %.3f | %s | %s | %s |" % (
            e["load"], key.split("@")[0], e["kernel"], e["fetch_bytes"], e["write_bytes"], e["algorithmic_bytes"],
            (e["fetch_bytes"] + e["write_bytes"]) / e["algorithmic_bytes"], e.get("mfma_util_pct", "-"),
            e.get("mfma_mops_bf16", "-"), e.get("lds_conflict_pct", "-")))
    L += ["", "Source hash of the kernels these counters belong to, as printed by the passes themselves: `%s` "
          "(bench.py reports `traffic` = null once the sources differ)." % pm["source_hash"], ""]
    return "\n".join(L)


def md_flush_study(line, bench_json):
    """profiles/flush_study.md from a bench line's flush_study."""
    fs = line["flush_study"]
    L = ["# Which flush empties the caches: 67 MB read floor and pooler decode-1 (MI355X, 1 GPU)", "",
         "Command (%s):" % CMD_VARS, "", "```", BENCH_CMD,
         "python bench.py --flush-study-md %s > profiles/flush_study.md" % shown(bench_json), "```", "",
         "Each condition is applied before every call (none: the call follows the previous call of the same",
         "kernel, its data still cached); conditions interleaved, %d repetitions, medians of the kernels' own"
         % fs["reps"],
         "event durations. A flush that leaves the weights in the 256 MB Infinity Cache reads faster than one",
         "that evicts them. The bench times every call after the `%s` flush." % fs["chosen"], "",
         "| condition | 67.1 MB read floor (us) | pooler decode-1 kernel (us) |", "|---|---|---|"]
    for c, v in fs["conditions"].items():
        L.append("| %s | %.2f | %.2f |" % (c, v["floor_us"], v["pooler_decode1_us"]))
    L.append("")
    return "\n".join(L)


PMC_REPS = 3


def pmc_sequence():
    """(load, layer) of the projection launches of `bench.py --pmc-pass`, in order."""
    from workload import LAYERS

    return [(name, l) for _ in range(PMC_REPS) for name in LOAD_ORDER for l in LAYERS]


def pass_source_hash(logs):
    """The kernel-source hash the counter passes printed (every log must name
    the same one): the counters belong to the sources that ran on the GPU, not
    to whatever the tree holds when the summary is rendered."""
    seen = set()
    for path in logs:
        with open(path) as f:
            tags = [l.split(PMC_HASH_TAG, 1)[1].strip() for l in f if PMC_HASH_TAG in l]
        if len(tags) != 1:
            raise SystemExit("%s: expected one '%s' line, found %d" % (path, PMC_HASH_TAG, len(tags)))
        seen.add(tags[0])
    if len(seen) != 1:
        raise SystemExit("the counter passes ran different kernel sources: %s" % sorted(seen))
    return seen.pop()


def summarize_pmc(fetch_csv, write_csv, mfma_csv=None, lds_csv=None, copy_bytes=64 << 20, sources=None):
    """HBM bytes (and MFMA use) per launch of every (load, layer) from the counter
    passes of `bench.py --pmc-pass`.

    FETCH_SIZE and WRITE_SIZE are scaled by what they read on the copy kernel
    of known size in the same pass (copy_bytes read and copy_bytes written).
    The optional third pass holds MfmaUtil (MFMA-busy cycles over all SIMD
    cycles of the dispatch, percent) and SQ_INSTS_VALU_MFMA_MOPS_BF16; the
    optional fourth SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE (their ratio per
    launch, percent; "-" where a launch makes no indexed LDS access).
    `sources`: the kernel-source hash the passes ran (pass_source_hash).
    """
    from gemv_decode_projections_amd import roofline as rf
    from workload import LOADS

    seq = pmc_sequence()
    res = {"source_hash": sources, "copy_bytes": copy_bytes, "launches": {}}

    def launches(path, cname):
        rows = sorted((r for r in _read_csv(path) if r["Counter_Name"] == cname),
                      key=lambda r: int(r["Dispatch_Id"]))
        # proj_prepare's warm-up launches come before the pass's first flush.
        first = min((int(r["Dispatch_Id"]) for r in rows if "flush_kernel" in r["Kernel_Name"]), default=-1)
        sk = [r for r in rows if _is_proj_kernel(r["Kernel_Name"]) and int(r["Dispatch_Id"]) > first]
        if len(sk) != len(seq):
            raise SystemExit("%s: %d projection launches, the pass makes %d" % (path, len(sk), len(seq)))
        return rows, sk

    def entry(name, layer, r=None):
        m = LOADS[name]
        key = "%s@%d" % (layer, m)
        if key not in res["launches"]:
            res["launches"][key] = {"load": name, "kernel": _short(r["Kernel_Name"]),
                                    "grid": int(r["Grid_Size"]), "algorithmic_bytes": rf.bytes_of(layer, m)}
        return res["launches"][key]

    for path, cname, key in ((fetch_csv, "FETCH_SIZE", "fetch"), (write_csv, "WRITE_SIZE", "write")):
        rows, sk = launches(path, cname)
        cp = [float(r["Counter_Value"]) for r in rows if "copy_kernel" in r["Kernel_Name"]]
        scale = copy_bytes / (statistics.median(cp) * 1024.0)
        res[key + "_scale"] = round(scale, 4)
        vals = {}
        for (name, layer), r in zip(seq, sk):
            vals.setdefault((name, layer), []).append(float(r["Counter_Value"]) * 1024.0 * scale)
            entry(name, layer, r)
        for (name, layer), v in vals.items():
            entry(name, layer)[key + "_bytes"] = round(statistics.median(v))
    if mfma_csv:
        for cname, key in (("MfmaUtil", "mfma_util_pct"), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "mfma_mops_bf16")):
            _, sk = launches(mfma_csv, cname)
            vals = {}
            for (name, layer), r in zip(seq, sk):
                vals.setdefault((name, layer), []).append(float(r["Counter_Value"]))
            for (name, layer), v in vals.items():
                entry(name, layer)[key] = round(statistics.median(v), 2)
    if lds_csv:
        got = {}
        for cname in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"):
            _, sk = launches(lds_csv, cname)
            got[cname] = [float(r["Counter_Value"]) for r in sk]
        vals = {}
        for i, (name, layer) in enumerate(seq):
            act = got["SQ_LDS_IDX_ACTIVE"][i]
            if act > 0:
                vals.setdefault((name, layer), []).append(100.0 * got["SQ_LDS_BANK_CONFLICT"][i] / act)
        for (name, layer), v in vals.items():
            entry(name, layer)["lds_conflict_pct"] = round(statistics.median(v), 1)
    return res


def pmc_pass():
    """Short deterministic pass for rocprofv3 --pmc: every load's kernels, cold,
    PMC_REPS times, then a copy of known size (the counters' scale)."""
    import torch

    from gemv_decode_projections_amd import binding as B

    print(PMC_HASH_TAG, source_hash(), flush=True)
    b = Bench()
    n = 64 << 20
    src = torch.ones(n, dtype=torch.uint8, device=b.dev)
    dst = torch.empty(n, dtype=torch.uint8, device=b.dev)
    for name, layer in pmc_sequence():
        b.kernel_us(layer, b.LOADS[name])
    torch.cuda.synchronize()
    for _ in range(3):
        b.flush()
        B.proj_bench_copy(src, dst, n)
    torch.cuda.synchronize()
    log("pmc pass done: every load's kernels x%d, copy of %d bytes x3" % (PMC_REPS, n))


# ------------------------------------------------------------------ main

def run(args):
    import torch

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    from gemv_decode_projections_amd import roofline as rf
    from gemv_decode_projections_amd import binding as B

    b = Bench()
    layers = b.LAYERS
    plans = {(name, l): B.proj_plan(l, b.LOADS[name]) for name in LOAD_ORDER for l in layers}
    zcr = {l: B.proj_compressed(l) for l in layers}

    # Warm-up steps (untimed), then the timed steps: every load once per step.
    for _ in range(args.warmup):
        for name in LOAD_ORDER:
            for l in layers:
                b.kernel_us(l, b.LOADS[name])
    per = {(name, l): [] for name in LOAD_ORDER for l in layers}
    step_us = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        tot = 0.0
        for name in LOAD_ORDER:
            for l in layers:
                t = b.kernel_us(l, b.LOADS[name], variant=s % 2)
                per[(name, l)].append(t)
                tot += t
        step_us.append(tot)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = statistics.median(step_us)
    log("timed %d steps: %.2f us per step (median)" % (args.steps, value))

    # Read floors over each shape's bytes (what its kernel reads), best of the
    # read kernel's configurations with the projection kernel's own grid among them.
    loads = {}
    for name in LOAD_ORDER:
        m = b.LOADS[name]
        lay, fl, frac, tb, eff, cfgs = {}, {}, {}, {}, {}, {}
        for l in layers:
            cfg = plans[(name, l)]
            t = statistics.median(per[(name, l)])
            sb = stored_bytes(l, m, cfg, zcr[l])
            f, fc = b.floor_us(sb, args.floor_reps, extra=((cfg.grid, min(cfg.block // 64, 16), 4),))
            lay[l], fl[l] = round(t, 3), round(f, 3)
            frac[l] = round(f / t, 3)
            tb[l] = round(sb / t / 1e6, 3)
            eff[l] = round(rf.bytes_of(l, m) / t / 1e6, 3)
            cfgs[l] = {"kernel": kernel_name(cfg, l == "router"), "grid": cfg.grid, "block": cfg.block,
                       "stored_bytes": sb, "floor_config": list(fc)}
        tot = sum(lay.values())
        loads[name] = {
            "m": m, "us": round(tot, 2), "layers_us": lay, "read_floor_us": fl, "frac_of_read_floor": frac,
            "read_floor_sum_us": round(sum(fl.values()), 2),
            "TBps_read": tb, "TBps_bf16_equivalent": eff,
            "TFLOPs": round(sum(rf.flops_of(l, m) for l in layers) / tot / 1e6, 2),
            "nominal_floor_us": round(rf.load_floor_us(m, router_peak=rf.MI355X_FP32_FLOPS), 2),
            "h200_best_us_context": H200_BEST_US[name],
            "kernels": cfgs,
        }
        log("%-10s m=%-4d %8.2f us  %s" % (name, m, tot, lay))

    # Flush study: 67 MB read floor and pooler decode-1 under each condition,
    # conditions interleaved.
    nb67 = rf.bytes_of("pooler", 1) // 16 * 16
    _, fcfg = b.floor_us(nb67, args.floor_reps)
    study = {c: {"floor": [], "pooler": []} for c, _, _ in STUDY_CONDITIONS}
    for _ in range(args.study_reps):
        for c, mode, nbytes in STUDY_CONDITIONS:
            study[c]["floor"].append(b.floor_once(nb67, fcfg, flush=(mode, nbytes)))
            study[c]["pooler"].append(b.kernel_us("pooler", 1, flush=(mode, nbytes)))
    flush_study = {"reps": args.study_reps, "floor_config": list(fcfg), "floor_bytes": nb67,
                   "chosen": next(c for c, mo, nb in STUDY_CONDITIONS if mo == FLUSH_MODE and nb == FLUSH_BYTES),
                   "conditions": {c: {"floor_us": round(statistics.median(v["floor"]), 3),
                                      "pooler_decode1_us": round(statistics.median(v["pooler"]), 3)}
                                  for c, v in study.items()}}
    log("flush study: %s" % flush_study["conditions"])

    # The awkward token counts of the correctness sweep, timed the same way.
    from workload import AWKWARD_M
    awkward = {}
    for m in AWKWARD_M:
        lay = {l: round(statistics.median(b.kernel_us(l, m) for _ in range(args.awkward_reps)), 2) for l in layers}
        awkward[str(m)] = {"us": round(sum(lay.values()), 2), "layers_us": lay}
    log("awkward m: %s" % {m: v["us"] for m, v in awkward.items()})

    # Graph leg: each load as one graph, paired and alternated with its floor graph.
    khz = B.proj_bench_wallclock_khz()
    graph = {"wallclock_khz": khz, "reps": args.graph_reps, "loads": {}}
    for name in LOAD_ORDER:
        m = b.LOADS[name]
        gl, sl = b.load_graph(name)
        gf, sf = b.floor_graph([stored_bytes(l, m, plans[(name, l)], zcr[l]) for l in layers])
        raw = {"load": [], "floor": []}
        span = {"load": [], "floor": []}
        for r in range(args.graph_reps):
            order = (("load", gl, sl), ("floor", gf, sf)) if r % 2 == 0 else (("floor", gf, sf), ("load", gl, sl))
            for which, g, s in order:
                raw[which].append(b.replay(g, s))
                st = b.stamps[:4].cpu().tolist()
                i0 = 0 if which == "load" else 2
                span[which].append((st[i0 + 1] - st[i0]) * 1e3 / khz)
        gd = {"stamped_span_us": round(statistics.median(span["load"]), 2),
              "replay_event_us": round(statistics.median(raw["load"]), 2),
              "floor_stamped_span_us": round(statistics.median(span["floor"]), 2),
              "floor_replay_event_us": round(statistics.median(raw["floor"]), 2)}
        gd["frac_of_floor_graph"] = round(gd["floor_stamped_span_us"] / gd["stamped_span_us"], 3)
        graph["loads"][name] = gd
        del gl, gf
    graph["sum_stamped_span_us"] = round(sum(v["stamped_span_us"] for v in graph["loads"].values()), 2)
    log("graph replay (stamped spans): %s" % {k: v["stamped_span_us"] for k, v in graph["loads"].items()})

    # Roofline of the dominant kernel: the (load, layer) with the longest median time.
    dom = max(per, key=lambda k: statistics.median(per[k]))
    dname, dlayer = dom
    dm = b.LOADS[dname]
    dcfg = plans[dom]
    d_avg = statistics.mean(per[dom])
    d_stored = stored_bytes(dlayer, dm, dcfg, zcr[dlayer])
    t_hbm = d_stored / 8e12
    t_mfma = mfma_flops(dlayer, dm) / 2.5e15
    kname = kernel_name(dcfg, dlayer == "router")
    achieved = d_stored / d_avg / 1e3
    roof = {
        "bound": "hbm" if t_hbm >= t_mfma else "mfma",
        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic_for(dlayer, dm, kname),
        "load": dname, "layer": dlayer, "m": dm, "kernel": kname, "avg_us": round(d_avg, 3),
        "bytes_per_launch": d_stored,
        "bytes_rule": "W N_eff x K (x 3/4 plus the correction table on 12-bit weights) + x m x K x 2 + out m x N_eff "
                      "x o, each once",
        "effective_GBps": round(rf.bytes_of(dlayer, dm) / d_avg / 1e3, 1),
        "mfma_TFLOPs": round(mfma_flops(dlayer, dm) / d_avg / 1e6, 1),
        "mfma_frac": round(mfma_flops(dlayer, dm) / d_avg / 1e6 / MFMA_BF16_TFLOPS, 4),
        "nominal_hbm_us": round(t_hbm * 1e6, 3), "nominal_mfma_us": round(t_mfma * 1e6, 3),
        "measured_read_floor_us": loads[dname]["read_floor_us"][dlayer],
    }

    cpu = None if args.no_cpu_baseline else cpu_baseline(layers, b.LOADS)

    h200_sum = sum(H200_BEST_US.values())
    result = {
        "metric": "cold-cache us per load (sum of 5 layers) + achieved HBM TB/s vs roofline, m=1-256",
        "value": round(value, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(value / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(value / h200_sum, 4),
        "baseline": {"value": round(h200_sum, 2), "unit": "us",
                     "what": "sum of the pages' best per-load times on H200 SXM over the same six loads "
                             "(guide ch. 1 §1.8; context from other hardware, not a target)"},
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "six loads, each the sum of five cold projections x @ W^T: decode-1 (m=1), decode-16 (m=16), "
                        "decode-32 (m=32), verify-1 (m=8), verify-16 (m=128), verify-32 (m=256); layers qkv_gate "
                        "2304x8192, o 8192x1024, pooler 4096x8192, unpooler 8192x4096 (rows 0-1023 at m<=8), "
                        "router 256x8192 fp32 weights and output; x bf16",
            "loads": {name: b.LOADS[name] for name in LOAD_ORDER},
            "timing": "kernel duration from hipExtLaunchKernel start/stop events; %s flush of %d MiB before each call"
                      % ("plain" if FLUSH_MODE else "non-temporal", FLUSH_BYTES >> 20),
        },
        "loads": loads,
        "awkward_m": awkward,
        "graph_replay": graph,
        "flush_study": flush_study,
        "timed_wall_s": round(wall, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--floor-reps", type=int, default=5, help="cold reads per floor configuration and shape")
    ap.add_argument("--study-reps", type=int, default=15, help="repetitions of the flush study")
    ap.add_argument("--graph-reps", type=int, default=21, help="cold replays per load graph (and floor graph)")
    ap.add_argument("--awkward-reps", type=int, default=7, help="cold calls per layer at each awkward token count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--summarize-loads-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-(load, layer) kernel durations from a rocprofv3 trace of bench.py")
    ap.add_argument("--summarize-graph-trace", metavar="KERNEL_TRACE_CSV",
                    help="print in-graph kernel durations and gaps from a rocprofv3 trace of bench.py")
    ap.add_argument("--flush-study-md", metavar="BENCH_JSON", help="print profiles/flush_study.md from a bench line")
    ap.add_argument("--md", action="store_true", help="with --summarize-*: print the profiles/ Markdown page")
    ap.add_argument("--bench-json", metavar="PATH", help="with --summarize-loads-trace --md: the line of the same run")
    ap.add_argument("--out-root", metavar="DIR", help="with --md: show paths under DIR as $OUT/...")
    ap.add_argument("--pmc-logs", nargs="+", metavar="LOG",
                    help="with --summarize-pmc: the passes' output (names the kernel sources they ran)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print HBM bytes per launch from the --pmc passes: FETCH_SIZE csv, WRITE_SIZE csv "
                         "and optionally the MfmaUtil csv and the LDS bank-conflict csv")
    args = ap.parse_args()
    global OUT_ROOT
    OUT_ROOT = args.out_root

    def last_line(path):
        with open(path) as f:
            return json.loads(f.read().strip().splitlines()[-1])

    if args.summarize_loads_trace:
        counts = (args.steps, args.warmup, args.study_reps, args.awkward_reps, args.graph_reps)
        lt = summarize_loads_trace(args.summarize_loads_trace, *counts)
        if args.md:
            line = last_line(args.bench_json) if args.bench_json else None
            print(md_loads_trace(lt, args.summarize_loads_trace, counts, line))
        else:
            print(json.dumps(lt, indent=1))
        return
    if args.summarize_graph_trace:
        gt = summarize_graph_trace(args.summarize_graph_trace, args.graph_reps)
        print(md_graph_trace(gt, args.summarize_graph_trace, args.graph_reps) if args.md else json.dumps(gt, indent=1))
        return
    if args.flush_study_md:
        print(md_flush_study(last_line(args.flush_study_md), args.flush_study_md))
        return
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3, 4):
            raise SystemExit("--summarize-pmc takes FETCH_CSV WRITE_CSV [MFMA_CSV [LDS_CSV]]")
        if not args.pmc_logs:
            raise SystemExit("--summarize-pmc needs --pmc-logs (the passes' output, which names their sources)")
        pm = summarize_pmc(*args.summarize_pmc, sources=pass_source_hash(args.pmc_logs))
        print(md_pmc(pm, args.summarize_pmc, args.pmc_logs) if args.md else json.dumps(pm, indent=1))
        return

    if args.gpus != 1:
        sys.exit("bench.py measures one GPU only: this library has no multi-GPU path "
                 "(the projections are already one GPU's shard); run with --gpus 1")
    if args.pmc_pass:
        pmc_pass()
        return
    run(args)


if __name__ == "__main__":
    main()
