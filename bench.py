#!/usr/bin/env python3
"""Cold-cache benchmark of the five decode projections on one MI355X.

Metric: cold-cache microseconds per load (the sum of its five layers' times)
plus achieved HBM bandwidth against the roofline. Loads, layers and the
cold-cache protocol follow guide ch. 1 "The problem, the judge and the speed
of light" (§1.2 loads, §1.3 a load's time is the sum of its five shapes, §1.4
a buffer larger than the cache is read before every timed call).

Protocol per timed call: a 1 GiB read-only flush kernel (more than the 32 MB
of L2 plus the 256 MB Infinity Cache), then the projection kernel launched
with a pair of HIP events that the runtime stamps at the start and end of
that kernel's execution (hipExtLaunchKernel), then a sync. The flush is
outside the measured interval.

A step is one decode-1 load (m = 1, all five layers, cold before each layer):
the headline `value` is the median over the timed steps of the per-step sum.
The other loads (decode-16/32, verify-1/16/32) are measured the same way and
reported under `loads` (with achieved TB/s and TFLOP/s). `graph_replay`
repeats every load with the pages' method (each call captured in a HIP graph,
replayed cold, minus an empty-kernel graph) for context. Inputs are seeded synthetic tensors already resident
in device memory; weights are prepared (repacked) before timing.

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

FLUSH_BYTES = 1 << 30
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_TFLOPS = 2500.0   # MI355X dense BF16 matrix peak
# Pages' H200 per-load time for decode 1, best reported (guide ch. 1 §1.8 table).
H200_DECODE1_US = 38.25
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_loads.json")
LOAD_ORDER = ("decode-1", "decode-16", "decode-32", "verify-1", "verify-16", "verify-32")


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
        self.flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=self.dev)
        self.sink = torch.zeros(1 << 16, dtype=torch.int32, device=self.dev)
        self.floor_buf = torch.ones(80 << 20, dtype=torch.uint8, device=self.dev)
        self.timer = B.KernelTimer()
        self.inputs = {}
        torch.cuda.synchronize()

    def xin(self, layer, m, variant=0):
        key = (layer, m, variant)
        if key not in self.inputs:
            xs = self.make_x(layer, m, seed=1000 + variant, outliers=bool(variant % 2))
            x = self.torch.from_numpy(xs.bits.view(self.np.int16)).view(self.torch.bfloat16).to(self.dev)
            self.inputs[key] = (x, self.B.new_out(layer, m, device=self.dev))
        return self.inputs[key]

    def kernel_us(self, layer, m, variant=0):
        """One cold call: flush, then the projection kernel timed by its own events."""
        x, out = self.xin(layer, m, variant)
        self.B.proj_bench_flush(self.flush, self.sink)
        self.B.proj_run_timed(layer, x, m, out, self.timer)
        return self.timer.elapsed_us()

    def graph_us(self, layer, m, reps):
        """Median cold time of one captured proj_run replayed as a HIP graph.

        Events are recorded on the replay stream around graph.replay(), so the
        time includes the graph launch overhead; graph_net_us subtracts the
        same measurement of a graph holding one empty kernel.
        """
        torch, B = self.torch, self.B
        x, out = self.xin(layer, m, 0) if layer is not None else (None, None)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            if layer is None:
                B.proj_bench_empty(s)
            else:
                B.proj_run(layer, x, m, out, s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            if layer is None:
                B.proj_bench_empty(s)
            else:
                B.proj_run(layer, x, m, out, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(reps):
            with torch.cuda.stream(s):
                B.proj_bench_flush(self.flush, self.sink, s)
                e0.record(s)
                g.replay()
                e1.record(s)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(ts)

    def floor_us(self, nbytes, reps):
        """Cold pure-read kernel over the same byte count (16-byte multiple)."""
        nbytes = (nbytes + 15) // 16 * 16
        best = None
        for grid, waves, unroll in ((2048, 4, 4), (1024, 8, 4), (4096, 4, 2), (2048, 8, 2)):
            ts = []
            for _ in range(reps):
                self.B.proj_bench_flush(self.flush, self.sink)
                self.B.proj_bench_read_floor(self.floor_buf, nbytes, self.sink, grid, waves, unroll,
                                             events=self.timer)
                ts.append(self.timer.elapsed_us())
            med = statistics.median(ts)
            if best is None or med < best:
                best = med
        return best


def cpu_baseline(seconds):
    """The CPU oracle on the decode-1 load (all five layers, m = 1) on the host cores."""
    import numpy as np

    import oracle
    from workload import LAYERS, make_weight, make_x

    ws = {l: make_weight(l, 0) for l in LAYERS}
    xs = {l: make_x(l, 1, seed=1000) for l in LAYERS}
    times = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        for l in LAYERS:
            oracle.reference(l, xs[l].bits, ws[l])
        times.append((time.perf_counter() - t0) * 1e6)
    return {
        "value": round(statistics.median(times), 1),
        "unit": "us per decode-1 load",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": "%d full decode-1 loads (5 layers, m=1, all %d outputs each) in %.1f s on %s"
                  % (len(times), sum(oracle.out_cols(l, 1) for l in LAYERS), sum(times) / 1e6, _cpu_name()),
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
    if cfg.kind == 0:   # last argument: 12-bit weights
        return "skinny_kernel<%d, %d, %d, %d, %s, %s>" % (cfg.nt, cfg.rb, cfg.waves, cfg.spw, f,
                                                          "true" if cfg.flags & 4 else "false")
    if cfg.kind == 1:   # <rows per wave, token blocks, waves, k-steps per super-step, depth, fp32>
        return "tiled_kernel<%d, %d, %d, %d, %d, %s>" % (cfg.rb // cfg.waves, cfg.nt, cfg.waves,
                                                         min(4, cfg.spw // 2), cfg.spw, f)
    if cfg.kind == 3:   # <rows per wave, token blocks, depth, k-steps per super-step, fp32, stream>
        return "wide_kernel<%d, %d, %d, %d, %s, %s>" % (cfg.rb // 4, cfg.nt, cfg.spw, 4 if cfg.spw >= 16 else 2, f,
                                                       "true" if cfg.flags & 8 else "false")
    return "rowdot_kernel<%d, %d, %d, %s>" % (cfg.nt, cfg.rb, cfg.spw, f)


PROJ_KERNELS = ("skinny_kernel", "tiled_kernel", "rowdot_kernel", "wide_kernel")


def _is_proj_kernel(name):
    return any(k in name for k in PROJ_KERNELS)


def _read_csv(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(trace_csv, steps, warmup):
    """Per-layer kernel durations of the timed decode-1 steps, from a rocprofv3 kernel trace of bench.py."""
    from workload import LAYERS

    rows = sorted(_read_csv(trace_csv), key=lambda r: int(r["Start_Timestamp"]))
    sk = [r for r in rows if _is_proj_kernel(r["Kernel_Name"])]
    timed = sk[warmup * len(LAYERS):(warmup + steps) * len(LAYERS)]
    out = {}
    for i, layer in enumerate(LAYERS):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed[i::len(LAYERS)]]
        out[layer] = {"kernel": timed[i]["Kernel_Name"].split("(")[0].replace("void gdp::", ""),
                      "grid": int(timed[i]["Grid_Size_X"]), "n": len(d),
                      "mean_us": round(statistics.mean(d), 3), "median_us": round(statistics.median(d), 3)}
    return out


def call_sequence(steps, warmup, load_reps, graph_reps, awkward_reps, graph=True):
    """(load, layer) of every projection kernel bench.py launches, in launch order
    (the awkward token counts appear as loads named "m=<m>")."""
    from workload import AWKWARD_M, LAYERS

    seq = [("decode-1", l) for _ in range(warmup + steps) for l in LAYERS]
    for name in LOAD_ORDER[1:]:
        for l in LAYERS:
            seq += [(name, l)] * load_reps
    for m in AWKWARD_M:
        for l in LAYERS:
            seq += [("m=%d" % m, l)] * awkward_reps
    if graph:
        for name in LOAD_ORDER:
            for l in LAYERS:
                seq += [(name, l)] * (1 + graph_reps)   # one direct warm-up run, then the replays
    return seq


def summarize_loads_trace(trace_csv, steps, warmup, load_reps, graph_reps, awkward_reps):
    """Kernel durations of every (load, layer) from a rocprofv3 kernel trace of bench.py.

    The projection launches in the trace (in start order) are matched one to
    one with the launch sequence of the bench run; the run's step, warm-up and
    repetition counts must be the ones given here.
    """
    from gemv_decode_projections_amd import roofline as rf
    from workload import LOADS

    rows = sorted((r for r in _read_csv(trace_csv) if _is_proj_kernel(r["Kernel_Name"])),
                  key=lambda r: int(r["Start_Timestamp"]))
    seq = call_sequence(steps, warmup, load_reps, graph_reps, awkward_reps)
    if len(rows) != len(seq):
        raise SystemExit("trace has %d projection launches, the bench sequence %d: counts differ"
                         % (len(rows), len(seq)))
    per = {}
    for (name, layer), r in zip(seq, rows):
        e = per.setdefault((name, layer), {"kernel": r["Kernel_Name"].split("(")[0].replace("void gdp::", ""),
                                           "grid": int(r["Grid_Size_X"]), "d": []})
        e["d"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    from workload import AWKWARD_M

    out = {}
    for name in list(LOAD_ORDER) + ["m=%d" % m for m in AWKWARD_M]:
        m = LOADS[name] if name in LOADS else int(name[2:])
        lay = {}
        for (n2, layer), e in per.items():
            if n2 != name:
                continue
            med = statistics.median(e["d"])
            lay[layer] = {"kernel": e["kernel"], "grid": e["grid"], "n": len(e["d"]), "median_us": round(med, 3),
                          "TBps": round(rf.bytes_of(layer, m) / med / 1e6, 3),
                          "TFLOPs": round(rf.flops_of(layer, m) / med / 1e6, 1)}
        out[name] = {"m": m, "sum_median_us": round(sum(v["median_us"] for v in lay.values()), 2), "layers": lay}
    return out


CMD_VARS = "`$REPO`: the repository root on the MI355X host; `$OUT`: the directory the runs write to"
BENCH_CMD = "python3 $REPO/bench.py > $OUT/bench.json"
PROFILE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_bench "
               "-o bench -- python3 -u $REPO/bench.py --no-cpu-baseline")
PMC_CMDS = (
    "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o fetch "
    "-- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_fetch.log 2>&1",
    "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o write "
    "-- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_write.log 2>&1",
    "cd /tmp && rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv -d $OUT/pmc_mfma "
    "-o mfma -- python3 $REPO/bench.py --pmc-pass > $OUT/pmc_mfma.log 2>&1",
)
PMC_HASH_TAG = "pmc pass kernel sources:"


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


# With --out-root DIR, paths under DIR are shown as $OUT/... on the profile pages.
OUT_ROOT = None


def shown(path):
    if OUT_ROOT and os.path.abspath(path).startswith(os.path.abspath(OUT_ROOT) + os.sep):
        return "$OUT/" + os.path.relpath(path, OUT_ROOT)
    return path


def md_decode1_trace(tr, trace_csv, bench_line=None, steps=50, warmup=5, bench_json=None):
    """profiles/decode1_kernels_trace.md from summarize_trace()'s result (and,
    when given, the JSON line of the same bench run without the profiler)."""
    from gemv_decode_projections_amd import roofline as rf

    L = ["# Decode-1 kernels: rocprofv3 kernel trace of bench.py (MI355X, 1 GPU)", "",
         "Commands (%s):" % CMD_VARS, "", "```", BENCH_CMD, PROFILE_CMD,
         "python bench.py --summarize-trace %s --md --bench-json %s > profiles/decode1_kernels_trace.md"
         % (shown(trace_csv), shown(bench_json or "$OUT/bench.json")),
         "python bench.py --summarize-loads-trace %s --md > profiles/loads_kernels_trace.md" % shown(trace_csv), "```", "",
         "Timed region: the %d decode-1 steps after %d warmup steps (each call preceded by a 1 GiB flush)." % (steps, warmup),
         "Kernel durations are the trace's start/end stamps."]
    if bench_line:
        ev, roof = bench_line["decode1_layers_us"], bench_line["roofline"]
        dom = roof["layer"]
        L += ["The same bench command run without the profiler (and with the CPU baseline), in the same session,",
              "reported (hipExtLaunchKernel events, median): " + ", ".join("%s %.2f" % (l, v) for l, v in ev.items())
              + " us; dominant kernel %s (`%s`) event average %.3f us vs trace mean %.3f us." % (
                  dom, roof["kernel"], roof["avg_us"], tr[dom]["mean_us"]),
              "(Under the profiler the events themselves read longer per call, because tracing adds work around each",
              "dispatch; the trace stamps do not include it.)"]
        if roof.get("weights") == "12-bit lossless":
            L += ["", "Kernels whose last template argument is `true` read 12-bit lossless weights; the dominant one (%s)"
                  % dom, "reads %d bytes (%.3f of the BF16 bytes). Algorithmic bytes and GB/s below count the BF16 operation."
                  % (roof["stored_bytes"], roof["stored_bytes"] / roof["algorithmic_bytes"])]
    L += ["", "| layer | kernel | grid (threads) | n | mean us | median us | algorithmic bytes | GB/s (mean) |",
          "|---|---|---|---|---|---|---|---|"]
    for l, e in tr.items():
        by = rf.bytes_of(l, 1)
        L.append("| %s | `%s` | %d | %d | %.3f | %.3f | %d | %d |" % (l, e["kernel"], e["grid"], e["n"], e["mean_us"],
                                                                     e["median_us"], by, round(by / e["mean_us"] / 1e3)))
    L += ["", "Sum of the five trace medians: %.2f us per decode-1 load." % sum(e["median_us"] for e in tr.values()), ""]
    return "\n".join(L)


def md_loads_trace(lt, trace_csv):
    """profiles/loads_kernels_trace.md from summarize_loads_trace()'s result."""
    L = ["# Every load's kernels: rocprofv3 kernel trace of bench.py (MI355X, 1 GPU)", "",
         "Same trace as `decode1_kernels_trace.md` (command there); table from",
         "`python bench.py --summarize-loads-trace %s --md`." % shown(trace_csv),
         "Every launch is cold (1 GiB flush before it). Launches are matched in order with the bench's launch",
         "sequence (`bench.call_sequence`); n counts the event-timed calls, the graph warm-up run and the replays;",
         "loads named m=<m> are the awkward token counts. TB/s and TFLOP/s use algorithmic bytes and FLOPs",
         "(guide ch. 1 §1.7 formulas).", "",
         "| load | m | layer | kernel | grid (threads) | n | median us | TB/s | TFLOP/s |", "|---|---|---|---|---|---|---|---|---|"]
    for ld, d in lt.items():
        for l, e in d["layers"].items():
            L.append("| %s | %d | %s | `%s` | %d | %d | %.3f | %.3f | %.1f |" % (
                ld, d["m"], l, e["kernel"], e["grid"], e["n"], e["median_us"], e["TBps"], e["TFLOPs"]))
    L += ["", "Per-load sums of the trace medians (us): "
          + ", ".join("%s %.2f" % (ld, d["sum_median_us"]) for ld, d in lt.items()) + ".", ""]
    return "\n".join(L)


def md_pmc(pm, csvs, logs):
    """profiles/pmc_loads.md from summarize_pmc()'s result."""
    args = "%s --pmc-logs %s" % (" ".join(shown(c) for c in csvs), " ".join(shown(g) for g in logs))
    L = ["# HBM traffic and MFMA use per launch, every load: rocprofv3 --pmc (MI355X, 1 GPU)", "",
         "Commands (%s; one counter set per run):" % CMD_VARS, "", "```"] + list(PMC_CMDS) + [
         "python bench.py --summarize-pmc %s > profiles/pmc_loads.json" % args,
         "python bench.py --summarize-pmc %s --md > profiles/pmc_loads.md" % args, "```", "",
         "The pass runs every load's five kernels cold (1 GiB flush before each), %d times, then copies 64 MiB three"
         % PMC_REPS,
         "times. FETCH_SIZE reads %.4f x fewer KiB than that copy moves and WRITE_SIZE reads it with scale %.4f; both"
         % (pm["fetch_scale"], pm["write_scale"]),
         "are multiplied by their scale. Medians of the %d passes. MFMA util = MFMA-busy cycles over all SIMD cycles"
         % PMC_REPS,
         "of the dispatch (rocprofv3's MfmaUtil); MOPS = SQ_INSTS_VALU_MFMA_MOPS_BF16 as counted. Kernels whose last",
         "template argument is `true` read 12-bit lossless weights (3/4 of the BF16 bytes plus a correction table).",
         "FETCH_SIZE counts what the L2 caches fetch from memory (HBM or the Infinity Cache behind them); each XCD's",
         "L2 fetches its own copy of data that workgroups on several XCDs read (x at large m).", "",
         "| load | layer | kernel | fetched by L2 (FETCH_SIZE, bytes) | written (WRITE_SIZE, bytes) | algorithmic bytes "
         "| traffic / algorithmic | MFMA util % | MFMA MOPS (bf16) |",
         "|---|---|---|---|---|---|---|---|---|"]
    for key, e in pm["launches"].items():
        L.append("| %s | %s | `%s` | %d | %d | %d | %.3f | %s | %s |" % (
            e["load"], key.split("@")[0], e["kernel"], e["fetch_bytes"], e["write_bytes"], e["algorithmic_bytes"],
            (e["fetch_bytes"] + e["write_bytes"]) / e["algorithmic_bytes"], e.get("mfma_util_pct", "-"),
            e.get("mfma_mops_bf16", "-")))
    L += ["", "Source hash of the kernels these counters belong to, as printed by the passes themselves: `%s` "
          "(bench.py reports `traffic` = null once the sources differ)." % pm["source_hash"], ""]
    return "\n".join(L)


PMC_REPS = 3


def pmc_sequence():
    """(load, layer) of the projection launches of `bench.py --pmc-pass`, in order."""
    from workload import LAYERS

    return [(name, l) for _ in range(PMC_REPS) for name in LOAD_ORDER for l in LAYERS]


def summarize_pmc(fetch_csv, write_csv, mfma_csv=None, copy_bytes=64 << 20, sources=None):
    """HBM bytes (and MFMA use) per launch of every (load, layer) from the counter
    passes of `bench.py --pmc-pass`.

    FETCH_SIZE and WRITE_SIZE are scaled by what they read on the copy kernel
    of known size in the same pass (copy_bytes read and copy_bytes written).
    The optional third pass holds MfmaUtil (MFMA-busy cycles over all SIMD
    cycles of the dispatch, percent) and SQ_INSTS_VALU_MFMA_MOPS_BF16.
    `sources`: the kernel-source hash the passes ran (pass_source_hash).
    """
    from gemv_decode_projections_amd import roofline as rf
    from workload import LOADS

    seq = pmc_sequence()
    res = {"source_hash": sources, "copy_bytes": copy_bytes, "launches": {}}

    def launches(path, cname):
        rows = sorted((r for r in _read_csv(path) if r["Counter_Name"] == cname),
                      key=lambda r: int(r["Dispatch_Id"]))
        sk = [r for r in rows if _is_proj_kernel(r["Kernel_Name"])]
        if len(sk) != len(seq):
            raise SystemExit("%s: %d projection launches, the pass makes %d" % (path, len(sk), len(seq)))
        return rows, sk

    def entry(name, layer, r=None):
        m = LOADS[name]
        key = "%s@%d" % (layer, m)
        if key not in res["launches"]:
            res["launches"][key] = {"load": name, "kernel": r["Kernel_Name"].split("(")[0].replace("void gdp::", ""),
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
        B.proj_bench_flush(b.flush, b.sink)
        B.proj_bench_copy(src, dst, n)
    torch.cuda.synchronize()
    log("pmc pass done: every load's kernels x%d, copy of %d bytes x3" % (PMC_REPS, n))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--load-reps", type=int, default=20, help="cold calls per layer for the other loads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timings")
    ap.add_argument("--graph-reps", type=int, default=15)
    ap.add_argument("--awkward-reps", type=int, default=7, help="cold calls per layer at each awkward token count")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-layer durations of the timed steps from a rocprofv3 trace of bench.py")
    ap.add_argument("--summarize-loads-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-(load, layer) kernel durations from a rocprofv3 trace of bench.py")
    ap.add_argument("--md", action="store_true", help="with --summarize-*: print the profiles/ Markdown page")
    ap.add_argument("--bench-json", metavar="PATH", help="with --summarize-trace --md: the bench line of the same run")
    ap.add_argument("--out-root", metavar="DIR", help="with --md: show paths under DIR as $OUT/... (the runs' output directory)")
    ap.add_argument("--pmc-logs", nargs="+", metavar="LOG",
                    help="with --summarize-pmc: the passes' output (names the kernel sources they ran)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print HBM bytes per launch from the --pmc passes: FETCH_SIZE csv, WRITE_SIZE csv "
                         "and optionally the MfmaUtil csv")
    args = ap.parse_args()
    global OUT_ROOT
    OUT_ROOT = args.out_root

    if args.summarize_trace:
        tr = summarize_trace(args.summarize_trace, args.steps, args.warmup)
        if args.md:
            line = None
            if args.bench_json:
                with open(args.bench_json) as f:
                    line = json.loads(f.read().strip().splitlines()[-1])
            print(md_decode1_trace(tr, args.summarize_trace, line, args.steps, args.warmup, args.bench_json))
        else:
            print(json.dumps(tr, indent=1))
        return
    if args.summarize_loads_trace:
        lt = summarize_loads_trace(args.summarize_loads_trace, args.steps, args.warmup, args.load_reps,
                                   args.graph_reps, args.awkward_reps)
        print(md_loads_trace(lt, args.summarize_loads_trace) if args.md else json.dumps(lt, indent=1))
        return
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3):
            raise SystemExit("--summarize-pmc takes FETCH_CSV WRITE_CSV [MFMA_CSV]")
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

    import torch

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    from gemv_decode_projections_amd import roofline as rf
    from gemv_decode_projections_amd import binding as B
    from gemv_decode_projections_amd import layers as layers_mod

    b = Bench()
    layers = b.LAYERS

    # Warmup steps (untimed).
    for _ in range(args.warmup):
        for layer in layers:
            b.kernel_us(layer, 1)

    # Timed steps: one decode-1 load each.
    per_layer = {l: [] for l in layers}
    step_us = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        tot = 0.0
        for layer in layers:
            t = b.kernel_us(layer, 1, variant=s % 2)
            per_layer[layer].append(t)
            tot += t
        step_us.append(tot)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = statistics.median(step_us)

    # Read floor at each layer's byte count, and the other loads.
    floor = {l: b.floor_us(rf.bytes_of(l, 1), 15) for l in layers}
    loads = {}
    for name in LOAD_ORDER:
        m = b.LOADS[name]
        lay = {}
        for layer in layers:
            if name == "decode-1":
                t = statistics.median(per_layer[layer])
            else:
                t = statistics.median(b.kernel_us(layer, m, variant=r % 2) for r in range(args.load_reps))
            lay[layer] = round(t, 2)
        tot = sum(lay.values())
        nbytes = sum(rf.bytes_of(l, m) for l in layers)
        flops = sum(rf.flops_of(l, m) for l in layers)
        # The hand-written read kernel over each shape's algorithmic bytes.
        lfloor = {l: floor[l] if m == 1 else b.floor_us(rf.bytes_of(l, m), 9) for l in layers}
        loads[name] = {
            "m": m, "us": round(tot, 2), "layers_us": lay,
            "read_floor_us": {l: round(v, 2) for l, v in lfloor.items()},
            "frac_of_read_floor": {l: round(lfloor[l] / lay[l], 3) for l in layers},
            "TBps": round(nbytes / tot / 1e6, 3),
            "TFLOPs": round(flops / tot / 1e6, 2),
            "mfma_frac": round(flops / tot / 1e6 / MFMA_BF16_TFLOPS, 4),
            "nominal_floor_us": round(rf.load_floor_us(m, router_peak=rf.MI355X_FP32_FLOPS), 2),
        }
        log("%-10s m=%-4d %8.2f us  %s" % (name, m, tot, lay))

    # The awkward token counts of the correctness sweep, timed the same way
    # (cold, kernel-duration events): per layer and summed over the five.
    from workload import AWKWARD_M
    awkward = {}
    for m in AWKWARD_M:
        lay = {l: round(statistics.median(b.kernel_us(l, m) for _ in range(args.awkward_reps)), 2) for l in layers}
        awkward[str(m)] = {"us": round(sum(lay.values()), 2), "layers_us": lay}
    log("awkward m: %s" % {m: v["us"] for m, v in awkward.items()})

    # The pages' own timing method for context: each call captured in a HIP
    # graph and replayed cold, minus the same for a graph of one empty kernel.
    graph = None
    if not args.no_graph:
        empty = b.graph_us(None, 1, args.graph_reps)
        graph = {"empty_graph_us": round(empty, 2), "loads": {}}
        for name in LOAD_ORDER:
            m = b.LOADS[name]
            lay = {l: round(b.graph_us(l, m, args.graph_reps) - empty, 2) for l in layers}
            graph["loads"][name] = {"m": m, "us_net": round(sum(lay.values()), 2), "layers_net_us": lay}
        log("graph replay (net of an empty-kernel graph, %.2f us): %s" % (
            empty, {k: v["us_net"] for k, v in graph["loads"].items()}))

    # Roofline of the dominant kernel of the headline load.
    dom = max(layers, key=lambda l: statistics.median(per_layer[l]))
    dom_avg = statistics.mean(per_layer[dom])
    dom_bytes = rf.bytes_of(dom, 1)
    achieved = dom_bytes / dom_avg / 1e3  # GB/s
    cfg = B.proj_plan(dom, 1)
    kname = kernel_name(cfg, dom == "router")
    # With 12-bit weights the kernel reads 3/4 of the BF16 weight bytes plus
    # one correction table; "achieved" still counts the BF16 bytes the
    # operation is defined on, and stored_bytes says what is actually read.
    stored = dom_bytes
    if cfg.kind == 0 and cfg.flags & 4:
        n, k, _, _ = layers_mod.DIMS[dom]
        stored = dom_bytes - rf.weight_bytes(dom, 1) // 4 + n * B.proj_compressed(dom) * 8
    roof = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "stored_bytes": stored, "weights": "12-bit lossless" if stored != dom_bytes else "bf16" if dom != "router" else "fp32",
        "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_for(dom, 1, kname),
        "kernel": kname, "layer": dom, "algorithmic_bytes": dom_bytes, "avg_us": round(dom_avg, 3),
        "measured_read_floor_us": round(floor[dom], 3),
        "frac_of_read_floor": round(floor[dom] / statistics.median(per_layer[dom]), 4),
    }

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    floor_sum = sum(floor.values())
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
        "vs_baseline": round(value / H200_DECODE1_US, 4),
        "baseline": {"value": H200_DECODE1_US, "unit": "us", "what": "pages' best decode-1 load time on H200 SXM (context, other hardware)"},
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode-1 load: m=1 through qkv_gate 2304x8192, o 8192x1024, pooler 4096x8192, "
                        "unpooler rows 0-1023 of 8192x4096, router 256x8192 fp32; cold cache before each layer",
            "m": 1,
            "timing": "kernel duration from hipExtLaunchKernel start/stop events, 1 GiB read flush before each call",
        },
        "decode1_layers_us": {l: round(statistics.median(per_layer[l]), 3) for l in layers},
        "decode1_read_floor_us": {l: round(floor[l], 3) for l in layers},
        "decode1_frac_of_read_floor": round(floor_sum / value, 4),
        "decode1_TBps": round(sum(rf.bytes_of(l, 1) for l in layers) / value / 1e6, 3),
        "loads": loads,
        "awkward_m": awkward,
        "graph_replay": graph,
        "timed_wall_s": round(wall, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
