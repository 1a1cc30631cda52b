"""Host logic of bench.py: kernel names, and the summaries it builds from
rocprofv3 CSV files (synthetic files here; no GPU)."""

import csv

import pytest

import bench
from gemv_decode_projections_amd import binding, roofline as rf
from workload import AWKWARD_M, LAYERS, LOADS


def _cfg(kind, nt, rb, waves, spw, ksplit=1, flags=0):
    return binding.ProjConfig.make(kind, nt, rb, waves, spw, ksplit, flags)


def test_kernel_names_match_the_templates():
    assert bench.kernel_name(_cfg(0, 1, 1, 8, 32), False) == "skinny_kernel<1, 1, 8, 32, false, false>"
    assert bench.kernel_name(_cfg(0, 1, 1, 8, 32, flags=4), False) == "skinny_kernel<1, 1, 8, 32, false, true>"
    assert bench.kernel_name(_cfg(0, 2, 1, 4, 16, 4), True) == "skinny_kernel<2, 1, 4, 16, true, false>"
    assert bench.kernel_name(_cfg(3, 4, 8, 4, 8, 2), False) == "wide_kernel<2, 4, 8, 2, false, false>"
    assert bench.kernel_name(_cfg(3, 4, 8, 4, 16, 2), False) == "wide_kernel<2, 4, 16, 4, false, false>"
    assert bench.kernel_name(_cfg(3, 2, 4, 4, 8, 256, 8), True) == "wide_kernel<1, 2, 8, 2, true, true>"
    assert bench.kernel_name(_cfg(1, 2, 8, 4, 8), False) == "tiled_kernel<2, 2, 4, 4, 8, false>"
    assert bench.kernel_name(_cfg(2, 8, 1, 4, 4), True) == "rowdot_kernel<8, 1, 4, true>"


FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def _pmc_csv(path, counters, proj_value, copy_value=None, drop=0):
    """A counter CSV shaped like rocprofv3's: a flush before every projection
    launch of the pass, then three copies."""
    seq = bench.pmc_sequence()[drop:]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        d = 0
        for i, (name, layer) in enumerate(seq):
            d += 1
            for c in counters:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": "gdp::(anonymous namespace)::flush_kernel(x)",
                            "Grid_Size": 1, "Counter_Name": c, "Counter_Value": 1})
            d += 1
            for c in counters:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": "void gdp::skinny_kernel<1, 1, 8, 32, false, false>(a)",
                            "Grid_Size": 4096 + i, "Counter_Name": c, "Counter_Value": proj_value(name, layer, c)})
        for _ in range(3):
            d += 1
            for c in counters:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": "gdp::(anonymous namespace)::copy_kernel(x)",
                            "Grid_Size": 1, "Counter_Name": c, "Counter_Value": copy_value})


def test_pmc_summary_scales_by_the_copy_and_keys_every_shape(tmp_path):
    copy_kib = (64 << 20) / 1024 / 2          # FETCH_SIZE reading half of what the copy moves
    _pmc_csv(tmp_path / "f.csv", ["FETCH_SIZE"], lambda n, l, c: rf.bytes_of(l, LOADS[n]) / 2048.0, copy_kib)
    _pmc_csv(tmp_path / "w.csv", ["WRITE_SIZE"], lambda n, l, c: 8.0, 64 << 10)
    _pmc_csv(tmp_path / "m.csv", ["MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16"],
             lambda n, l, c: 12.5 if c == "MfmaUtil" else LOADS[n])
    r = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "m.csv"),
                            sources="abc")
    assert r["fetch_scale"] == pytest.approx(2.0) and r["write_scale"] == pytest.approx(1.0)
    assert len(r["launches"]) == len(LOADS) * len(LAYERS)
    for name, m in LOADS.items():
        for layer in LAYERS:
            e = r["launches"]["%s@%d" % (layer, m)]
            assert e["load"] == name
            assert e["fetch_bytes"] == pytest.approx(rf.bytes_of(layer, m), abs=1)
            assert e["write_bytes"] == 8192
            assert e["algorithmic_bytes"] == rf.bytes_of(layer, m)
            assert e["mfma_util_pct"] == 12.5 and e["mfma_mops_bf16"] == m
    assert r["source_hash"] == "abc"


def test_pmc_summary_takes_the_source_hash_from_the_passes(tmp_path):
    """The hash comes from what the counter passes printed, so counters taken
    with other sources than the tree's are never labelled as current."""
    for i, h in enumerate(("aaa", "aaa", "bbb")):
        (tmp_path / ("p%d.log" % i)).write_text("noise\n%s %s\nmore\n" % (bench.PMC_HASH_TAG, h))
    assert bench.pass_source_hash([str(tmp_path / "p0.log"), str(tmp_path / "p1.log")]) == "aaa"
    with pytest.raises(SystemExit):
        bench.pass_source_hash([str(tmp_path / "p0.log"), str(tmp_path / "p2.log")])
    (tmp_path / "none.log").write_text("no tag\n")
    with pytest.raises(SystemExit):
        bench.pass_source_hash([str(tmp_path / "none.log")])


def test_pmc_summary_refuses_a_pass_with_missing_launches(tmp_path):
    _pmc_csv(tmp_path / "f.csv", ["FETCH_SIZE"], lambda n, l, c: 1.0, 1.0, drop=1)
    _pmc_csv(tmp_path / "w.csv", ["WRITE_SIZE"], lambda n, l, c: 1.0, 1.0)
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))


def test_loads_trace_summary_matches_the_launch_sequence(tmp_path):
    steps, warmup, load_reps, graph_reps, awkward_reps = 3, 1, 2, 2, 1
    seq = bench.call_sequence(steps, warmup, load_reps, graph_reps, awkward_reps)
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"])
        w.writeheader()
        t = 0
        for i, (name, layer) in enumerate(seq):
            w.writerow({"Kernel_Name": "gdp::(anonymous namespace)::flush_kernel(x)", "Start_Timestamp": t,
                        "End_Timestamp": t + 100000, "Grid_Size_X": 1})
            t += 100000
            dur = 1000 * (LAYERS.index(layer) + 1) + LOADS.get(name, 999)   # ns
            w.writerow({"Kernel_Name": "void gdp::wide_kernel<2, 4, 8, 2, false, false>(a)", "Start_Timestamp": t,
                        "End_Timestamp": t + dur, "Grid_Size_X": 256})
            t += dur
    r = bench.summarize_loads_trace(str(path), steps, warmup, load_reps, graph_reps, awkward_reps)
    for name, m in LOADS.items():
        lay = r[name]["layers"]
        for layer in LAYERS:
            assert lay[layer]["median_us"] == pytest.approx((1000 * (LAYERS.index(layer) + 1) + m) / 1e3)
            assert lay[layer]["kernel"] == "wide_kernel<2, 4, 8, 2, false, false>"
    for m in AWKWARD_M:
        assert r["m=%d" % m]["m"] == m
        for layer in LAYERS:
            assert r["m=%d" % m]["layers"][layer]["median_us"] == pytest.approx((1000 * (LAYERS.index(layer) + 1) + 999) / 1e3)
            assert lay[layer]["kernel"] == "wide_kernel<2, 4, 8, 2, false, false>"
    with pytest.raises(SystemExit):
        bench.summarize_loads_trace(str(path), steps + 1, warmup, load_reps, graph_reps, awkward_reps)


def test_profile_pages_render(tmp_path):
    copy_kib = (64 << 20) / 1024 / 2
    _pmc_csv(tmp_path / "f.csv", ["FETCH_SIZE"], lambda n, l, c: rf.bytes_of(l, LOADS[n]) / 2048.0, copy_kib)
    _pmc_csv(tmp_path / "w.csv", ["WRITE_SIZE"], lambda n, l, c: 8.0, 64 << 10)
    pm = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    page = bench.md_pmc(pm, ["f.csv", "w.csv"], ["f.log", "w.log"])
    assert page.count("\n| ") >= len(LOADS) * len(LAYERS) and "rocprofv3 --pmc FETCH_SIZE" in page
    tr = {l: {"kernel": "skinny_kernel<1, 1, 8, 32, false, false>", "grid": 64, "n": 3, "mean_us": 5.0,
              "median_us": 5.0} for l in LAYERS}
    page = bench.md_decode1_trace(tr, "t.csv")
    assert "Sum of the five trace medians: 25.00 us" in page and "--kernel-trace" in page
