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
    assert bench.kernel_name(_cfg(0, 1, 1, 8, 32), False) == "skinny_kernel<1, 1, 8, 32, false, false, 0>"
    assert bench.kernel_name(_cfg(0, 1, 1, 8, 32, flags=4), False) == "skinny_kernel<1, 1, 8, 32, false, true, 0>"
    assert bench.kernel_name(_cfg(0, 2, 1, 4, 16, 4), True) == "skinny_kernel<2, 1, 4, 16, true, false, 0>"
    assert bench.kernel_name(_cfg(3, 4, 8, 4, 8, 2), False) == "wide_kernel<2, 4, 8, 2, false, false, 4, false>"
    assert bench.kernel_name(_cfg(3, 4, 8, 4, 16, 2), False) == "wide_kernel<2, 4, 16, 4, false, false, 4, false>"
    assert bench.kernel_name(_cfg(3, 2, 4, 4, 8, 256, 8), True) == "wide_kernel<1, 2, 8, 2, true, true, 4, false>"
    assert bench.kernel_name(_cfg(3, 4, 16, 8, 8, 2), False) == "wide_kernel<2, 4, 8, 2, false, false, 8, false>"
    assert bench.kernel_name(_cfg(3, 8, 8, 8, 8, 4, 128), False) == "wide_kernel<1, 8, 8, 2, false, false, 8, true>"
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
        for _ in range(5):       # prepare's warm-up launches, before the pass's first flush
            d += 1
            for c in counters:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": "void gdp::skinny_kernel<1, 1, 8, 32, false, true, 0>(a)",
                            "Grid_Size": 256, "Counter_Name": c, "Counter_Value": 1e9})
        for i, (name, layer) in enumerate(seq):
            d += 1
            for c in counters:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": "gdp::(anonymous namespace)::flush_kernel(x)",
                            "Grid_Size": 1, "Counter_Name": c, "Counter_Value": 1})
            d += 1
            for c in counters:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": "void gdp::skinny_kernel<1, 1, 8, 32, false, false, 0>(a)",
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
    # LDS pass: conflicts on half the active cycles except the router's launches (no indexed LDS use)
    _pmc_csv(tmp_path / "l.csv", ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"],
             lambda n, l, c: 0.0 if l == "router" else (50.0 if c == "SQ_LDS_BANK_CONFLICT" else 100.0))
    r = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "m.csv"),
                            str(tmp_path / "l.csv"), sources="abc")
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
            assert e.get("lds_conflict_pct") == (None if layer == "router" else 50.0)
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


TRACE_FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]


def test_loads_trace_summary_matches_the_launch_sequence(tmp_path):
    counts = (3, 1, 2, 1, 2)     # steps, warmup, study reps, awkward reps, graph reps
    seq = bench.call_sequence(*counts)
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        t = 0
        for i in range(7):     # prepare's warm-up launches, before any flush
            w.writerow({"Kernel_Name": "void gdp::skinny_kernel<1, 1, 8, 32, false, true, 0>(a)", "Start_Timestamp": t,
                        "End_Timestamp": t + 5000, "Grid_Size_X": 256})
            t += 6000
        for i, (tag, layer, m) in enumerate(seq):
            w.writerow({"Kernel_Name": "gdp::(anonymous namespace)::flush_kernel<false>(x)", "Start_Timestamp": t,
                        "End_Timestamp": t + 100000, "Grid_Size_X": 1})
            t += 100000
            dur = 1000 * (LAYERS.index(layer) + 1) + m + (500 if tag.startswith("warmup") else 0)   # ns
            w.writerow({"Kernel_Name": "void gdp::wide_kernel<2, 4, 8, 2, false, false, 4, false>(a)",
                        "Start_Timestamp": t, "End_Timestamp": t + dur, "Grid_Size_X": 256})
            t += dur
    r = bench.summarize_loads_trace(str(path), *counts)
    assert not any(k.startswith("warmup") for k in r)
    for name, m in LOADS.items():
        lay = r[name]["layers"]
        assert r[name]["m"] == m
        for layer in LAYERS:
            assert lay[layer]["n"] == counts[0]
            assert lay[layer]["median_us"] == pytest.approx((1000 * (LAYERS.index(layer) + 1) + m) / 1e3)
            assert lay[layer]["kernel"] == "wide_kernel<2, 4, 8, 2, false, false, 4, false>"
        assert r["graph:" + name]["layers"]["o"]["n"] == counts[4]
    for m in AWKWARD_M:
        assert r["m=%d" % m]["m"] == m
    assert r["study:none"]["layers"]["pooler"]["n"] == counts[2]
    with pytest.raises(SystemExit):
        bench.summarize_loads_trace(str(path), counts[0] + 1, *counts[1:])


def _graph_trace(path, reps, gap_ns=700):
    """A kernel trace of the graph leg: per load, `reps` pairs of (load graph,
    floor graph), each a stamp, five kernels, a stamp, separated by flushes."""
    t = 0
    rows = []

    def add(name, dur):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur, "Grid_Size_X": 1})
        t += dur + gap_ns
    for j, name in enumerate(bench.LOAD_ORDER):
        for r in range(reps):
            for which in (("load", "floor") if r % 2 == 0 else ("floor", "load")):
                add("gdp::(anonymous namespace)::flush_kernel<false>(a)", 200000)
                add("gdp::(anonymous namespace)::stamp_kernel(a, b)", 1000)
                for i, layer in enumerate(LAYERS):
                    k = ("void gdp::skinny_kernel<1, 1, 8, 32, false, false, 0>(a)" if which == "load"
                         else "gdp::(anonymous namespace)::read_floor_kernel<4, false>(a)")
                    add(k, 1000 * (i + 1) + (100 * j if which == "load" else 0))
                add("gdp::(anonymous namespace)::stamp_kernel(a, b)", 1000)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        w.writerows(rows)


def test_graph_trace_summary_gives_kernels_gaps_and_span(tmp_path):
    _graph_trace(tmp_path / "g.csv", 3)
    r = bench.summarize_graph_trace(str(tmp_path / "g.csv"), 3)
    assert list(r) == list(bench.LOAD_ORDER)
    for j, name in enumerate(bench.LOAD_ORDER):
        g, fl = r[name]["graph"], r[name]["floor_graph"]
        assert g["kernel_median_us"] == pytest.approx([(1000 * (i + 1) + 100 * j) / 1e3 for i in range(5)])
        assert fl["kernel_median_us"] == pytest.approx([i + 1.0 for i in range(5)])
        assert g["gap_median_us"] == pytest.approx([0.7] * 6)
        assert g["span_median_us"] == pytest.approx(sum(g["kernel_median_us"]) + 4 * 0.7)
        assert g["kernels"][0].startswith("skinny_kernel") and g["n"] == 3
    page = bench.md_graph_trace(r, "g.csv", 3)
    assert "median gap is 0.70 us" in page
    with pytest.raises(SystemExit):
        bench.summarize_graph_trace(str(tmp_path / "g.csv"), 4)


def test_profile_pages_render(tmp_path):
    copy_kib = (64 << 20) / 1024 / 2
    _pmc_csv(tmp_path / "f.csv", ["FETCH_SIZE"], lambda n, l, c: rf.bytes_of(l, LOADS[n]) / 2048.0, copy_kib)
    _pmc_csv(tmp_path / "w.csv", ["WRITE_SIZE"], lambda n, l, c: 8.0, 64 << 10)
    pm = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    page = bench.md_pmc(pm, ["f.csv", "w.csv"], ["f.log", "w.log"])
    assert page.count("\n| ") >= len(LOADS) * len(LAYERS) and "rocprofv3 --pmc FETCH_SIZE" in page
    line = {"flush_study": {"reps": 5, "chosen": "plain-1GiB",
                            "conditions": {c: {"floor_us": 11.0 + i, "pooler_decode1_us": 9.0 + i}
                                           for i, (c, _, _) in enumerate(bench.STUDY_CONDITIONS)}}}
    page = bench.md_flush_study(line, "b.json")
    assert "| plain-2GiB | 14.00 | 12.00 |" in page and "`plain-1GiB` flush" in page


def test_stored_bytes_of_12bit_kernels():
    cfg = _cfg(0, 1, 1, 8, 32, flags=4)
    w = rf.weight_bytes("pooler", 1)
    assert bench.stored_bytes("pooler", 1, cfg, 7) == rf.bytes_of("pooler", 1) - w // 4 + 4096 * 7 * 8
    assert bench.stored_bytes("pooler", 1, _cfg(0, 1, 1, 8, 32), 7) == rf.bytes_of("pooler", 1)
    assert bench.mfma_flops("router", 256) == 3 * rf.flops_of("router", 256)
