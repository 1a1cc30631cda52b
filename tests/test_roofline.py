"""The byte/FLOP accounting reproduces the numbers the pages print."""

import json
import os

import pytest

from gemv_decode_projections_amd import roofline as rf
from gemv_decode_projections_amd.layers import LAYERS, DIMS, n_eff

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_h200_load_floors_match_page_table():
    g = _load("h200_load_floors.json")
    for load, row in g["loads"].items():
        got = rf.load_floor_us(row["m"], bw=g["hbm_bytes_per_s"], peak=g["bf16_flops"])
        assert round(got, g["print_decimals"]) == pytest.approx(row["floor_us"], abs=1e-9), load


def test_h200_worked_examples():
    g = _load("h200_worked_examples.json")
    for c in g["cases"]:
        count = rf.weight_bytes if c["count"] == "weights" else rf.bytes_of
        b_us = count(c["layer"], c["m"]) / rf.H200_HBM_BPS * 1e6
        f_us = rf.flops_of(c["layer"], c["m"]) / rf.H200_BF16_FLOPS * 1e6
        assert round(b_us, c["decimals_bytes"]) == pytest.approx(c["bytes_us"]), c
        assert round(f_us, c["decimals_math"]) == pytest.approx(c["math_us"]), c


def test_weight_megabytes_match_layer_table():
    g = _load("h200_worked_examples.json")["weight_mb"]
    for name in LAYERS:
        assert round(rf.weight_bytes(name, 16) / 1e6, 1) == g[name]
    assert round(rf.weight_bytes("unpooler", 8) / 1e6, 1) == g["unpooler_slice"]


def test_slice_rule_and_flops():
    assert n_eff("unpooler", 8) == 1024 and n_eff("unpooler", 9) == 8192
    assert n_eff("pooler", 1) == 4096
    assert rf.flops_of("pooler", 1) == 2 * 4096 * 8192
    # router: FP32 weights and FP32 output are counted at 4 bytes
    assert rf.bytes_of("router", 2) == 256 * 8192 * 4 + 2 * 8192 * 2 + 2 * 256 * 4


def test_mi355x_floors_are_hbm_bound_for_bf16():
    for name in LAYERS:
        if name == "router":
            continue
        for m in (1, 8, 16, 32, 128, 256):
            assert rf.bytes_of(name, m) / rf.MI355X_HBM_BPS >= rf.flops_of(name, m) / rf.MI355X_BF16_FLOPS
