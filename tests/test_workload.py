"""The seeded generators: BF16 rounding, probe rows, outliers, determinism, tables."""

import numpy as np
import torch

from workload import (SHAPES, LAYERS, LOADS, AWKWARD_M, make_weight, make_x,
                      bf16_bits_from_f32, f32_from_bf16_bits)


def test_rne_matches_torch_bfloat16():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        # exact ties: bit 15 set, low 15 bits clear, both parities of bit 16
        (np.arange(2000, dtype=np.uint32) * 0x10000 + 0x3F808000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38], np.float32),
    ])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(a), want)
    assert np.array_equal(f32_from_bf16_bits(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_weights_seeded_and_scaled():
    w = make_weight("o", seed=1)
    assert w.dtype == np.uint16 and w.shape == SHAPES["o"]
    assert np.array_equal(w, make_weight("o", seed=1))
    assert not np.array_equal(w, make_weight("o", seed=2))
    std = f32_from_bf16_bits(w).std()
    assert abs(std - 1 / np.sqrt(1024)) < 0.01 / np.sqrt(1024)
    r = make_weight("router", seed=0)
    assert r.dtype == np.float32 and r.shape == (256, 8192)
    # router weights are not BF16-representable in general
    assert np.mean(f32_from_bf16_bits(bf16_bits_from_f32(r)) != r) > 0.9


def test_probe_rows_structure():
    for m, want in [(1, 0), (2, 1), (7, 1), (8, 1), (16, 2), (32, 4), (128, 16), (1000, 125)]:
        xs = make_x("pooler", m, seed=4, outliers=(m % 2 == 0))
        assert len(xs.probes) == want
        xf = f32_from_bf16_bits(xs.bits)
        for r, k, e in xs.probes:
            assert -3 <= e <= 3
            row = xf[r]
            assert row[k] == 2.0 ** e
            assert np.count_nonzero(row) == 1
    xs = make_x("o", 1, seed=0, probe_variant=True)
    assert len(xs.probes) == 1 and xs.probes[0][0] == 0


def test_outliers_fraction():
    xs_n = make_x("qkv_gate", 32, seed=9)
    xs_o = make_x("qkv_gate", 32, seed=9, outliers=True)
    big_n = np.abs(f32_from_bf16_bits(xs_n.bits)) > 16
    big_o = np.abs(f32_from_bf16_bits(xs_o.bits)) > 16
    non_probe = 32 - len(xs_o.probes)
    frac = big_o.sum() / (non_probe * 8192)
    assert big_n.sum() == 0 and 0.006 < frac < 0.0101


def test_tables_agree_across_sides():
    import oracle
    from gemv_decode_projections_amd import layers as pl

    assert tuple(pl.LAYERS) == tuple(LAYERS)
    for name in LAYERS:
        n, k = SHAPES[name]
        assert pl.DIMS[name][:2] == (n, k)
        assert oracle._LAYERS[name][:2] == (n, k)
        for m in (1, 8, 9, 256):
            assert oracle.out_cols(name, m) == pl.n_eff(name, m)
    assert sorted(LOADS.values()) == [1, 8, 16, 32, 128, 256]
    assert AWKWARD_M == (5, 7, 9, 33, 130, 512, 1000)
