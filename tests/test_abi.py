"""The C-ABI library loads and exports what include/*.h declares (CPU only: no GPU calls)."""

import ctypes
import os
import re

import pytest

from gemv_decode_projections_amd import binding, layers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in ("proj.h", "proj_bench.h"):
        with open(os.path.join(ROOT, "include", h)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(proj_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from gemv_decode_projections_amd import build

        build.build()
    return binding._lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 15, names
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_layer_table_matches_python_side(lib):
    for name in layers.LAYERS:
        n, k, wb, ob = binding.proj_layer_dims(name)
        assert (n, k, wb, ob) == layers.DIMS[name]
        for m in (1, 8, 9, 256, 4096):
            assert binding.proj_out_cols(name, m) == layers.n_eff(name, m)


def test_compressed_query_without_gpu(lib):
    assert lib.proj_compressed(9) == -1          # PROJ_ERR_LAYER
    assert lib.proj_compressed(4) == -5          # router not prepared here


def test_host_side_errors_without_gpu(lib):
    vp = ctypes.c_void_p
    assert lib.proj_out_cols(5, 1) == -1
    assert lib.proj_out_cols(-1, 1) == -1
    assert lib.proj_out_cols(0, 0) == -2
    assert lib.proj_out_cols(0, (1 << 30) + 1) == -2
    assert lib.proj_out_cols(0, 1 << 30) == 2304         # any m from 1 to 2^30
    assert lib.proj_out_cols(3, 4097) == 8192
    assert lib.proj_split_giveups(9, 0) == -1
    assert lib.proj_split_giveups(4, 0) == -5             # not prepared here
    assert lib.proj_run(7, vp(16), 1, vp(16), vp(0)) == -1
    assert lib.proj_run(0, vp(16), 0, vp(16), vp(0)) == -2
    assert lib.proj_run(0, vp(0), 1, vp(16), vp(0)) == -3
    assert lib.proj_run(0, vp(8), 1, vp(16), vp(0)) == -4
    assert lib.proj_run(0, vp(16), 1, vp(16), vp(0)) == -5       # not prepared
    assert lib.proj_prepare(9, vp(16)) == -1
    assert lib.proj_prepare(0, vp(0)) == -3
    assert lib.proj_prepare(0, vp(4)) == -4
    assert lib.proj_release(2) == 0 and lib.proj_release(2) == 0  # idempotent
    assert lib.proj_release(11) == -1
    for s in range(-8, 1):
        assert binding.proj_strerror(s) != "unknown status"


def test_dispatch_plans_tile_every_layer(lib):
    # Every (layer, m) resolves to a compiled variant that tiles the layer exactly.
    for name in layers.LAYERS:
        n, k, _, _ = layers.DIMS[name]
        for m in list(range(1, 41)) + [64, 100, 127, 128, 129, 130, 200, 256, 512, 1000, 4096, 4097, 8192, 8193,
                                       100000, 1 << 24, 1 << 30]:
            cfg = binding.proj_plan(name, m)
            ne = layers.n_eff(name, m)
            assert cfg.block == 64 * (cfg.waves + (1 if cfg.flags & 4 else 0))
            if cfg.kind == 2:
                # whole rows per workgroup: router and the unpooler slice at m <= 8
                assert name in ("router", "unpooler") and m <= cfg.nt <= 8 and cfg.ksplit == 1
                assert cfg.spw * 2048 == k
                assert ne % cfg.rb == 0 and cfg.grid == ne // cfg.rb
                continue
            if cfg.kind == 0 and cfg.flags & 256:
                # stream partition: qkv_gate at 9-15 tokens, its (row block, k-step) units dealt in
                # shares of waves x spw, one share per workgroup
                assert name == "qkv_gate" and 8 < m <= 15 and (cfg.nt, cfg.rb, cfg.ksplit) == (1, 1, 1)
                units = ne // 16 * (k // 32)
                assert units % (cfg.waves * cfg.spw) == 0 and cfg.grid == units // (cfg.waves * cfg.spw)
                continue
            if cfg.kind == 0:
                assert cfg.waves * cfg.spw * cfg.ksplit == k // 32
                # preloaded activations: one 16-token block, at most 4 (bit 5) or 8 (bit 6) tokens
                assert cfg.flags & 96 != 96
                assert not cfg.flags & 32 or (m <= 4 and cfg.nt == 1)
                assert not cfg.flags & 64 or (4 < m <= 8 and cfg.nt == 1)
                assert bool(cfg.flags & 96) == (m <= 8 and name in ("qkv_gate", "unpooler"))
            elif cfg.kind == 1:
                assert (k // 32) % (cfg.spw * cfg.ksplit) == 0
                assert m > 32
            elif m <= 32:
                # qkv_gate at 16-32 tokens and the pooler at 17-32 on wide tiles: 64 rows, one
                # (m = 16) or two token blocks, 4 waves, a 6- / 4-way split, the pooler's by LDS DMA
                qkv = name == "qkv_gate"
                assert cfg.kind == 3 and ((qkv and m >= 16) or (name == "pooler" and m >= 17))
                assert (cfg.nt, cfg.rb, cfg.waves, cfg.spw, cfg.ksplit, cfg.flags) == \
                    (1 if m <= 16 else 2, 4, 4, 16 if qkv else 8, 6 if qkv else 4, 0 if qkv else 128)
            else:
                # wide tiles: 4 waves (8 past 256 tokens, 256-row tiles), whole row blocks per
                # wave, any split up to one super-step each
                assert cfg.kind == 3 and m > 32 and cfg.waves in (4, 8) and cfg.rb % cfg.waves == 0
                # 8 waves: 256-row tiles past 256 tokens and for the pooler at 129-192; 128-row
                # tiles (one row block per wave) for the pooler at 193-256
                assert cfg.waves == 4 or (cfg.rb == 16 and (m > 256 and cfg.nt in (4, 8) or
                                                             name == "pooler" and 128 < m <= 192 and cfg.nt == 4)) \
                    or (name == "pooler" and 64 < m <= 256 and cfg.rb == 8)
                assert 1 <= cfg.ksplit <= k // (128 if cfg.spw >= 16 else 64)
                # activations by LDS DMA (bit 7) where it measured faster; no other bit
                dma = (name == "pooler" and m > 64) or (name == "unpooler" and m > 128) or \
                      (name == "qkv_gate" and 128 < m <= 256) or (name == "o" and 128 < m <= 512)
                assert cfg.flags == (128 if dma else 0)
            assert ne % (16 * cfg.rb) == 0
            n_tt = -(-m // (16 * cfg.nt))
            assert cfg.grid == ne // (16 * cfg.rb) * n_tt * cfg.ksplit


def test_variant_registry(lib):
    nv = binding.proj_num_variants()
    assert nv > 0
    seen = set()
    for i in range(nv):
        f32, cfg = binding.proj_variant(i)
        key = (f32, cfg.kind, cfg.nt, cfg.rb, cfg.waves, cfg.spw, cfg.flags & (4 | 32 | 64 | 128 | 256))
        assert key not in seen
        seen.add(key)
    with pytest.raises(binding.ProjError):
        binding.proj_variant(nv)


def test_run_config_rejects_untiled_configs(lib):
    # Host-side rejection happens before any GPU work; the layer is unprepared
    # here, so the first error reported is NOT_PREPARED for valid pointers.
    cfg = binding.ProjConfig.make(nt=1, rb=1, waves=8, spw=3, ksplit=1)
    rc = lib.proj_run_config(0, ctypes.c_void_p(16), 1, ctypes.c_void_p(16), ctypes.c_void_p(0),
                             ctypes.byref(cfg))
    assert rc == -5


def test_large_m_split_counts_keep_one_workgroup_per_cu(lib):
    # Past 128 tokens the K split is the largest that keeps the wide kernel's
    # grid within 256 workgroups (one per compute unit); grids above that only
    # come from the tiles themselves, without a split.
    for name in ("qkv_gate", "o", "pooler", "unpooler"):
        for m in list(range(129, 520, 7)) + [1000, 4096]:
            cfg = binding.proj_plan(name, m)
            assert cfg.kind == 3, (name, m)
            if cfg.ksplit > 1:
                assert cfg.grid <= 256, (name, m, cfg.as_dict())
                tiles = cfg.grid // cfg.ksplit
                assert tiles * (cfg.ksplit + 1) > 256 or cfg.ksplit == 4, (name, m, cfg.as_dict())


def test_wide_plans_between_129_and_256_tokens(lib):
    # The pooler at 129-192 tokens: 256 x 64 tiles on 8 waves, a 16-k-step prefetch, 5 splits.
    # The unpooler: 128 x 64 tiles without a split, or 128 x 128 tiles with 2 splits once the
    # last 64-token tile holds more than 32 tokens.
    for m in range(129, 257):
        p = binding.proj_plan("pooler", m)
        if m <= 192:
            assert (p.kind, p.rb, p.nt, p.waves, p.spw, p.ksplit, p.flags) == (3, 16, 4, 8, 16, 5, 128), m
        u = binding.proj_plan("unpooler", m)
        big = (m - 1) % 64 >= 32
        assert (u.kind, u.rb, u.nt, u.waves, u.ksplit, u.flags) == \
            ((3, 8, 8, 4, 2, 128) if big else (3, 8, 4, 4, 1, 128)), (m, u.as_dict())
        assert u.grid == (256 if big else 64 * -(-m // 64)), (m, u.as_dict())


def test_router_plans_past_256_tokens(lib):
    # Up to 256 tokens the skinny kernel with a 4-way polled split; past that
    # the wide kernel's FP32 tiles (64 rows, 64 tokens up to 1024 and 128
    # beyond) with a counted split of at most 8 whose partials fit the 32 MB
    # workspace, down to no split where the tiles alone fill the chip.
    assert binding.proj_plan("router", 256).as_dict()["kind"] == 0
    assert binding.proj_plan("router", 256).ksplit == 4
    for m in (257, 300, 512, 1000, 1024, 1025, 2048, 4096, 8192, 8193, 20000, 1 << 20):
        cfg = binding.proj_plan("router", m)
        nt = 4 if m <= 1024 else 8
        assert (cfg.kind, cfg.nt, cfg.rb, cfg.waves, cfg.spw, cfg.flags) == (3, nt, 4, 4, 4, 0), (m, cfg.as_dict())
        tiles = 4 * -(-m // (16 * nt))
        assert 1 <= cfg.ksplit <= 8 and cfg.grid == tiles * cfg.ksplit
        assert cfg.ksplit == 1 or tiles * cfg.ksplit * 64 * 16 * nt * 4 <= 32 << 20, (m, cfg.as_dict())
    assert binding.proj_plan("router", 1 << 20).ksplit == 1


def test_binding_rejects_bad_tensors_before_launch():
    # Shapes, dtypes, layout and placement are checked on the host; nothing
    # reaches the library (which is not even consulted for these).
    import torch

    bf, f32 = torch.bfloat16, torch.float32
    good_x = torch.zeros((4, 1024), dtype=bf)
    good_out = torch.zeros((4, 8192), dtype=bf)
    cases = [
        ("o", torch.zeros((4, 1000), dtype=bf), good_out, "shape"),          # wrong K
        ("o", torch.zeros((3, 1024), dtype=bf), good_out, "shape"),          # fewer than m rows
        ("o", torch.zeros((4, 1024), dtype=f32), good_out, "dtype"),         # x not BF16
        ("o", good_x, torch.zeros((4, 4096), dtype=bf), "shape"),            # wrong out width
        ("o", good_x, torch.zeros((4, 8192), dtype=f32), "dtype"),           # BF16 layer, FP32 out
        ("o", torch.zeros((1024, 4), dtype=bf).t(), good_out, "contiguous"), # transposed view
        ("o", torch.zeros((4, 2048), dtype=bf)[:, ::2], good_out, "contiguous"),
        ("router", torch.zeros((4, 8192), dtype=bf), torch.zeros((4, 256), dtype=bf), "dtype"),
        ("unpooler", torch.zeros((4, 4096), dtype=bf), torch.zeros((4, 8192), dtype=bf), "shape"),  # slice: 1024
        ("o", good_x, good_out, "not a GPU"),                                # right shapes, CPU memory
    ]
    for layer, x, out, what in cases:
        with pytest.raises(ValueError, match=what):
            binding.proj_run(layer, x, 4, out)
        with pytest.raises(ValueError, match=what):
            binding.proj_run_config(layer, x, 4, out, binding.ProjConfig.make())
