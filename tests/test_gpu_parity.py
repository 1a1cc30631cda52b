"""GPU parity: the HIP path through the C ABI against the FP64 oracle.

Bounds (guide ch. 1 "The problem, the judge and the speed of light", §1.5):
global relative L2 <= 1e-2 (router 1e-4), probe rows <= 1e-3, no row above
5x the bound, no NaN/Inf. Inputs are the seeded synthetic workloads of
workload/ (shapes of §1.1, loads and awkward m of §1.2).
"""

import numpy as np
import pytest
import torch

from workload import LAYERS, LOADS, AWKWARD_M, SHAPES, make_weight, make_x, bf16_bits_from_f32
from workload.generate import f32_from_bf16_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only with -m gpu
    pytest.skip("no GPU", allow_module_level=True)

from gemv_decode_projections_amd import binding  # noqa: E402
from tests.gpu_util import (Prepared, run_layer, compare, sample_rows, say, to_device_x,  # noqa: E402
                            to_device_weight, out_to_f64)

_state = {"seed": None, "prep": None}
WS_BYTES = 32 << 20  # split-K workspace per layer (proj_prepare)


def prepared(seed):
    if _state["seed"] != seed:
        say("preparing all layers, weight seed", seed)
        _state["prep"] = Prepared(seed)
        _state["seed"] = seed
    return _state["prep"]


def _dirty():
    _state["seed"] = None


def test_mfma_lane_layout():
    rng = np.random.default_rng(0)
    A = rng.integers(-4, 5, size=(16, 32)).astype(np.float32)
    B = rng.integers(-4, 5, size=(32, 16)).astype(np.float32)
    Ad = to_device_x(bf16_bits_from_f32(A))
    Bd = to_device_x(bf16_bits_from_f32(B))
    C = torch.full((16, 16), float("nan"), dtype=torch.float32, device="cuda")
    binding.proj_bench_mfma_layout(Ad, Bd, C)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), A @ B)


@pytest.mark.parametrize("variant", ["normal", "probe"])
def test_o_projection_m1(variant):
    p = prepared(0)
    xs = make_x("o", 1, seed=100, probe_variant=(variant == "probe"))
    say("o m=1", variant)
    got = run_layer("o", xs.bits)
    r = compare("o", got, p.w["o"], xs)
    assert r.ok, r
    if variant == "probe":
        (row, k, e), = xs.probes
        col = f32_from_bf16_bits(p.w["o"][:, k]).astype(np.float64) * 2.0 ** e
        assert np.array_equal(got[row], col)   # an exact scaled weight column


@pytest.mark.parametrize("outliers", [False, True], ids=["normal", "outlier"])
@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("load", list(LOADS))
@pytest.mark.parametrize("wseed", [0, 1])
def test_loads(wseed, load, layer, outliers):
    p = prepared(wseed)
    m = LOADS[load]
    xs = make_x(layer, m, seed=200 + wseed, outliers=outliers)
    say("load", load, layer, "m=%d" % m, "wseed=%d" % wseed, "outliers" if outliers else "normal")
    got = run_layer(layer, xs.bits)
    r = compare(layer, got, p.w[layer], xs)
    assert r.ok, r


@pytest.mark.parametrize("outliers", [False, True], ids=["normal", "outlier"])
@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("m", AWKWARD_M)
@pytest.mark.parametrize("wseed", [0, 1])
def test_awkward_m(wseed, m, layer, outliers):
    p = prepared(wseed)
    xs = make_x(layer, m, seed=300 + wseed, outliers=outliers)
    say("awkward", layer, "m=%d" % m, "wseed=%d" % wseed, "outliers" if outliers else "normal")
    got = run_layer(layer, xs.bits)
    rows = sample_rows(xs, m) if m >= 100 else None
    r = compare(layer, got, p.w[layer], xs, rows)
    assert r.ok, r


@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("m", [4096, 4097, 8192])
def test_large_token_counts(m, layer):
    """Any m >= 1 is a valid call; large ones (the router's split partials
    stop fitting its workspace past 8192 tokens) are checked on sampled rows
    (every probe row, the first and last rows and random ones), all outputs
    finite."""
    p = prepared(0)
    xs = make_x(layer, m, seed=1100, outliers=True)
    say("large m", layer, "m=%d" % m, binding.proj_plan(layer, m).as_dict())
    got = run_layer(layer, xs.bits)
    r = compare(layer, got, p.w[layer], xs, sample_rows(xs, m))
    assert r.ok, r


@pytest.mark.parametrize("m", [1, 2, 3, 4, 6, 11, 13, 15, 17, 20, 24, 31, 40, 48, 64, 100])
def test_more_token_counts(m):
    p = prepared(0)
    for layer in LAYERS:
        xs = make_x(layer, m, seed=400, outliers=(m % 2 == 1))
        say("extra m", layer, "m=%d" % m)
        got = run_layer(layer, xs.bits)
        r = compare(layer, got, p.w[layer], xs)
        assert r.ok, (layer, r)


def _variant_cases():
    """Every compiled variant on a layer it tiles: (layer, kind, nt, rb, waves, spw, ksplit, flags)."""
    cases = []
    for i in range(binding.proj_num_variants()):
        f32, cfg = binding.proj_variant(i)
        if cfg.kind == 2:
            cases.append(("router" if f32 else "unpooler", 2, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 1, 0))
            continue
        cands = ["router"] if f32 else ["o", "unpooler", "qkv_gate"]
        for layer in cands:
            n, k = SHAPES[layer]
            ks = k // 32
            if cfg.kind == 0:
                if ks % (cfg.waves * cfg.spw) == 0:
                    split = ks // (cfg.waves * cfg.spw)
                    cases.append((layer, 0, cfg.nt, cfg.rb, cfg.waves, cfg.spw, split, cfg.flags))
                    break
            elif cfg.kind == 1 and n % (16 * cfg.rb) == 0:
                cases.append((layer, 1, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 1, 0))
                cases.append((layer, 1, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 2, 0))
                cases.append((layer, 1, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 2, 1))  # split groups across XCDs
                break
            elif cfg.kind == 3 and n % (16 * cfg.rb) == 0:
                f = cfg.flags                                                            # bit 7: LDS DMA
                cases.append((layer, 3, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 1, f))
                cases.append((layer, 3, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 3, f))   # uneven split lengths
                cases.append((layer, 3, cfg.nt, cfg.rb, cfg.waves, cfg.spw, 5, f | 1))   # uneven, across XCDs
                break
    return cases


@pytest.mark.parametrize("case", _variant_cases(), ids=lambda c: "%s-kind%d-nt%d-rb%d-w%d-s%d-k%d-f%d" % c)
def test_every_compiled_variant(case):
    layer, kind, nt, rb, waves, spw, split, flags = case
    p = prepared(0)
    if kind == 0 and flags & (32 | 64):
        ms = [1, 3, 4] if flags & 32 else [1, 5, 8]     # preloaded activations: at most 4 / 8 tokens
    elif kind == 0:
        ms = [1, 16 * nt - 3, 16 * nt + 5]
    elif kind == 1:
        ms = [33, 16 * nt + 5, 3 * 16 * nt - 7]
    elif kind == 3:
        ms = [1, 16 * nt - 3, 33, 16 * nt + 5, 3 * 16 * nt - 7]   # dispatched from 16 tokens up
    else:
        ms = [1, nt // 2 + 1, nt]      # row-dot: up to its token capacity
    for m in sorted(set(ms)):
        if layer == "unpooler" and m > 8 and kind == 0:
            continue
        if kind in (1, 3) and split > 1:
            n_tiles = (SHAPES[layer][0] // (16 * rb)) * -(-m // (16 * nt))
            if n_tiles * split * rb * nt * 1024 > WS_BYTES:
                continue  # the library rejects it: split-K workspace is 32 MB per layer
        cfg = binding.ProjConfig.make(kind=kind, nt=nt, rb=rb, waves=waves, spw=spw, ksplit=split, flags=flags)
        xs = make_x(layer, m, seed=500 + m, outliers=True)
        say("variant", case, "m=%d" % m)
        got = run_layer(layer, xs.bits, cfg=cfg)
        r = compare(layer, got, p.w[layer], xs)
        assert r.ok, (case, m, r)


# Stream mode of the wide-tile kernel: (layer, m, rb, nt, depth, workgroups,
# flags). Covers the production shape, an uneven share count without XCD
# grouping, the depth-16 prefetch, one super-step per workgroup (the most
# parts per tile), one workgroup for the whole layer, 128-token tiles and
# FP32 weights.
_STREAM_CASES = [("qkv_gate", 256, 8, 4, 8, 256, 8), ("qkv_gate", 130, 4, 4, 8, 250, 9),
                 ("pooler", 200, 8, 4, 16, 256, 8), ("o", 33, 8, 4, 4, 1024, 8), ("o", 33, 8, 4, 8, 1, 8),
                 ("unpooler", 400, 8, 8, 8, 264, 8), ("router", 256, 4, 2, 8, 256, 8),
                 # activations by LDS DMA (bit 7): several segments per workgroup refill the ring
                 ("qkv_gate", 130, 4, 4, 8, 250, 137), ("pooler", 200, 8, 4, 16, 256, 136),
                 ("o", 33, 8, 4, 8, 1, 136)]


@pytest.mark.parametrize("case", _STREAM_CASES, ids=lambda c: "%s-m%d-rb%d-nt%d-d%d-g%d-f%d" % c)
def test_wide_stream_mode(case):
    """The tiles' K super-steps dealt evenly to the workgroups (a share may end
    one tile and start the next) give oracle-exact results, and the same
    input twice gives the same bits (parts summed in workgroup order)."""
    layer, m, rb, nt, depth, groups, flags = case
    p = prepared(0)
    cfg = binding.ProjConfig.make(kind=3, nt=nt, rb=rb, waves=4, spw=depth, ksplit=groups, flags=flags)
    xs = make_x(layer, m, seed=1400 + m, outliers=True)
    say("stream", case)
    got = run_layer(layer, xs.bits, cfg=cfg)
    r = compare(layer, got, p.w[layer], xs)
    assert r.ok, (case, r)
    again = run_layer(layer, xs.bits, cfg=cfg)
    assert np.array_equal(got, again)


@pytest.mark.parametrize("layer,m", [("qkv_gate", 33), ("qkv_gate", 256), ("o", 256), ("pooler", 130),
                                     ("pooler", 256), ("unpooler", 128), ("unpooler", 300), ("pooler", 1000)])
def test_wide_dma_matches_register_staging(layer, m):
    """The wide-tile plan with its activations moved by LDS DMA (flags bit 7)
    gives the same bits as with them staged through registers: the same
    products summed in the same order."""
    p = prepared(0)
    cfg = binding.proj_plan(layer, m)
    if cfg.kind != 3:
        pytest.skip("plan is not the wide-tile kernel")
    xs = make_x(layer, m, seed=2200 + m, outliers=True)
    base = run_layer(layer, xs.bits, cfg=cfg)
    dma = binding.ProjConfig.make(kind=3, nt=cfg.nt, rb=cfg.rb, waves=cfg.waves, spw=cfg.spw,
                                  ksplit=cfg.ksplit, flags=(cfg.flags & ~128) | 128)
    say("dma", layer, "m=%d" % m, dma.as_dict())
    got = run_layer(layer, xs.bits, cfg=dma)
    assert np.array_equal(got, base)
    nodma = binding.ProjConfig.make(kind=3, nt=cfg.nt, rb=cfg.rb, waves=cfg.waves, spw=cfg.spw,
                                    ksplit=cfg.ksplit, flags=cfg.flags & ~128)
    assert np.array_equal(run_layer(layer, xs.bits, cfg=nodma), base)
    rows = sample_rows(xs, m) if m >= 100 else None
    assert compare(layer, got, p.w[layer], xs, rows=rows).ok


def test_wide_stream_mode_rejects_more_workgroups_than_super_steps():
    prepared(0)
    m, n_rt, nss = 33, 8192 // 128, 1024 // 32 // 2        # layer o, 128-row tiles, one token tile
    x = to_device_x(make_x("o", m, seed=3).bits)
    out = binding.new_out("o", m)
    ok = binding.ProjConfig.make(kind=3, nt=4, rb=8, waves=4, spw=8, ksplit=n_rt * nss, flags=8)
    binding.proj_run_config("o", x, m, out, ok)
    torch.cuda.synchronize()
    for bad in (binding.ProjConfig.make(kind=3, nt=4, rb=8, waves=4, spw=8, ksplit=n_rt * nss + 1, flags=8),
                binding.ProjConfig.make(kind=3, nt=4, rb=8, waves=4, spw=8, ksplit=2, flags=16),
                binding.ProjConfig.make(kind=3, nt=4, rb=8, waves=4, spw=8, ksplit=2, flags=32),
                binding.ProjConfig.make(kind=1, nt=2, rb=4, waves=4, spw=8, ksplit=1, flags=8)):
        with pytest.raises(binding.ProjError):
            binding.proj_run_config("o", x, m, out, bad)


def test_preload_flags_checked_against_token_count():
    """Preloaded activations hold 4 (bit 5) or 8 (bit 6) token rows of one
    16-token block: more tokens, both bits or two token blocks are rejected
    before launch; within the limit the output matches the per-k-step form
    bit for bit (same arithmetic, same summation order)."""
    p = prepared(0)
    mk = binding.ProjConfig.make
    for m in (4, 5, 8, 9):
        xs = make_x("qkv_gate", m, seed=2100 + m, outliers=True)
        x = to_device_x(xs.bits)
        out = binding.new_out("qkv_gate", m)
        base = run_layer("qkv_gate", xs.bits, cfg=mk(kind=0, nt=1, rb=1, waves=8, spw=32, ksplit=1, flags=4))
        for flags, fits in ((4 | 32, m <= 4), (4 | 64, m <= 8), (4 | 96, False)):
            cfg = mk(kind=0, nt=1, rb=1, waves=8, spw=32, ksplit=1, flags=flags)
            if not fits:
                with pytest.raises(binding.ProjError):
                    binding.proj_run_config("qkv_gate", x, m, out, cfg)
                continue
            say("preload", "qkv_gate", "m=%d flags=%d" % (m, flags))
            got = run_layer("qkv_gate", xs.bits, cfg=cfg)
            assert np.array_equal(got, base), (m, flags)
            assert compare("qkv_gate", got, p.w["qkv_gate"], xs).ok
    with pytest.raises(binding.ProjError):
        binding.proj_run_config("qkv_gate", to_device_x(make_x("qkv_gate", 4, seed=1).bits), 4,
                                binding.new_out("qkv_gate", 4),
                                mk(kind=0, nt=2, rb=1, waves=8, spw=32, ksplit=1, flags=64))


@pytest.mark.parametrize("layer,m", [("router", 1), ("router", 32), ("unpooler", 8)])
def test_split_k_across_xcds(layer, m):
    """Split-K groups spread over different XCDs (no workgroup grouping) still reduce correctly."""
    p = prepared(0)
    cfg = binding.proj_plan(layer, m)
    if cfg.kind != 0 or cfg.ksplit == 1:
        ks = SHAPES[layer][1] // 32
        cfg = binding.ProjConfig.make(nt=1, rb=1, waves=4, spw=ks // 16, ksplit=4)
    cfg.flags = 1
    for rep in range(3):
        xs = make_x(layer, m, seed=900 + rep, outliers=True)
        got = run_layer(layer, xs.bits, cfg=cfg)
        r = compare(layer, got, p.w[layer], xs)
        assert r.ok, (rep, r)


def _split_configs(layer):
    """Skinny splits of 2..16 workgroups (XCD-grouped and not) and a tiled split, all at 32 tokens."""
    ks_all = SHAPES[layer][1] // 32
    mk = binding.ProjConfig.make
    cfgs = [mk(kind=0, nt=2, rb=1, waves=8, spw=ks_all // (8 * ks), ksplit=ks, flags=f)
            for ks in (2, 4, 8, 16) for f in (0, 1)]
    cfgs.append(mk(kind=1, nt=2, rb=4, waves=4, spw=8, ksplit=4, flags=0))
    return cfgs


@pytest.mark.parametrize("layer", ["router", "qkv_gate"])
def test_split_workspaces_clean_between_kernels(layer):
    """Skinny splits poll their partials for an empty mark that the reducer puts
    back; tiled splits count arrivals. Interleaving both, with different split
    counts over the same tiles, never shows a stale partial: every rerun is bit
    identical to the first run of its configuration, which matches the oracle."""
    p = prepared(0)
    m = 32
    xs = make_x(layer, m, seed=950, outliers=True)
    first = {}
    cfgs = _split_configs(layer)
    for rnd in range(3):
        for i, cfg in enumerate(cfgs if rnd % 2 == 0 else cfgs[::-1]):
            key = str(cfg.as_dict())
            got = run_layer(layer, xs.bits, cfg=cfg)
            if key not in first:
                r = compare(layer, got, p.w[layer], xs)
                assert r.ok, (key, r)
                first[key] = got
            else:
                assert np.array_equal(got, first[key], equal_nan=True), (rnd, key)


def test_split_partial_with_all_ones_bits_is_not_lost():
    """A weight whose bits are all ones (a NaN) makes the partials of its row
    NaN; the polled reduction still ends at once, that row reads NaN and every
    other row is bit identical to a run without it."""
    import time
    _dirty()
    w = make_weight("router", 0).copy()
    w[5, 1000] = 0.0
    m = 16
    xs = make_x("router", m, seed=960)
    cfgs = [binding.proj_plan("router", m)] + [c for c in _split_configs("router") if c.kind == 0][:4]
    binding.proj_prepare("router", to_device_weight("router", w))
    clean = [run_layer("router", xs.bits, cfg=c) for c in cfgs]
    w[5, 1000] = np.uint32(0xFFFFFFFF).view(np.float32)
    binding.proj_prepare("router", to_device_weight("router", w))
    for c, ref in zip(cfgs, clean):
        t0 = time.perf_counter()
        got = run_layer("router", xs.bits, cfg=c)
        dt = time.perf_counter() - t0
        assert dt < 0.05, (c.as_dict(), dt)
        assert np.isnan(got[:, 5]).all(), c.as_dict()
        keep = np.arange(got.shape[1]) != 5
        assert np.array_equal(got[:, keep], ref[:, keep]), c.as_dict()
    _dirty()


@pytest.mark.parametrize("layer", LAYERS)
def test_output_rows_beyond_m_untouched(layer):
    prepared(0)
    m = 5
    xs = make_x(layer, m, seed=600)
    ncol = binding.proj_out_cols(layer, m)
    big = torch.full((m + 3, ncol), float("nan"), dtype=binding.out_dtype(layer), device="cuda")
    say("tail", layer)
    binding.proj_run(layer, to_device_x(xs.bits), m, big)
    torch.cuda.synchronize()
    g = out_to_f64(big)
    assert np.all(np.isfinite(g[:m])) and np.all(np.isnan(g[m:]))


@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("m", [1, 8, 16, 32, 33, 300, 700])
def test_graph_replay_fresh_inputs(layer, m):
    """Captured once, replayed with new x each time: split-K counters must reset
    on the GPU and nothing may be cached from an earlier x (guide ch. 1 §1.6)."""
    p = prepared(0)
    k = SHAPES[layer][1]
    x_static = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    out = binding.new_out(layer, m)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.proj_run(layer, x_static, m, out, s)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.proj_run(layer, x_static, m, out, s)
    say("graph", layer, "m=%d" % m)
    prev_bits = None
    for rep in range(6):
        xs = make_x(layer, m, seed=700 + rep, outliers=(rep % 2 == 1))
        x_static.copy_(to_device_x(xs.bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_to_f64(out)
        r = compare(layer, got, p.w[layer], xs, sample_rows(xs, m) if m >= 100 else None)
        assert r.ok, (rep, r)
        if rep == 0:
            prev_bits = out.clone()
    # Same x again: bit-identical result (fixed reduction order).
    xs = make_x(layer, m, seed=700)
    x_static.copy_(to_device_x(xs.bits))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       prev_bits.view(torch.int16) if out.dtype == torch.bfloat16 else prev_bits.view(torch.int32))


@pytest.mark.parametrize("layer,m", [("router", 16), ("qkv_gate", 32), ("pooler", 256), ("unpooler", 1)])
def test_first_call_after_prepare_captured_in_graph(layer, m):
    """Prepare warms every kernel its plans can pick, so the very first
    proj_run of a freshly prepared layer may be the one captured in a graph;
    the replays are exact and bit identical."""
    _dirty()
    w = make_weight(layer, 3)
    binding.proj_prepare(layer, to_device_weight(layer, w))
    torch.cuda.synchronize()
    k = SHAPES[layer][1]
    x_static = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    out = binding.new_out(layer, m)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.proj_run(layer, x_static, m, out, s)   # first call of the layer since prepare
    say("first call captured", layer, "m=%d" % m)
    first = None
    for rep in range(3):
        xs = make_x(layer, m, seed=1500 + rep % 2, outliers=True)
        x_static.copy_(to_device_x(xs.bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_to_f64(out)
        r = compare(layer, got, w, xs, sample_rows(xs, m) if m >= 100 else None)
        assert r.ok, (rep, r)
        if rep == 0:
            first = got
        if rep == 2:
            assert np.array_equal(got, first)
    _dirty()


@pytest.mark.parametrize("layer,m", [("router", 32), ("qkv_gate", 32)])
def test_split_giveup_is_counted_and_cleaned(layer, m):
    """A polled split-K reducer that stops waiting is visible to the host. The
    test configuration (flags bit 4) makes the splits that do not reduce drop
    their partials and the reducer poll once: every kernel still exits at
    once, the missing partials read NaN, each give-up is counted, the marks
    are restored, and the next launch of the normal plan is exact."""
    p = prepared(0)
    assert binding.proj_split_giveups(layer, reset=True) == 0
    ks = SHAPES[layer][1] // 32
    cfg = binding.ProjConfig.make(kind=0, nt=2, rb=1, waves=8, spw=ks // 32, ksplit=4, flags=16)
    xs = make_x(layer, m, seed=1600, outliers=True)
    say("forced give-up", layer, "m=%d" % m, cfg.as_dict())
    got = run_layer(layer, xs.bits, cfg=cfg)
    assert np.isnan(got).all()
    n_tiles = (SHAPES[layer][0] // 16) * -(-m // 32)
    assert binding.proj_split_giveups(layer) == n_tiles * 3        # one per reducer wave and missing split
    for c in (binding.proj_plan(layer, m), binding.ProjConfig.make(kind=0, nt=2, rb=1, waves=8, spw=ks // 32,
                                                                    ksplit=4)):
        got = run_layer(layer, xs.bits, cfg=c)
        r = compare(layer, got, p.w[layer], xs)
        assert r.ok, (c.as_dict(), r)
    assert binding.proj_split_giveups(layer, reset=True) == n_tiles * 3
    assert binding.proj_split_giveups(layer) == 0


# (token blocks, waves, k-steps per wave, 12-bit flag): every compiled stream-partition variant.
_SK_CFGS = [(nt, w, s, z) for (nt, w, s) in ((1, 4, 36), (1, 6, 24), (1, 9, 16), (1, 12, 12), (2, 6, 24), (2, 9, 16))
            for z in (0, 4)] + [(1, 2, 72, 4), (1, 3, 48, 4), (2, 4, 36, 4), (2, 3, 48, 4), (2, 2, 72, 4)]


@pytest.mark.parametrize("nt,waves,spw,z", _SK_CFGS)
def test_stream_partition(nt, waves, spw, z):
    """The skinny kernel's stream partition (flags bit 8): qkv_gate's 144 row
    blocks x 256 k-steps dealt in 256 shares of waves x spw = 144 units, a
    share spanning the end of one row block and the start of the next, each
    row block's two or three parts summed by the share dispatched last. Exact
    against the oracle (BF16 and 12-bit weights, one and two token blocks,
    ragged m), bit-identical on a rerun, and no reducer gives up."""
    p = prepared(0)
    layer = "qkv_gate"
    mk = binding.ProjConfig.make
    cfg = mk(kind=0, nt=nt, rb=1, waves=waves, spw=spw, ksplit=1, flags=256 | z)
    for m in ((1, 7, 16) if nt == 1 else (17, 24, 32)):
        xs = make_x(layer, m, seed=2500 + m, outliers=True)
        say("stream partition", cfg.as_dict(), "m=%d" % m)
        got = run_layer(layer, xs.bits, cfg=cfg)
        r = compare(layer, got, p.w[layer], xs)
        assert r.ok, (m, r)
        assert np.array_equal(run_layer(layer, xs.bits, cfg=cfg), got)
    assert binding.proj_split_giveups(layer) == 0


def test_stream_partition_rejects_what_it_cannot_cover():
    """Host-side checks: too many tokens for its token blocks, a share count
    that does not divide the layer's units, another flag with it."""
    prepared(0)
    mk = binding.ProjConfig.make
    x = to_device_x(make_x("qkv_gate", 17, seed=3).bits)
    out = binding.new_out("qkv_gate", 17)
    with pytest.raises(binding.ProjError):                       # 17 tokens, one token block
        binding.proj_run_config("qkv_gate", x, 17, out, mk(kind=0, nt=1, rb=1, waves=6, spw=24, ksplit=1, flags=256))
    xo = to_device_x(make_x("o", 4, seed=3).bits)
    with pytest.raises(binding.ProjError):                       # o: 512 x 32 units, not a multiple of 144
        binding.proj_run_config("o", xo, 4, binding.new_out("o", 4),
                                mk(kind=0, nt=1, rb=1, waves=6, spw=24, ksplit=1, flags=256))
    for bad in (mk(kind=0, nt=1, rb=1, waves=6, spw=24, ksplit=2, flags=256),
                mk(kind=0, nt=1, rb=2, waves=6, spw=24, ksplit=1, flags=256),
                mk(kind=0, nt=1, rb=1, waves=6, spw=24, ksplit=1, flags=256 | 32)):
        with pytest.raises(binding.ProjError):
            binding.proj_run_config("qkv_gate", x, 4, out, bad)


def test_stream_partition_giveup_is_counted_and_cleaned():
    """With the test flag (bit 4) the shares that do not reduce publish
    nothing and each reducer polls once: outputs of row blocks with several
    parts read NaN, one give-up per reducer wave, the marks restored, and the
    same configuration without the flag is exact afterwards."""
    p = prepared(0)
    layer = "qkv_gate"
    assert binding.proj_split_giveups(layer, reset=True) == 0
    mk = binding.ProjConfig.make
    xs = make_x(layer, 16, seed=2600, outliers=True)
    got = run_layer(layer, xs.bits, cfg=mk(kind=0, nt=1, rb=1, waves=6, spw=24, ksplit=1, flags=256 | 16 | 4))
    assert np.isnan(got).all()              # every row block of qkv_gate has two or three parts
    assert binding.proj_split_giveups(layer) > 0
    got = run_layer(layer, xs.bits, cfg=mk(kind=0, nt=1, rb=1, waves=6, spw=24, ksplit=1, flags=256 | 4))
    assert compare(layer, got, p.w[layer], xs).ok
    binding.proj_split_giveups(layer, reset=True)
    assert binding.proj_split_giveups(layer) == 0


def test_no_split_giveups_in_normal_use():
    """No polled split-K reducer gives up in normal use: not in prepare's
    warm-up launches and not over every load's plans (a give-up there would
    mean a reducer stopped waiting for a partial that was on its way, whose
    late words would then read as arrived in a later launch)."""
    prepared(0)
    for layer in SHAPES:
        assert binding.proj_split_giveups(layer) == 0, layer
    for m in LOADS.values():
        for layer in SHAPES:
            xs = make_x(layer, m, seed=2300 + m)
            run_layer(layer, xs.bits)
    for m in (33, 64, 130, 300, 512, 1000):
        for layer in SHAPES:
            run_layer(layer, make_x(layer, m, seed=2400 + m).bits)
    for layer in SHAPES:
        assert binding.proj_split_giveups(layer) == 0, layer


def _exception_columns(w, limit=3):
    """Columns holding weights outside the 12-bit exponent table: the eight
    consecutive values of BF16 bits 14..8 that cover the most weights (the
    report's round-5 rule, recomputed here from the host weights)."""
    h = (w >> 8) & 0x7F
    hist = np.bincount(h.ravel(), minlength=128)
    base = int(np.argmax([hist[b:b + 8].sum() for b in range(121)]))
    exc = (h < base) | (h > base + 7)
    cols = np.nonzero(exc.any(axis=0))[0]
    return [int(c) for c in cols[:limit]], exc


def test_layers_keep_a_12bit_form():
    prepared(0)
    for layer in ("qkv_gate", "o", "pooler", "unpooler"):
        assert 0 <= binding.proj_compressed(layer) <= 8, layer
    assert binding.proj_compressed("router") == -1


# (m, 16-token blocks, row blocks, waves, largest k-steps per wave): one and
# two token blocks, one and two row blocks, with and without a K split across
# workgroups (the corrections of a slot are applied only by its split).
_Z_CASES = [(1, 1, 1, 8, 32), (5, 1, 1, 8, 32), (16, 1, 1, 8, 32), (16, 1, 1, 4, 8),
            (24, 2, 2, 4, 32), (32, 2, 1, 8, 16)]


def _z_config(layer, nt, rb, waves, spw_max):
    ks_total = SHAPES[layer][1] // 32
    spw_min = 2 if nt == 1 else 8             # smallest compiled 12-bit stage depth
    if ks_total // waves < spw_min:
        waves = 4
    spw = min(spw_max, ks_total // waves)
    return binding.ProjConfig.make(kind=0, nt=nt, rb=rb, waves=waves, spw=spw,
                                   ksplit=ks_total // (waves * spw), flags=4)


@pytest.mark.parametrize("layer", ["qkv_gate", "o", "pooler", "unpooler"])
@pytest.mark.parametrize("case", _Z_CASES, ids=lambda c: "m%d-nt%d-rb%d-w%d" % c[:4])
def test_12bit_exception_columns_bit_exact(layer, case):
    """A one-hot activation row on a column holding out-of-table weights returns
    that weight column times the scale bit for bit through the 12-bit path
    (report round 5: the corrections restore the original weights exactly);
    the other rows are ordinary inputs checked against the oracle."""
    m = case[0]
    p = prepared(0)
    w = p.w[layer]
    cols, exc = _exception_columns(w)
    assert cols, "weights without any out-of-table value"
    n_eff = binding.proj_out_cols(layer, m)
    cfg = _z_config(layer, *case[1:])
    for k in cols:
        xs = make_x(layer, m, seed=1200 + k)
        bits = xs.bits.copy()
        bits[0, :] = 0
        bits[0, k] = bf16_bits_from_f32(np.array([2.0 ** -3], dtype=np.float32))[0]
        xs.bits = bits
        say("12-bit exception column", layer, "m=%d" % m, "k=%d" % k, "rows with exceptions", int(exc[:n_eff, k].sum()),
            cfg.as_dict())
        got = run_layer(layer, bits, cfg=cfg)
        want = f32_from_bf16_bits(w[:n_eff, k]).astype(np.float64) * 2.0 ** -3
        assert np.array_equal(got[0], want)
        if m > 1:
            xs.probes = [pr for pr in xs.probes if pr[0] != 0]
            r = compare(layer, got[1:], w, _RowsView(xs, 1))
            assert r.ok, r


class _RowsView:
    """x rows [start:] of a seeded input, with its probe rows renumbered."""

    def __init__(self, xs, start):
        self.bits = xs.bits[start:]
        self.probes = [(r - start, k, e) for (r, k, e) in xs.probes if r >= start]
        self.probe_rows = [r for (r, _, _) in self.probes]


def test_12bit_form_skipped_when_a_row_needs_too_many_corrections():
    """Weights with more out-of-table values in one row than the correction
    slots hold: prepare keeps only the BF16 form, the dispatch does not ask
    for 12-bit weights, and results stay exact."""
    _dirty()
    w = make_weight("pooler", 0).copy()
    w[7, 100:140:4] = 0                      # ten exact zeros in row 7: all outside the table
    binding.proj_prepare("pooler", to_device_weight("pooler", w))
    assert binding.proj_compressed("pooler") == -1
    assert binding.proj_plan("pooler", 1).flags & 4 == 0
    with pytest.raises(binding.ProjError):
        binding.proj_run_config("pooler", to_device_x(make_x("pooler", 1, seed=5).bits), 1,
                                binding.new_out("pooler", 1),
                                binding.ProjConfig.make(kind=0, nt=1, rb=1, waves=8, spw=32, ksplit=1, flags=4))
    for m in (1, 16):
        xs = make_x("pooler", m, seed=1300 + m)
        got = run_layer("pooler", xs.bits)
        r = compare("pooler", got, w, xs)
        assert r.ok, r
    _dirty()


def test_bf16_output_rounding_is_nearest_even():
    """Exact FP32 sums that fall halfway between two BF16 values round to the even one."""
    _dirty()
    n, k = SHAPES["o"]
    j = np.arange(n) % 128
    a = (1.0 + j * 2.0 ** -7).astype(np.float32)                 # exact in BF16
    b = np.choose(np.arange(n) % 4, [1.0, -1.0, 3.0, 0.5]).astype(np.float32)
    w = np.zeros((n, k), dtype=np.float32)
    w[:, 0] = a
    w[:, 1] = b
    wb = bf16_bits_from_f32(w)
    binding.proj_prepare("o", to_device_weight("o", wb))
    x = np.zeros((1, k), dtype=np.float32)
    x[0, 0] = 1.0
    x[0, 1] = 2.0 ** -8
    got = run_layer("o", bf16_bits_from_f32(x))
    exact = (a.astype(np.float64) + b.astype(np.float64) * 2.0 ** -8)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)  # sums exact in FP32
    want = f32_from_bf16_bits(bf16_bits_from_f32(exact.astype(np.float32))).astype(np.float64)
    assert np.array_equal(got[0], want)
    _dirty()


@pytest.mark.parametrize("m", [1, 16, 256, 300, 1100, 2048])
def test_router_keeps_fp32_weight_bits(m):
    """Router weights that BF16 cannot hold must still reach the sum exactly: a
    probe row returns the FP32 weight column bit for bit, on every router
    kernel (row-dot at 1 token, the skinny kernel's three-part split at 16 and
    256, the wide-tile kernel's at 300-2048)."""
    p = prepared(0)
    xs = make_x("router", m, seed=800 + m, probe_variant=True)
    say("router exact bits", binding.proj_plan("router", m).as_dict(), "m=%d" % m)
    got = run_layer("router", xs.bits)
    assert xs.probes
    for row, kk, e in xs.probes:
        want = p.w["router"][:, kk].astype(np.float64) * 2.0 ** e
        assert np.array_equal(got[row], want), (m, row, kk)
