"""proj_run_noalloc: the same plan and kernels as proj_run with the split-K
scratch in the library's fixed device array, called through the C ABI.

Checked against proj_run on the same inputs (bit-identical: same kernels, same
summation order) and against the oracle, for two calls in a row on one layer,
the second with fewer tokens (the array keeps the first call's state), over
plans with every kind of split-K scratch: polled partials (the router at 16-32
tokens, the unpooler slice at 5, qkv_gate's stream partition at 9), counted
partials with
arrival counters (wide-tile splits: qkv_gate at 16-32 tokens, 130-256 tokens on
the BF16 layers, the router's FP32 tiles at 300 and 1024 tokens, the unpooler's 128 x 128 tiles at 256 tokens,
whose 16 MiB of partials fill the array's counted region exactly), and none.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gemv_decode_projections_amd import binding  # noqa: E402
from tests.gpu_util import compare, sample_rows, say, to_device_weight, to_device_x, out_to_f64  # noqa: E402
from workload import make_weight, make_x  # noqa: E402

_W = {}


def _weights(layer):
    if layer not in _W:
        _W[layer] = make_weight(layer, 0)
        binding.proj_prepare(layer, to_device_weight(layer, _W[layer]))
        torch.cuda.synchronize()
    return _W[layer]


def _run(fn, layer, xd, m):
    out = binding.new_out(layer, m)
    out.fill_(float("nan"))
    fn(layer, xd, m, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("layer,m1,m2", [("router", 32, 16), ("qkv_gate", 32, 17), ("qkv_gate", 16, 9),
                                         ("pooler", 256, 130), ("qkv_gate", 256, 200), ("o", 300, 64),
                                         ("unpooler", 9, 5), ("router", 1024, 300),
                                         ("unpooler", 256, 200)])
def test_noalloc_matches_proj_run(layer, m1, m2):
    w = _weights(layer)
    for m in (m1, m2):
        cfg = binding.proj_plan(layer, m)
        say("noalloc", layer, "m=%d" % m, cfg.as_dict())
        xs = make_x(layer, m, seed=2000 + m, outliers=True)
        xd = to_device_x(xs.bits)
        ref_out = _run(binding.proj_run, layer, xd, m)
        got = _run(binding.proj_run_noalloc, layer, xd, m)
        assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                           ref_out.view(torch.int16) if got.dtype == torch.bfloat16 else ref_out.view(torch.int32))
        r = compare(layer, out_to_f64(got), w, xs, sample_rows(xs, m) if m >= 100 else None)
        assert r.ok, (m, r)
    assert binding.proj_split_giveups(layer) == 0


def test_noalloc_rejects_plans_beyond_its_scratch():
    """The pooler's counted partials at 1000 tokens (256 x 128 tiles, 2 K
    splits) need 32 MiB, more than the fixed array's 16 MiB for them: the call
    is refused on the host and launches nothing."""
    _weights("pooler")
    m = 1000
    cfg = binding.proj_plan("pooler", m)
    assert (cfg.kind, cfg.rb, cfg.nt, cfg.ksplit) == (3, 16, 8, 2)
    xd = to_device_x(make_x("pooler", m, seed=7).bits)
    out = binding.new_out("pooler", m)
    out.fill_(float("nan"))
    with pytest.raises(binding.ProjError) as e:
        binding.proj_run_noalloc("pooler", xd, m, out)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    binding.proj_run("pooler", xd, m, out)        # the allocating entry point still serves it
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
