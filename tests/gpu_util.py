"""Helpers shared by the GPU tests: upload seeded inputs, run through the C ABI,
compare with the oracle."""

import sys

import numpy as np
import torch

import oracle
from oracle.check import check
from workload import SHAPES, make_weight, make_x
from gemv_decode_projections_amd import binding

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device_weight(layer, w):
    if w.dtype == np.float32:
        return torch.from_numpy(w).to(DEV)
    return torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(DEV)


def to_device_x(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def out_to_f64(out):
    return out.detach().to("cpu").double().numpy()


class Prepared:
    """Host copies of the weights of every layer for one weight seed, prepared on the GPU."""

    def __init__(self, seed):
        self.seed = seed
        self.w = {}
        for layer in SHAPES:
            w = make_weight(layer, seed)
            self.w[layer] = w
            wd = to_device_weight(layer, w)
            binding.proj_prepare(layer, wd)
            del wd
        torch.cuda.synchronize()


def run_layer(layer, x_bits, stream=None, cfg=None):
    m = x_bits.shape[0]
    x = to_device_x(x_bits)
    out = binding.new_out(layer, m)
    out.fill_(float("nan"))
    if cfg is None:
        binding.proj_run(layer, x, m, out, stream)
    else:
        binding.proj_run_config(layer, x, m, out, cfg, stream)
    torch.cuda.synchronize()
    return out_to_f64(out)


def compare(layer, got, w, xs, rows=None):
    """Check `got` against the oracle with every rule of oracle.check (norms,
    probe rows, per-element bound); `rows` restricts the comparison to sampled
    token rows. Every output, sampled or not, must be finite."""
    if not np.all(np.isfinite(got)):
        bad = np.argwhere(~np.isfinite(got))
        raise AssertionError("%s: %d non-finite outputs, first at %s" % (layer, len(bad), tuple(bad[0])))
    K = w.shape[1]
    if rows is None:
        ref = oracle.reference(layer, xs.bits, w)
        mag = oracle.magnitude(layer, xs.bits, w)
        probe_rows = xs.probe_rows
        g = got
    else:
        rows = np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
        ref = oracle.reference_rows(layer, xs.bits, w, rows)
        mag = oracle.magnitude_rows(layer, xs.bits, w, rows)
        pos = {int(r): i for i, r in enumerate(rows)}
        probe_rows = [pos[r] for r in xs.probe_rows if r in pos]
        g = got[rows]
    return check(layer, g, ref, probe_rows, mag=mag, K=K)


def sample_rows(xs, m, n_random=16, seed=0):
    rng = np.random.default_rng(seed + m)
    rows = set(xs.probe_rows)
    rows.update(int(r) for r in rng.choice(m, size=min(n_random, m), replace=False))
    rows.update({0, m - 1})
    return sorted(rows)
