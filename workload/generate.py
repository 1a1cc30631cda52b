"""Seeded input generators (numpy PCG64).

Recipe (the pages leave the judge's generator unstated, guide ch. 1 §1.1 says
only that the weights are generated once; the readings below are the plain
ones that the rest of the pages support):

* W: i.i.d. N(0, 1) float32 scaled by 1/sqrt(K) (read as the standard
  deviation), then rounded to BF16 with round-to-nearest-even. The router keeps
  the float32 values (guide ch. 1 §1.1: router weights are FP32).
* x: i.i.d. N(0, 1) float32, rounded to BF16 (RNE).
* Probe rows (guide ch. 1 §1.5): about one row in eight holds a single nonzero
  entry, a power of two 2^e with e uniform in {-3..3}, at a uniform column k.
  For m >= 8 that is m // 8 rows picked by a seeded permutation; for
  1 < m < 8 one row; for m == 1 none unless a probe variant is asked for, in
  which case the single row is the probe.
* Outliers (the pages' sweeps mix normal and outlier inputs, report
  "What was built"/Method): when asked, 1 % of the entries outside probe rows,
  chosen uniformly without replacement, are multiplied by 64 before rounding
  (a power of two, so the scaling itself is exact).

Random numbers are drawn here only; nothing in this module computes a
projection.
"""

from dataclasses import dataclass, field

import numpy as np

from .shapes import LAYER_ID, SHAPES, ROUTER

# Distinct stream tags keep weight and activation streams apart for equal seeds.
_W_TAG = 0x57
_X_TAG = 0x58


def bf16_bits_from_f32(a):
    """Round float32 values to BF16 (round to nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def f32_from_bf16_bits(b):
    """Widen BF16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_weight(layer, seed=0):
    """Weight matrix of `layer` as handed to prepare: N x K row-major.

    Returns uint16 BF16 bits for the BF16 layers and float32 for the router.
    """
    n, k = SHAPES[layer]
    rng = np.random.default_rng([_W_TAG, int(seed), LAYER_ID[layer]])
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(k))
    if layer == ROUTER:
        return w
    return bf16_bits_from_f32(w)


@dataclass
class XSample:
    """One activation batch: BF16 bits (m x K) and where its probe rows are."""

    bits: np.ndarray
    probes: list = field(default_factory=list)  # (row, k, e): x[row, k] = 2**e, rest of row 0

    @property
    def probe_rows(self):
        return [p[0] for p in self.probes]


def _probe_count(m, probe_variant):
    if m >= 8:
        return m // 8
    if m > 1:
        return 1
    return 1 if probe_variant else 0


def make_x(layer, m, seed=0, outliers=False, probe_variant=False, probes=True):
    """Activation batch for `layer` at `m` tokens.

    `seed` selects the stream together with (layer, m, outliers, probe_variant);
    `probes=False` gives a batch with no probe rows at all.
    """
    _, k = SHAPES[layer]
    rng = np.random.default_rng(
        [_X_TAG, int(seed), LAYER_ID[layer], int(m), int(outliers), int(probe_variant)]
    )
    x = rng.standard_normal((m, k), dtype=np.float32)
    n_probe = _probe_count(m, probe_variant) if probes else 0
    probe_rows = rng.permutation(m)[:n_probe] if n_probe else np.zeros(0, dtype=np.int64)
    probes_out = []
    for r in sorted(int(v) for v in probe_rows):
        kk = int(rng.integers(0, k))
        e = int(rng.integers(-3, 4))
        x[r, :] = 0.0
        x[r, kk] = np.float32(2.0 ** e)
        probes_out.append((r, kk, e))
    if outliers:
        mask = np.ones(m, dtype=bool)
        mask[[p[0] for p in probes_out]] = False
        rows = np.nonzero(mask)[0]
        n_cand = rows.size * k
        n_out = int(round(0.01 * n_cand))
        if n_out:
            flat = rng.choice(n_cand, size=n_out, replace=False)
            rr = rows[flat // k]
            cc = flat % k
            x[rr, cc] *= np.float32(64.0)
    return XSample(bits=bf16_bits_from_f32(x), probes=probes_out)
