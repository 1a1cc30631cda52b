"""Algorithmic bytes, FLOPs and the nominal floor of one projection call.

The floor is the slower of moving the bytes at the memory bandwidth and doing
the FLOPs at the arithmetic peak (guide ch. 1 "The problem, the judge and the
speed of light", §1.7): bytes = W + x + out, FLOPs = 2 m N K, with the
unpooler's 1024-row slice at <= 8 tokens and FP32 router weights and output
(§1.1). The same formula with the H200 constants of §1.7 reproduces the
floor column of §1.8's per-load table.

Algorithmic bytes count each operand once: no scratch, no partial sums, no
re-reads. They are the numerator of every achieved-bandwidth figure.
"""

from .layers import DIMS, LAYERS, layer_name, n_eff

# MI355X published peaks.
MI355X_HBM_BPS = 8.0e12
MI355X_BF16_FLOPS = 2.5e15
MI355X_FP32_FLOPS = 157.3e12

# H200 constants the pages use for their floors (guide ch. 1 §1.7).
H200_HBM_BPS = 4.8e12
H200_BF16_FLOPS = 989e12


def bytes_of(layer, m):
    """Algorithmic bytes of one call: W rows read + x + out."""
    name = layer_name(layer)
    n, k, wb, ob = DIMS[name]
    ne = n_eff(name, m)
    return ne * k * wb + m * k * 2 + m * ne * ob


def weight_bytes(layer, m):
    name = layer_name(layer)
    n, k, wb, _ = DIMS[name]
    return n_eff(name, m) * k * wb


def flops_of(layer, m):
    name = layer_name(layer)
    _, k, _, _ = DIMS[name]
    return 2 * m * n_eff(name, m) * k


def floor_us(layer, m, bw=MI355X_HBM_BPS, peak=MI355X_BF16_FLOPS, router_peak=None):
    """Nominal floor in microseconds. `router_peak` overrides `peak` for the router."""
    name = layer_name(layer)
    p = router_peak if (name == "router" and router_peak is not None) else peak
    return max(bytes_of(name, m) / bw, flops_of(name, m) / p) * 1e6


def load_floor_us(m, **kw):
    """Sum of the five layers' floors for one load (guide ch. 1 §1.3: load time is a sum)."""
    return sum(floor_us(name, m, **kw) for name in LAYERS)
