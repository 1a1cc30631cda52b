"""Acceptance check of a computed output against the FP64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Rules (guide ch. 1 "The problem, the judge and the speed of light", §1.5):
* global relative L2 error against the FP64 reference <= tau, with tau = 1e-2
  for the BF16 layers and 1e-4 for the router;
* probe rows (one power-of-two nonzero in the x row) match within 0.1 %;
* no row is off by more than 5 x tau;
* no NaN or Inf anywhere.

Readings where the page leaves the norm open:
* "match within 0.1 %" is a per-row relative L2 error <= 1e-3, the same norm
  as the other bounds; the router's probe rows also meet its 5 x tau row rule;
* a row whose reference is exactly zero must be exactly zero.

Per-element rule (a reading: the page's norms alone let a few wrong outputs of
a long row pass). The notebook's note "Numerical formats and error" fixes the
arithmetic: BF16 operands, products summed in FP32, the summation order free,
the BF16 layers' outputs rounded to BF16. For any such result g of an output
whose exact value is r,

    |g - r| <= u_out * |r| + (1 + u_out) * (gamma_n * S + 2^-133),

with S = sum over the terms of |x * w| (oracle.magnitude), n the number of
terms (the K products; 3 K for the router, whose FP32 weights enter as three
exact BF16 parts; 16 more for the 12-bit form's corrections, two per slot),
gamma_n = n u / (1 - n u) the classic bound of an n-term floating-point sum in
any order (u = 2^-23: twice FP32's unit roundoff, so that an adder that does
not round to nearest is covered too), u_out = 2^-8 the relative error of
rounding to BF16's 8-bit significand (0 for the router's FP32 output), and
2^-133 half of the smallest BF16 subnormal. Every correct result passes it;
a wrong output that is off by more than that bound fails, however long its
row.
"""

from dataclasses import dataclass, field

import numpy as np

TAU_BF16 = 1e-2
TAU_ROUTER = 1e-4
PROBE_TOL = 1e-3
ROW_FACTOR = 5.0

ACC_UNIT = 2.0 ** -23        # per-addition relative error allowed for the FP32 sum
BF16_OUT_UNIT = 2.0 ** -8    # round to nearest with an 8-bit significand
ABS_FLOOR = 2.0 ** -133      # half the smallest BF16 subnormal
CORRECTION_TERMS = 16        # 12-bit form: up to 8 slots per row, two products each


def tau_for(layer):
    return TAU_ROUTER if layer == "router" else TAU_BF16


def n_terms(layer, K):
    """Products an output of `layer` sums (see the per-element rule above)."""
    return 3 * K if layer == "router" else K + CORRECTION_TERMS


def element_bound(layer, ref, mag, K):
    """Largest |got - ref| the per-element rule accepts, elementwise."""
    n = n_terms(layer, K)
    gamma = n * ACC_UNIT / (1.0 - n * ACC_UNIT)
    u_out = 0.0 if layer == "router" else BF16_OUT_UNIT
    return u_out * np.abs(ref) + (1.0 + u_out) * (gamma * mag + ABS_FLOOR)


@dataclass
class CheckResult:
    ok: bool
    rel_l2: float
    worst_row: int
    worst_row_err: float
    probe_max_err: float
    reasons: list = field(default_factory=list)
    elem_worst: float = float("nan")   # largest |got - ref| / element bound (nan: rule not applied)

    def __str__(self):
        return ("ok" if self.ok else "FAIL(" + "; ".join(self.reasons) + ")") + (
            " rel_l2=%.3e worst_row=%d err=%.3e probe_max=%.3e elem_worst=%.3g"
            % (self.rel_l2, self.worst_row, self.worst_row_err, self.probe_max_err, self.elem_worst)
        )


def _row_errors(got, ref):
    diff = np.linalg.norm(got - ref, axis=1)
    norm = np.linalg.norm(ref, axis=1)
    err = np.empty_like(diff)
    nz = norm > 0
    err[nz] = diff[nz] / norm[nz]
    err[~nz] = np.where(diff[~nz] == 0, 0.0, np.inf)
    return err


def check(layer, got, ref, probe_rows=(), tau=None, mag=None, K=None):
    """Apply the acceptance rules. `got` may be any float array; it is widened to FP64.

    `mag` (oracle.magnitude of the same outputs) and `K` (the layer's
    contraction length) turn on the per-element rule; both or neither.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        return CheckResult(False, np.inf, -1, np.inf, np.inf,
                           ["shape %s != %s" % (got.shape, ref.shape)])
    if (mag is None) != (K is None):
        raise ValueError("the per-element rule needs both mag and K")
    if mag is not None:
        mag = np.asarray(mag, dtype=np.float64)
        if mag.shape != ref.shape:
            raise ValueError("mag shape %s != ref shape %s" % (mag.shape, ref.shape))
    tau = tau_for(layer) if tau is None else tau
    reasons = []
    if not np.all(np.isfinite(got)):
        reasons.append("NaN/Inf in output")
        return CheckResult(False, np.inf, -1, np.inf, np.inf, reasons)
    if got.size == 0:
        return CheckResult(True, 0.0, -1, 0.0, 0.0, reasons)
    rnorm = np.linalg.norm(ref)
    dnorm = np.linalg.norm(got - ref)
    rel = dnorm / rnorm if rnorm > 0 else (0.0 if dnorm == 0 else np.inf)
    if not rel <= tau:
        reasons.append("global rel L2 %.3e > %.1e" % (rel, tau))
    rows = _row_errors(got, ref)
    worst = int(np.argmax(rows))
    if not rows[worst] <= ROW_FACTOR * tau:
        reasons.append("row %d rel L2 %.3e > %.1e" % (worst, rows[worst], ROW_FACTOR * tau))
    probe_max = 0.0
    for r in probe_rows:
        e = float(rows[int(r)])
        probe_max = max(probe_max, e)
        if not e <= PROBE_TOL:
            reasons.append("probe row %d rel L2 %.3e > %.1e" % (r, e, PROBE_TOL))
    elem_worst = float("nan")
    if mag is not None:
        ratio = np.abs(got - ref) / element_bound(layer, ref, mag, K)
        elem_worst = float(ratio.max())
        if not elem_worst <= 1.0:
            bad = np.argwhere(ratio > 1.0)
            i, j = (int(v) for v in bad[0])
            reasons.append("%d outputs outside the element bound, first at (%d, %d): got %.9g ref %.9g"
                           % (len(bad), i, j, got[i, j], ref[i, j]))
    return CheckResult(not reasons, float(rel), worst, float(rows[worst]), probe_max, reasons, elem_worst)
