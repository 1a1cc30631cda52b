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
"""

from dataclasses import dataclass, field

import numpy as np

TAU_BF16 = 1e-2
TAU_ROUTER = 1e-4
PROBE_TOL = 1e-3
ROW_FACTOR = 5.0


def tau_for(layer):
    return TAU_ROUTER if layer == "router" else TAU_BF16


@dataclass
class CheckResult:
    ok: bool
    rel_l2: float
    worst_row: int
    worst_row_err: float
    probe_max_err: float
    reasons: list = field(default_factory=list)

    def __str__(self):
        return ("ok" if self.ok else "FAIL(" + "; ".join(self.reasons) + ")") + (
            " rel_l2=%.3e worst_row=%d err=%.3e probe_max=%.3e"
            % (self.rel_l2, self.worst_row, self.worst_row_err, self.probe_max_err)
        )


def _row_errors(got, ref):
    diff = np.linalg.norm(got - ref, axis=1)
    norm = np.linalg.norm(ref, axis=1)
    err = np.empty_like(diff)
    nz = norm > 0
    err[nz] = diff[nz] / norm[nz]
    err[~nz] = np.where(diff[~nz] == 0, 0.0, np.inf)
    return err


def check(layer, got, ref, probe_rows=(), tau=None):
    """Apply the acceptance rules. `got` may be any float array; it is widened to FP64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        return CheckResult(False, np.inf, -1, np.inf, np.inf,
                           ["shape %s != %s" % (got.shape, ref.shape)])
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
    return CheckResult(not reasons, float(rel), worst, float(rows[worst]), probe_max, reasons)
