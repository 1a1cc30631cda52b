"""Negative and positive controls of the acceptance check (guide ch. 1 §1.5).

The check must bite where the page says it bites: a BF16 router, weights with a
dropped mantissa bit (probe rows catch them while the global norm passes), one
bad row among good ones, a NaN.
"""

import numpy as np

import oracle
from oracle.check import check, TAU_BF16, TAU_ROUTER
from workload import make_weight, make_x, bf16_bits_from_f32, f32_from_bf16_bits


def _bf16_round(a):
    return f32_from_bf16_bits(bf16_bits_from_f32(np.asarray(a, np.float32))).astype(np.float64)


def test_exact_and_bf16_rounded_results_pass(oracle_mod):
    w = make_weight("o", seed=0)
    xs = make_x("o", 32, seed=1, outliers=True)
    ref = oracle.reference("o", xs.bits, w)
    assert check("o", ref, ref, xs.probe_rows).ok
    r = check("o", _bf16_round(ref), ref, xs.probe_rows)
    assert r.ok, r
    assert r.probe_max_err == 0.0  # probe outputs are BF16 weights times 2^e: exact in BF16


def test_router_with_bf16_weights_fails(oracle_mod):
    # "rules out ... plain BF16 for the router" (guide ch. 1 §1.5).
    w = make_weight("router", seed=0)
    xs = make_x("router", 16, seed=1)
    ref = oracle.reference("router", xs.bits, w)
    wb = bf16_bits_from_f32(w)
    bad = oracle.matmul_bits(xs.bits, wb)
    r = check("router", bad, ref, xs.probe_rows)
    assert not r.ok and r.rel_l2 > TAU_ROUTER
    # ...while the same result would pass the BF16 layers' 1 % bound.
    assert r.rel_l2 < TAU_BF16


def test_dropped_mantissa_bit_fails_only_on_probe_rows(oracle_mod):
    # Lossy weights: clear the lowest mantissa bit. The global error stays under
    # 1 %, but probe rows expose the weight column itself.
    w = make_weight("qkv_gate", seed=2)
    xs = make_x("qkv_gate", 16, seed=3)
    assert len(xs.probes) == 2
    ref = oracle.reference("qkv_gate", xs.bits, w)
    lossy = w & np.uint16(0xFFFE)
    got = oracle.matmul_bits(xs.bits, lossy)
    r = check("qkv_gate", got, ref, xs.probe_rows)
    assert r.rel_l2 < TAU_BF16
    assert not r.ok
    assert all("probe" in s for s in r.reasons)


def test_single_bad_row_fails_per_row_rule():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((200, 64))
    got = ref.copy()
    got[17] *= 1.08  # row off by 8 %: more than 5 x 1 %
    r = check("pooler", got, ref)
    assert r.rel_l2 < TAU_BF16
    assert not r.ok and r.worst_row == 17


def test_nan_and_inf_fail():
    ref = np.ones((2, 4))
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[1, 2] = bad
        assert not check("o", got, ref).ok


def test_zero_reference_row_requires_zero():
    ref = np.zeros((1, 8))
    assert check("o", np.zeros((1, 8)), ref).ok
    got = np.zeros((1, 8))
    got[0, 3] = 1e-30
    assert not check("o", got, ref).ok


def test_shape_mismatch_fails():
    assert not check("o", np.zeros((2, 3)), np.zeros((3, 2))).ok
