"""Negative and positive controls of the acceptance check (guide ch. 1 §1.5).

The check must bite where the page says it bites: a BF16 router, weights with a
dropped mantissa bit (probe rows catch them while the global norm passes), one
bad row among good ones, a NaN.
"""

import numpy as np
import pytest

import oracle
from oracle.check import check, element_bound, TAU_BF16, TAU_ROUTER
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


def _fp32_sums(xb, w, order):
    """out = x @ W^T summed in FP32 in a given order (a correct GPU-like result).

    Products of BF16 activations with BF16 weights are exact in FP32; FP32
    router weights are first split into three BF16 parts (hi + mid + lo == w
    exactly), whose products are exact too.
    """
    xf = f32_from_bf16_bits(xb)
    if w.dtype == np.uint16:
        parts = [f32_from_bf16_bits(w)]
    else:
        u = w.view(np.uint32)
        hi = (u & np.uint32(0xFFFF0000)).view(np.float32)
        r1 = w - hi
        mid = (r1.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        lo = r1 - mid
        assert np.array_equal(hi.astype(np.float64) + mid + lo, w.astype(np.float64))
        parts = [hi, mid, lo]
    terms = np.concatenate([xf[:, None, :] * p[None, :, :] for p in parts], axis=2)   # exact in FP32
    if order == "reverse":
        terms = terms[:, :, ::-1]
    if order in ("sequential", "reverse"):
        return np.cumsum(terms, axis=2, dtype=np.float32)[:, :, -1]
    if order == "blocked":     # 32-term blocks, then a chain over the blocks
        n = terms.shape[2]
        pad = (-n) % 32
        t = np.concatenate([terms, np.zeros(terms.shape[:2] + (pad,), np.float32)], axis=2)
        blocks = t.reshape(t.shape[0], t.shape[1], -1, 32).sum(axis=3, dtype=np.float32)
        return np.cumsum(blocks, axis=2, dtype=np.float32)[:, :, -1]
    return terms.sum(axis=2, dtype=np.float32)    # numpy's pairwise sum


def _bf16_out(a32):
    return f32_from_bf16_bits(bf16_bits_from_f32(a32)).astype(np.float64)


@pytest.mark.parametrize("layer", ["o", "router"])
@pytest.mark.parametrize("order", ["sequential", "reverse", "blocked", "pairwise"])
def test_fp32_accumulation_in_any_order_passes_element_rule(oracle_mod, layer, order):
    w = make_weight(layer, seed=1)
    if layer == "router":
        w = w[:24]
    else:
        w = w[:96]
    xs = make_x(layer, 8, seed=2, outliers=True)
    K = w.shape[1]
    ref = oracle.matmul_bits(xs.bits, w)
    mag = oracle.magnitude_bits(xs.bits, w)
    s32 = _fp32_sums(xs.bits, w, order)
    got = s32.astype(np.float64) if layer == "router" else _bf16_out(s32)
    r = check(layer, got, ref, xs.probe_rows, mag=mag, K=K)
    assert r.ok, r
    if layer == "router":
        # FP32 output: only the sum's error counts, far below its worst case.
        assert r.elem_worst < 0.05, r


def test_few_wrong_outputs_in_a_long_row_fail_only_the_element_rule(oracle_mod):
    # A 256 x 8192 BF16 result (layer o, 256 tokens) with three wrong outputs in
    # one row: the global and per-row L2 rules pass it, the element rule does not.
    w = make_weight("o", seed=0)
    xs = make_x("o", 256, seed=5, outliers=True)
    ref = oracle.reference("o", xs.bits, w)
    mag = oracle.magnitude("o", xs.bits, w)
    good = _bf16_round(ref)
    assert check("o", good, ref, xs.probe_rows, mag=mag, K=1024).ok
    row = next(i for i in range(256) if i not in xs.probe_rows)
    cols = np.argsort(-np.abs(ref[row]))[[2000, 3000, 4000]]   # outputs of middling size
    bad = good.copy()
    bad[row, cols[0]] = 0.0                             # an unwritten-as-zero output
    bad[row, cols[1]] = -good[row, cols[1]]             # a sign slip
    bad[row, cols[2]] = good[row, (cols[2] + 16) % 8192]   # an output from the wrong column
    norms_only = check("o", bad, ref, xs.probe_rows)
    assert norms_only.ok, norms_only                     # what the norms alone miss
    r = check("o", bad, ref, xs.probe_rows, mag=mag, K=1024)
    assert not r.ok and "element bound" in r.reasons[-1], r
    ratio = np.abs(bad - ref) / element_bound("o", ref, mag, 1024)
    assert set(map(tuple, np.argwhere(ratio > 1))) == {(row, int(c)) for c in cols}


def test_element_rule_needs_both_inputs():
    ref = np.ones((2, 4))
    with pytest.raises(ValueError):
        check("o", ref, ref, mag=np.ones((2, 4)))
    with pytest.raises(ValueError):
        check("o", ref, ref, mag=np.ones((2, 3)), K=4)
