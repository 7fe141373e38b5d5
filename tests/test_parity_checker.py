"""CPU tests of the GPU-vs-oracle comparison (tests/parity.py) itself.

The checker must pass the oracle's own correctly rounded output and catch each
kind of mistake a GPU path could make: a wrong or reordered expert id, a
weight error of a few parts per million, and a single output element one ulp
off away from a rounding midpoint. Mistakes are planted in copies of the
oracle's results, on the CPU.
"""

import numpy as np

from oracle import gen as ogen
from oracle.moe import layer_forward
from tests.parity import check_layer, oracle_shape, ulp_check

KW = dict(hidden=256, n_experts=16, inter=128, top_k=3, shared_inter=128, router_bits=8, expert_bits=4,
          shared_bits=6, rms_eps=1e-6)


def _ref(T=3, seed=7):
    lw = ogen.GeneratedLayer(oracle_shape(KW), 0, 0)
    x = ogen.gen_x(seed, T, KW["hidden"])
    return layer_forward(lw, x)


def test_correct_rounding_passes():
    ref = _ref()
    y = ogen.f64_to_bf16_bits(ref["y"])
    r = check_layer(y, ref["ids"].copy(), ref["w"].astype(np.float32), ref)
    assert r.ok and r.ulp_bad == 0 and r.max_w_err < 1e-7, r


def test_wrong_id_fails():
    ref = _ref()
    ids = ref["ids"].copy()
    ids[1, 0] = [e for e in range(16) if e not in ids[1]][0]
    r = check_layer(ogen.f64_to_bf16_bits(ref["y"]), ids, ref["w"].astype(np.float32), ref)
    if ref["gap"][1] >= 1e-5:
        assert not r.ok and r.id_mismatch == [1]


def test_swapped_order_fails():
    ref = _ref()
    ids = ref["ids"].copy()
    w = ref["w"].astype(np.float32)
    t = 0
    lam = ref["logits"][t]
    assert abs(lam[ids[t, 0]] - lam[ids[t, 1]]) > 1e-5
    ids[t, [0, 1]] = ids[t, [1, 0]]
    w[t, [0, 1]] = w[t, [1, 0]]
    r = check_layer(ogen.f64_to_bf16_bits(ref["y"]), ids, w, ref)
    assert not r.ok and r.id_mismatch == [0]


def test_weight_error_fails():
    ref = _ref()
    w = ref["w"].astype(np.float32)
    w[2, 1] += 5e-6
    r = check_layer(ogen.f64_to_bf16_bits(ref["y"]), ref["ids"].copy(), w, ref)
    assert not r.ok and r.max_w_err > 4e-6


def test_one_ulp_off_midpoint_fails():
    ref = _ref()
    y = ogen.f64_to_bf16_bits(ref["y"])
    yr = ref["y"]
    # an element far from a rounding midpoint: y_ref close to its own bf16 value
    lo = ogen.bf16_bits_to_f64(y)
    dist = np.abs(yr - lo) / np.maximum(np.abs(yr), 1e-30)
    t, j = np.unravel_index(np.argmin(dist + (np.abs(yr) < 0.5)), yr.shape)
    bad = y.copy()
    bad[t, j] = bad[t, j] + 1  # next pattern: one ulp away in magnitude
    nbad, noff, nmax, _ = ulp_check(bad, yr)
    assert nbad == 1 and noff == 1 and nmax == 1
    r = check_layer(bad, ref["ids"].copy(), ref["w"].astype(np.float32), ref)
    assert not r.ok and r.ulp_bad == 1
    # the max-error bound alone would not have seen it
    assert r.ratio <= 4e-3


def test_tiny_elements_allow_the_absolute_budget():
    # y = h + moe cancelling to ~1e-5 next to elements of size 3: a few ulps of the small
    # element are within 2e-6 * max|y| and pass; an error of 1e-5 absolute does not
    yr = np.array([[2.0146e-5, 3.0, -1.5]])
    base = ogen.f64_to_bf16_bits(yr)
    y = base.copy()
    y[0, 0] = ogen.f64_to_bf16_bits(np.array([2.0146e-5 + 4e-7]))[0]
    assert ulp_check(y, yr)[0] == 0 and ulp_check(y, yr)[2] >= 2
    y[0, 0] = ogen.f64_to_bf16_bits(np.array([2.0146e-5 + 1e-5]))[0]
    assert ulp_check(y, yr)[0] == 1


def test_one_ulp_at_midpoint_allowed():
    # y_ref exactly halfway between two bf16 values (1 and 1 + 2^-7): either neighbour passes
    yr = np.array([[1.0 + 2.0**-8, 2.0, -3.0]])
    base = ogen.f64_to_bf16_bits(yr)
    for v in (0x3F80, 0x3F81):
        y = base.copy()
        y[0, 0] = v
        assert ulp_check(y, yr)[0] == 0
    y = base.copy()
    y[0, 0] = 0x3F82  # two ulps away
    assert ulp_check(y, yr)[0] == 1
