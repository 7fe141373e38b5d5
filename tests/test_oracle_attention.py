"""Pins of the GQA decode attention oracle (oracle/attention.py), on the CPU.

Each check is fixed by the mathematics of softmax attention, not by the
oracle's code: a single visible key returns its value; equal keys average
the visible values; the 1/sqrt(d) scale against a hand-computed two-key
case; the query-head to KV-head grouping (h // g); the causal limit of each
verify row; value affinity (weights sum to one); invariance under a
permutation of the visible positions; and rows of a verify call equal
one-row calls at their positions.
"""

import math

import numpy as np
import pytest

from oracle.attention import gqa_decode


def _rand(rng, *shape):
    return rng.normal(size=shape)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(0)
    q = _rand(rng, 1, 4, 8)
    k = _rand(rng, 2, 5, 8)
    v = _rand(rng, 2, 5, 8)
    o = gqa_decode(q, k, v, p0=0)
    assert np.array_equal(o[0, :2], np.broadcast_to(v[0, 0], (2, 8)))
    assert np.array_equal(o[0, 2:], np.broadcast_to(v[1, 0], (2, 8)))


def test_equal_keys_average_visible_values():
    rng = np.random.default_rng(1)
    q = _rand(rng, 2, 2, 4)
    k = np.broadcast_to(_rand(rng, 1, 1, 4), (1, 6, 4)).copy()
    v = _rand(rng, 1, 6, 4)
    o = gqa_decode(q, k, v, p0=2)
    assert np.allclose(o[0, 0], v[0, :3].mean(axis=0), rtol=1e-13, atol=1e-15)
    assert np.allclose(o[1, 1], v[0, :4].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_scale_two_keys_by_hand():
    d = 16
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 2.0
    k = np.zeros((1, 2, d))
    k[0, 0, 0], k[0, 1, 0] = 3.0, 1.0
    v = np.zeros((1, 2, d))
    v[0, 0, 1], v[0, 1, 1] = 1.0, -1.0
    o = gqa_decode(q, k, v, p0=1)
    s0, s1 = 2 * 3 / 4.0, 2 * 1 / 4.0  # scores / sqrt(16)
    w0 = math.exp(s0) / (math.exp(s0) + math.exp(s1))
    assert o[0, 0, 1] == pytest.approx(w0 - (1 - w0), rel=1e-14)
    assert np.all(o[0, 0, [0] + list(range(2, d))] == 0)


def test_query_heads_use_their_group_kv_head():
    rng = np.random.default_rng(2)
    n_kv, g, d, s = 2, 8, 8, 7
    q = _rand(rng, 1, n_kv * g, d)
    k = _rand(rng, n_kv, s, d)
    v = np.stack([np.zeros((s, d)), np.ones((s, d))])
    o = gqa_decode(q, k, v, p0=s - 1)
    assert np.allclose(o[0, :g], 0.0) and np.allclose(o[0, g:], 1.0, rtol=1e-14)


def test_causal_limit_of_verify_rows():
    rng = np.random.default_rng(3)
    d = 8
    q = np.abs(_rand(rng, 3, 1, d))
    k = 0.1 * _rand(rng, 1, 10, d)
    v = 0.1 * _rand(rng, 1, 10, d)
    k[0, 9] = 50.0  # the last verify row's own key dominates its scores
    v[0, 9] = 100.0
    o = gqa_decode(q, k, v, p0=7)
    assert np.abs(o[:2]).max() < 1.0  # rows at positions 7 and 8 cannot see position 9
    assert np.all(o[2, 0] > 99.0)


def test_values_affine_and_positions_permutable():
    rng = np.random.default_rng(4)
    q = _rand(rng, 1, 4, 8)
    k = _rand(rng, 2, 9, 8)
    v = _rand(rng, 2, 9, 8)
    o = gqa_decode(q, k, v, p0=8)
    c = _rand(rng, 8)
    assert np.allclose(gqa_decode(q, k, 3.0 * v + c, p0=8), 3.0 * o + c, rtol=1e-12, atol=1e-12)
    perm = rng.permutation(9)
    assert np.allclose(gqa_decode(q, k[:, perm], v[:, perm], p0=8), o, rtol=1e-12, atol=1e-13)


def test_verify_rows_equal_one_row_calls():
    rng = np.random.default_rng(5)
    q = _rand(rng, 3, 4, 8)
    k = _rand(rng, 2, 12, 8)
    v = _rand(rng, 2, 12, 8)
    o = gqa_decode(q, k, v, p0=6)
    for i in range(3):
        assert np.array_equal(o[i], gqa_decode(q[i:i + 1], k, v, p0=6 + i)[0])
