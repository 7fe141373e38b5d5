"""Pins for the oracle's method (CPU only).

What pins each function (none of these re-types the function under test):

* dequant: exact rational arithmetic of the group-affine identity
  ``sum_j (q_j s + b) x_j = s sum_j q_j x_j + b sum_j x_j`` (the FMA
  reordering on the flash-moe news page), plus one-hot probes that expose a
  transposed operand or a wrong group index;
* rmsnorm: closed forms (constant rows, zero rows, scale invariance);
* route: brute force over every k-subset on tiny E, the softmax restricted to
  the selection computed independently, tie and degenerate cases;
* expert_ffn: a hand-computed one-unit expert and SwiGLU's asymmetry in
  gate vs up;
* layer_forward / stack_forward: invariants that must hold for any correct
  implementation (identical experts make the router irrelevant, a one-hot
  router reproduces one expert, expert permutation, zero input, zero down
  projections make every layer the identity).
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import gen
from oracle.gen import ExplicitLayer, GeneratedLayer, MoEShape
from oracle.moe import dequant, expert_ffn, layer_forward, rmsnorm, route, shared_gate, silu, stack_forward

TINY = MoEShape(hidden=256, n_experts=16, inter=128, top_k=2, shared_inter=128,
                router_bits=16, expert_bits=4, shared_bits=4)


# ------------------------------------------------------------------ dequant
def test_dequant_matches_exact_rational_group_identity():
    rng = np.random.default_rng(1)
    rows, k = 3, 192
    for bits in (2, 3, 4, 6, 8):
        codes = rng.integers(0, 2**bits, size=(rows, k)).astype(np.uint8)
        s = gen.bf16_round(rng.uniform(0.001, 0.01, size=(rows, k // 64)))
        b = gen.bf16_round(-s * (2**bits - 1) / 2 + rng.normal(0, 0.001, size=s.shape))
        x = gen.bf16_round(rng.normal(size=k))
        y = dequant(codes, s, b) @ x
        for i in range(rows):
            exact = Fraction(0)
            for g in range(k // 64):
                sl = slice(64 * g, 64 * g + 64)
                sq = sum(Fraction(int(q)) * Fraction(float(v)) for q, v in zip(codes[i, sl], x[sl]))
                sx = sum(Fraction(float(v)) for v in x[sl])
                exact += Fraction(float(s[i, g])) * sq + Fraction(float(b[i, g])) * sx
            assert abs(y[i] - float(exact)) <= 1e-13 * max(1.0, abs(float(exact)))


def test_dequant_entries_exact_and_indexed_by_row_and_group():
    rows, k = 4, 128
    codes = np.zeros((rows, k), dtype=np.uint8)
    codes[2, 70] = 9  # row 2, column 70 -> group 1
    s = np.zeros((rows, 2))
    b = np.zeros((rows, 2))
    s[2, 1] = 0.25
    b[2, 1] = -0.5
    w = dequant(codes, s, b)
    # group 1 of row 2: every entry is b except column 70
    assert w[2, 70] == 9 * 0.25 - 0.5
    assert np.all(w[2, 64:70] == -0.5) and np.all(w[2, 71:128] == -0.5)
    assert np.all(w[2, :64] == 0.0)
    assert np.all(w[[0, 1, 3]] == 0.0)
    x = np.zeros(k)
    x[70] = 1.0
    y = w @ x
    assert np.array_equal(y, np.array([0.0, 0.0, 1.75, 0.0]))


# ------------------------------------------------------------------ rmsnorm
def test_rmsnorm_closed_forms():
    c = 3.0
    u = rmsnorm(np.full(64, c), eps=1e-6)
    assert np.allclose(u, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    assert np.all(rmsnorm(np.zeros(32)) == 0.0)
    rng = np.random.default_rng(2)
    h = rng.normal(size=256)
    u1 = rmsnorm(h, eps=0.0)
    assert abs(np.mean(u1 * u1) - 1.0) < 1e-14
    assert np.allclose(rmsnorm(7.5 * h, eps=0.0), u1, rtol=1e-14)
    # eps enters as mean(h^2) + eps
    h2 = np.array([1.0, -1.0, 1.0, -1.0])
    assert np.allclose(rmsnorm(h2, eps=3.0), h2 / 2.0, rtol=1e-15)


# -------------------------------------------------------------------- route
def test_route_matches_brute_force_subsets():
    rng = np.random.default_rng(3)
    e, k = 8, 3
    for _ in range(50):
        lam = rng.normal(size=e)
        ids, w, gap = route(lam, k)
        best = max(itertools.combinations(range(e), k), key=lambda c: sum(lam[list(c)]))
        assert set(ids.tolist()) == set(best)
        assert np.all(np.diff(lam[ids]) < 0)  # descending
        # weights: softmax over the selected logits alone
        sel = lam[ids]
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.allclose(w, ref, rtol=1e-14, atol=0)
        assert abs(w.sum() - 1.0) < 1e-15
        rest = np.sort(np.delete(lam, ids))[::-1]
        assert gap == pytest.approx(sel.min() - rest[0], abs=0)


def test_route_ties_and_degenerate_cases():
    ids, w, gap = route(np.zeros(16), 4)
    assert ids.tolist() == [0, 1, 2, 3]
    assert np.all(w == 0.25)
    assert gap == 0.0
    lam = np.array([0.5, 2.0, 0.5, 2.0, -1.0])
    ids, w, _ = route(lam, 3)
    assert ids.tolist() == [1, 3, 0]  # equal logits: lower index first
    ids, w, gap = route(np.array([0.1, 0.9, 0.3]), 1)
    assert ids.tolist() == [1] and w.tolist() == [1.0]
    assert gap == pytest.approx(0.6, abs=1e-15)
    ids, w, gap = route(np.array([1.0, 2.0]), 2)
    assert ids.tolist() == [1, 0] and gap == math.inf
    assert w[0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    # shift invariance of the weights
    lam = np.array([3.0, 1.0, 2.0, 0.0])
    assert np.allclose(route(lam, 2)[1], route(lam + 100.0, 2)[1], rtol=1e-13)


# ------------------------------------------------------------------- expert
def test_expert_ffn_one_unit_hand_computed():
    wg = np.array([[1.0, 0.0]])
    wu = np.array([[0.0, 1.0]])
    wd = np.array([[2.0], [-1.0], [0.5]])
    u = np.array([2.0, 3.0])
    a = 2.0 / (1.0 + math.exp(-2.0)) * 3.0
    assert np.allclose(expert_ffn(wg, wu, wd, u), [2 * a, -a, 0.5 * a], rtol=1e-15)
    # swapping gate and up changes the result (SwiGLU is not symmetric)
    b = 3.0 / (1.0 + math.exp(-3.0)) * 2.0
    assert np.allclose(expert_ffn(wu, wg, wd, u), [2 * b, -b, 0.5 * b], rtol=1e-15)
    assert silu(np.array([0.0]))[0] == 0.0
    assert silu(np.array([-1000.0]))[0] == 0.0
    assert silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)


def test_shared_gate_closed_forms():
    assert shared_gate(np.zeros(8), np.ones(8)) == 0.5
    assert shared_gate(np.ones(4), np.full(4, 0.5)) == pytest.approx(1 / (1 + math.exp(-2)), rel=1e-15)
    assert shared_gate(np.ones(4), np.full(4, 1e4)) == 1.0


# ------------------------------------------------------------ layer / stack
def _ffn_q(rng, inter, h, bits, scale=0.02):
    def m(r, k):
        c = rng.integers(0, 2**bits, size=(r, k)).astype(np.uint8)
        s = gen.bf16_round(rng.uniform(0.5, 1.5, size=(r, k // 64)) * scale / 2 ** (bits - 1))
        b = gen.bf16_round(-s * (2**bits - 1) / 2)
        return c, s, b
    return {"gate": m(inter, h), "up": m(inter, h), "down": m(h, inter)}


def _zero_down(q):
    c, s, b = q["down"]
    return {"gate": q["gate"], "up": q["up"], "down": (c, np.zeros_like(s), np.zeros_like(b))}


def _explicit(shape, experts, shared, router, gatevec):
    return ExplicitLayer(shape, experts, shared, router, gatevec)


def test_layer_zero_input():
    lw = GeneratedLayer(TINY, 0, 0)
    r = layer_forward(lw, np.zeros((1, 256)))
    assert np.all(r["y"] == 0.0)
    assert r["ids"][0].tolist() == [0, 1]
    assert np.all(r["w"] == 0.5)
    assert r["sgate"][0] == 0.5


def test_layer_identical_experts_router_irrelevant():
    rng = np.random.default_rng(4)
    sh = MoEShape(hidden=128, n_experts=6, inter=64, top_k=2, shared_inter=64,
                  router_bits=16, expert_bits=4, shared_bits=8)
    one = _ffn_q(rng, 64, 128, 4)
    shared = _ffn_q(rng, 64, 128, 8)
    gv = gen.bf16_round(rng.normal(size=128) / math.sqrt(128))
    h = gen.bf16_round(rng.normal(size=(3, 128)))
    ys = []
    for seed in (10, 11):
        wr = gen.bf16_round(np.random.default_rng(seed).normal(size=(6, 128)) / math.sqrt(128))
        ys.append(layer_forward(_explicit(sh, [one] * 6, shared, ("dense", wr), gv), h)["y"])
    assert not np.array_equal(
        layer_forward(_explicit(sh, [one] * 6, shared, ("dense", wr), gv), h)["ids"], np.zeros((3, 2)))
    assert np.allclose(ys[0], ys[1], rtol=0, atol=1e-12)


def test_layer_one_hot_router_reproduces_single_expert():
    rng = np.random.default_rng(5)
    sh = MoEShape(hidden=128, n_experts=5, inter=64, top_k=1, shared_inter=64,
                  router_bits=16, expert_bits=6, shared_bits=8)
    experts = [_ffn_q(rng, 64, 128, 6) for _ in range(5)]
    shared = _ffn_q(rng, 64, 128, 8)
    gv = gen.bf16_round(rng.normal(size=128) / math.sqrt(128))
    h = gen.bf16_round(rng.normal(size=(1, 128)))
    u = rmsnorm(h[0])
    estar = 3
    wr = np.zeros((5, 128))
    wr[estar] = gen.bf16_round(np.sign(u))  # logit = |u|_1 ~ 100
    r = layer_forward(_explicit(sh, experts, shared, ("dense", wr), gv), h)
    assert r["ids"][0].tolist() == [estar] and r["w"][0].tolist() == [1.0]
    dq = lambda q: tuple(dequant(*q[m]) for m in ("gate", "up", "down"))
    expect = h[0] + expert_ffn(*dq(experts[estar]), u) + shared_gate(gv, u) * expert_ffn(*dq(shared), u)
    assert np.allclose(r["y"][0], expect, rtol=0, atol=1e-13)
    # k = 3 with the same router: e* first, then the tied zero logits by index
    sh3 = MoEShape(hidden=128, n_experts=5, inter=64, top_k=3, shared_inter=64,
                   router_bits=16, expert_bits=6, shared_bits=8)
    r3 = layer_forward(_explicit(sh3, experts, shared, ("dense", wr), gv), h)
    assert r3["ids"][0].tolist() == [estar, 0, 1]
    assert 1.0 - r3["w"][0][0] < 1e-30
    assert np.allclose(r3["y"][0], expect, rtol=0, atol=1e-12)


def test_layer_expert_permutation():
    rng = np.random.default_rng(6)
    sh = MoEShape(hidden=128, n_experts=8, inter=64, top_k=3, shared_inter=64,
                  router_bits=8, expert_bits=4, shared_bits=8)
    experts = [_ffn_q(rng, 64, 128, 4) for _ in range(8)]
    shared = _ffn_q(rng, 64, 128, 8)
    gv = gen.bf16_round(rng.normal(size=128) / math.sqrt(128))
    rq = _ffn_q(rng, 8, 128, 8, scale=0.2)["gate"]
    h = gen.bf16_round(rng.normal(size=(4, 128)))
    perm = rng.permutation(8)  # new slot j holds old expert perm[j]
    inv = np.argsort(perm)
    r0 = layer_forward(_explicit(sh, experts, shared, ("q", rq), gv), h)
    rq_p = (rq[0][perm], rq[1][perm], rq[2][perm])
    r1 = layer_forward(_explicit(sh, [experts[p] for p in perm], shared, ("q", rq_p), gv), h)
    assert np.array_equal(inv[r0["ids"]], r1["ids"])
    assert np.allclose(r0["y"], r1["y"], rtol=0, atol=1e-12)


def test_layer_rows_independent():
    lw = GeneratedLayer(TINY, 0, 0)
    x = gen.gen_x(3, 4, 256)
    r = layer_forward(lw, x)
    for t in range(4):
        rt = layer_forward(lw, x[t:t + 1])
        assert np.array_equal(rt["ids"][0], r["ids"][t])
        assert np.allclose(rt["y"][0], r["y"][t], rtol=0, atol=1e-14)


def test_stack_zero_down_is_identity_and_boundaries_are_bf16():
    rng = np.random.default_rng(7)
    sh = MoEShape(hidden=128, n_experts=4, inter=64, top_k=2, shared_inter=64,
                  router_bits=16, expert_bits=4, shared_bits=4)
    gv = gen.bf16_round(rng.normal(size=128) / math.sqrt(128))
    wr = gen.bf16_round(rng.normal(size=(4, 128)) / math.sqrt(128))
    layers = [_explicit(sh, [_zero_down(_ffn_q(rng, 64, 128, 4)) for _ in range(4)],
                        _zero_down(_ffn_q(rng, 64, 128, 4)), ("dense", wr), gv) for _ in range(3)]
    x = gen.gen_x(11, 2, 128)
    out = stack_forward(layers, x)
    for r in out:
        assert np.array_equal(r["y"], x)
    # a live stack: each layer input is the bf16 rounding of the previous output
    live = [GeneratedLayer(TINY, 0, l) for l in range(3)]
    out = stack_forward(live, gen.gen_x(12, 1, 256))
    for a, b in zip(out[:-1], out[1:]):
        assert np.array_equal(b["h"], gen.bf16_round(a["y"]))
        assert not np.array_equal(b["h"], a["h"])


def test_tiny_workload_end_to_end_sanity():
    lw = GeneratedLayer(TINY, 0, 0)
    r = layer_forward(lw, gen.gen_x(1000, 1, 256))
    assert r["ids"].shape == (1, 2)
    assert abs(r["w"].sum() - 1.0) < 1e-15
    assert np.all(r["w"] > 0)
    delta = r["y"][0] - gen.gen_x(1000, 1, 256)[0]
    assert 0 < np.abs(delta).max() < 10
