"""Pins of the Gated DeltaNet decode-step oracle (oracle/gdn.py), on the CPU.

The recurrence is the gated delta rule of Yang, Kautz & Hatamizadeh
(ICLR 2025); the pages name only the BLAS calls (scale, matrix-vector
products, rank-one update) that compute it. Pins:
* the paper's closed matrix form alpha S (I - beta k k^T) + beta v k^T,
  computed with full matrix products, equals the oracle's BLAS-ordered
  update (a sign, a missing decay or a transposed outer product fails);
* the delta rule's defining property: with beta = 1 and a unit key the new
  state maps k exactly to v;
* special cases: alpha = 1, beta = 0 keeps the state; alpha = 0 forgets it;
  from a zero state with beta = 1 the output is v (k . q);
* value heads share the key/query head h // (n_v / n_k);
* T rows equal T single steps in order.
"""

import numpy as np

from oracle.gdn import gdn_rows, gdn_step


def _unit(rng, *shape):
    x = rng.normal(size=shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(seed, n_k=2, n_v=4, dk=8, dv=6):
    rng = np.random.default_rng(seed)
    return dict(state=rng.normal(size=(n_v, dv, dk)), q=_unit(rng, n_k, dk), k=_unit(rng, n_k, dk),
                v=rng.normal(size=(n_v, dv)), alpha=rng.uniform(0.5, 1.0, n_v), beta=rng.uniform(0, 1, n_v))


def test_matches_the_papers_closed_form():
    c = _case(0)
    s1, o = gdn_step(**c)
    g = c["v"].shape[0] // c["k"].shape[0]
    for h in range(c["v"].shape[0]):
        k, q = c["k"][h // g], c["q"][h // g]
        m = np.eye(k.size) - c["beta"][h] * np.outer(k, k)
        ref = c["alpha"][h] * c["state"][h] @ m + c["beta"][h] * np.outer(c["v"][h], k)
        assert np.allclose(s1[h], ref, rtol=1e-13, atol=1e-13)
        assert np.allclose(o[h], ref @ q, rtol=1e-13, atol=1e-13)


def test_delta_rule_stores_v_at_k():
    c = _case(1)
    c["beta"][:] = 1.0
    s1, _ = gdn_step(**c)
    g = c["v"].shape[0] // c["k"].shape[0]
    for h in range(c["v"].shape[0]):
        assert np.allclose(s1[h] @ c["k"][h // g], c["v"][h], rtol=1e-12, atol=1e-12)


def test_special_gates():
    c = _case(2)
    c["alpha"][:] = 1.0
    c["beta"][:] = 0.0
    s1, o = gdn_step(**c)
    assert np.array_equal(s1, c["state"])
    g = c["v"].shape[0] // c["k"].shape[0]
    for h in range(c["v"].shape[0]):
        assert np.allclose(o[h], c["state"][h] @ c["q"][h // g], rtol=1e-14)
    c = _case(3)
    c["alpha"][:] = 0.0
    s1, _ = gdn_step(**c)
    for h in range(c["v"].shape[0]):
        assert np.allclose(s1[h], c["beta"][h] * np.outer(c["v"][h], c["k"][h // g]), rtol=1e-14)
    c = _case(4)
    c["state"][:] = 0.0
    c["beta"][:] = 1.0
    _, o = gdn_step(**c)
    for h in range(c["v"].shape[0]):
        assert np.allclose(o[h], c["v"][h] * (c["k"][h // g] @ c["q"][h // g]), rtol=1e-13)


def test_value_heads_share_key_heads():
    c = _case(5, n_k=2, n_v=4)
    s1, o = gdn_step(**c)
    # swapping key heads swaps which value heads see them
    c2 = dict(c, k=c["k"][::-1].copy(), q=c["q"][::-1].copy())
    perm = [2, 3, 0, 1]
    c2["state"] = c["state"][perm]
    c2["v"], c2["alpha"], c2["beta"] = c["v"][perm], c["alpha"][perm], c["beta"][perm]
    s2, o2 = gdn_step(**c2)
    assert np.allclose(s2, s1[perm], rtol=1e-14) and np.allclose(o2, o[perm], rtol=1e-14)


def test_rows_are_steps_in_order():
    rng = np.random.default_rng(6)
    T, n_k, n_v, dk, dv = 3, 2, 4, 8, 6
    st = rng.normal(size=(n_v, dv, dk))
    q, k = _unit(rng, T, n_k, dk), _unit(rng, T, n_k, dk)
    v = rng.normal(size=(T, n_v, dv))
    a, b = rng.uniform(0.5, 1, (T, n_v)), rng.uniform(0, 1, (T, n_v))
    s_end, o = gdn_rows(st, q, k, v, a, b)
    s = st
    for t in range(T):
        s, ot = gdn_step(s, q[t], k[t], v[t], a[t], b[t])
        assert np.array_equal(o[t], ot)
    assert np.array_equal(s, s_end)
