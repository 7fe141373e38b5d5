"""Pins of the dense projection oracle (oracle/dense.py), on the CPU.

Each check is fixed by the mathematics, not by the oracle's own code:
* exact rational arithmetic (Python Fractions) on small integer-coded
  matrices with bf16 scales/biases and bf16 inputs, for a three-output fused
  call (a dropped term, a wrong group index or a transposed operand fails);
* a one-hot input picks one dequantised column: code * scale + bias;
* an all-ones input gives the closed form sum over groups of
  scale * (sum of codes) + 64 * bias;
* the fused call equals the three one-matrix calls, and each output keeps its
  own row count (no mixing of outputs).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import gen as ogen
from oracle.dense import gemv


def _qmat(rng, rows, k, bits):
    c = rng.integers(0, 2**bits, size=(rows, k)).astype(np.uint8)
    s = ogen.bf16_round(rng.uniform(0.01, 0.05, size=(rows, k // 64)))
    b = ogen.bf16_round(rng.uniform(-1.0, 1.0, size=(rows, k // 64)) * s * 2**(bits - 1))
    return c, s, b


def _exact(qm, x):
    c, s, b = qm
    rows, k = c.shape
    out = []
    for t in range(x.shape[0]):
        row = []
        for r in range(rows):
            acc = Fraction(0)
            for j in range(k):
                w = Fraction(int(c[r, j])) * Fraction(float(s[r, j // 64])) + Fraction(float(b[r, j // 64]))
                acc += w * Fraction(float(x[t, j]))
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("bits", [3, 6, 8])
def test_fused_three_outputs_exact_rational(bits):
    rng = np.random.default_rng(bits)
    mats = [_qmat(rng, r, 128, bits) for r in (3, 2, 2)]
    x = ogen.bf16_round(rng.normal(size=(2, 128)))
    ys = gemv(mats, x)
    for qm, y in zip(mats, ys):
        ex = _exact(qm, x)
        assert y.shape == (2, qm[0].shape[0])
        for t in range(2):
            for r in range(qm[0].shape[0]):
                assert abs(Fraction(float(y[t, r])) - ex[t][r]) <= abs(ex[t][r]) * Fraction(1, 2**50) + Fraction(1, 2**60)


def test_one_hot_input_selects_a_column():
    rng = np.random.default_rng(5)
    c, s, b = _qmat(rng, 4, 192, 8)
    for j in (0, 63, 64, 191):
        x = np.zeros((1, 192))
        x[0, j] = 1.0
        (y,) = gemv([(c, s, b)], x)
        assert np.array_equal(y[0], c[:, j] * s[:, j // 64] + b[:, j // 64])


def test_all_ones_input_closed_form():
    rng = np.random.default_rng(6)
    c, s, b = _qmat(rng, 5, 256, 4)
    (y,) = gemv([(c, s, b)], np.ones((1, 256)))
    ref = np.zeros(5)
    for g in range(4):
        ref += s[:, g] * c[:, 64 * g:64 * (g + 1)].astype(np.int64).sum(axis=1) + 64 * b[:, g]
    assert np.allclose(y[0], ref, rtol=1e-14, atol=0)


def test_fused_equals_separate_calls():
    rng = np.random.default_rng(7)
    mats = [_qmat(rng, r, 64, 8) for r in (5, 1, 3)]
    x = ogen.bf16_round(rng.normal(size=(3, 64)))
    fused = gemv(mats, x)
    for m, y in zip(mats, fused):
        assert np.array_equal(y, gemv([m], x)[0])
    with pytest.raises(ValueError):
        gemv([_qmat(rng, 2, 128, 8)], x)
