"""Pins for the oracle's synthetic-input generator (CPU only).

Each test checks the generator against something other than itself: the
published splitmix64 reference outputs, exact bf16 rounding cases, closed
forms of the Irwin-Hall decoder, and distribution statistics that the
workload definition fixes (uniform codes, scales in [0.5, 1.5] * C, bias
centred on -m_b * s with spread 0.1 * s, N(0, sigma) vectors)."""

import math
import os

import numpy as np
import pytest

from oracle import gen

GAMMA = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1


def _read_golden(golden_dir, name):
    vals = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(int(line))
    return vals


def test_mix64_matches_published_splitmix64_sequence(golden_dir):
    ref = _read_golden(golden_dir, "splitmix64_seed1234567.txt")
    states = np.array([(1234567 + i * GAMMA) & M64 for i in range(len(ref))], dtype=np.uint64)
    got = [int(v) for v in gen.mix64(states)]
    assert got == ref


def test_mix64_vectorised_equals_scalar_calls():
    xs = np.array([0, 1, 2**63, M64, 0xDEADBEEF], dtype=np.uint64)
    v = gen.mix64(xs)
    for i, x in enumerate(xs):
        assert int(gen.mix64(int(x))[0]) == int(v[i])


@pytest.mark.parametrize(
    "x,expect",
    [
        (1.0, 1.0),
        (1.0 + 2.0**-8, 1.0),  # halfway, ties to even (down)
        (1.0 + 3 * 2.0**-8, 1.0 + 2.0**-6),  # halfway, ties to even (up)
        (1.0 + 2.0**-8 + 2.0**-20, 1.0 + 2.0**-7),  # just above halfway
        (-(1.0 + 2.0**-8 + 2.0**-20), -(1.0 + 2.0**-7)),
        (0.0, 0.0),
        (3.0, 3.0),
        (255.0, 255.0),  # 8 significant bits: 0b11111111 is exact
        (511.0, 512.0),  # 9 bits: halfway between 510 (odd mantissa) and 512 -> even
        (257.0, 256.0),
        (2.0**-130, 2.0**-130),  # subnormal f32, exactly representable in bf16
    ],
)
def test_bf16_rounding_cases(x, expect):
    assert gen.bf16_round(np.array([x]))[0] == expect


def test_bf16_bits_roundtrip_and_known_patterns():
    assert int(gen.f64_to_bf16_bits(np.array([1.0]))[0]) == 0x3F80
    assert int(gen.f64_to_bf16_bits(np.array([-2.0]))[0]) == 0xC000
    assert int(gen.f64_to_bf16_bits(np.array([0.5]))[0]) == 0x3F00
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)  # finite positives
    assert np.array_equal(gen.f64_to_bf16_bits(gen.bf16_bits_to_f64(bits)), bits)


def test_irwin_hall_closed_forms():
    zero = np.zeros((1, 3), dtype=np.uint64)
    assert gen.irwin_hall(zero)[0] == (6 - 6 * 65536) / 65536.0
    full = np.full((1, 3), M64, dtype=np.uint64)
    assert gen.irwin_hall(full)[0] == (12 * 65535 + 6 - 6 * 65536) / 65536.0
    # lanes 1,2,...,12 in draw order (lane 0 of draw 0 is the low 16 bits)
    d = np.zeros((1, 3), dtype=np.uint64)
    lane = 1
    for j in range(3):
        v = 0
        for sh in (0, 16, 32, 48):
            v |= lane << sh
            lane += 1
        d[0, j] = v
    assert gen.irwin_hall(d)[0] == (sum(range(1, 13)) + 6 - 6 * 65536) / 65536.0


def test_irwin_hall_moments():
    d = gen.draws(12345, gen.T_X, gen.F_CODE, np.arange(3 * 200000, dtype=np.uint64)).reshape(-1, 3)
    z = gen.irwin_hall(d)
    assert abs(z.mean()) < 0.01
    assert abs(z.var() - 1.0) < 0.01  # Irwin-Hall(12) - 6 has variance exactly 1
    assert np.all(np.abs(z) <= 6.0)


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_codes_uniform(bits):
    c = gen.gen_codes(gen.sub_seed(0, 3, 5), gen.T_GATE, 256, 1024, bits)
    assert c.dtype == np.uint8
    n = 1 << bits
    hist = np.bincount(c.ravel(), minlength=n)
    assert hist.shape[0] == n  # nothing above 2^b - 1
    expect = c.size / n
    chi2 = float(((hist - expect) ** 2 / expect).sum())
    # chi-square with n-1 dof: mean n-1, sd sqrt(2(n-1)); 6 sd bound
    assert chi2 < (n - 1) + 6 * math.sqrt(2 * (n - 1))
    assert hist.min() > 0


@pytest.mark.parametrize("bits,d_in", [(4, 256), (4, 128), (6, 2048), (8, 2048), (2, 4096), (3, 4096), (8, 512)])
def test_scales_range_and_mean(bits, d_in):
    s = gen.gen_scales(gen.sub_seed(0, 1, 2), gen.T_UP, 128, d_in, bits)
    c = 1.0 / (2 ** (bits - 1) * math.sqrt(d_in))
    lo = gen.bf16_round(np.array([0.5 * c]))[0]
    hi = gen.bf16_round(np.array([1.5 * c]))[0]
    assert s.min() >= lo and s.max() <= hi
    # U uniform on [0.5, 1.5): sd 1/sqrt(12) per sample; 5-sigma bound on the mean (+ bf16 rounding)
    assert abs(s.mean() / c - 1.0) < 5 / math.sqrt(12 * s.size) + 2.0**-9
    assert np.array_equal(gen.bf16_round(s), s)


def test_tiny_workload_scale_reading():
    # 4-bit codes with d_in 256: scales uniform in [0.5, 1.5] / (8 * sqrt(256)) = [0.5, 1.5] / 128
    assert gen.scale_const(4, 256) == 1.0 / 128.0


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_bias_centre_and_spread(bits):
    sub = gen.sub_seed(7, 0, 1)
    s = gen.gen_scales(sub, gen.T_DOWN, 512, 512, bits)
    b = gen.gen_biases(sub, gen.T_DOWN, s, bits)
    m_b = (2**bits - 1) / 2
    assert np.array_equal(gen.bf16_round(b), b)
    # hard bound: the noise term is at most 6 * 0.1 * s, then one bf16 rounding (half ulp <= 2^-8 |b|)
    assert np.all(np.abs(b + m_b * s) <= 0.6 * s + 2.0**-8 * np.abs(b) * (1 + 1e-12))
    z = (b + m_b * s) / (0.1 * s)  # recovered noise, up to the bf16 rounding of b
    if bits <= 4:
        # rounding moves z by at most 2^-8 * m_b / 0.1 (0.06 at 2 bits, 0.3 at 4 bits)
        slack = 2.0**-8 * (m_b + 0.6) / 0.1
        assert abs(z.mean()) < 5 / math.sqrt(z.size) + slack
        assert abs(z.std() - 1.0) < 0.05 + slack


@pytest.mark.parametrize("bits,d_in", [(2, 1024), (3, 4096), (4, 256), (6, 2048), (8, 2048), (8, 512)])
def test_dequantised_weight_spread_independent_of_bits(bits, d_in):
    """Reading of 'scaled by 2^bits': std(w) * sqrt(d_in) ~ sqrt(13/12 * 4/12) ~ 0.601 for every width."""
    from oracle.moe import dequant

    sub = gen.sub_seed(0, 2, 9)
    c, s, b = gen.gen_qmat(sub, gen.T_GATE, 64, d_in, bits)
    w = dequant(c, s, b)
    sd = w.std() * math.sqrt(d_in)
    expect = math.sqrt(13 / 12 * (4**bits - 1) / 12 / 4 ** (bits - 1) + 13 / 12 * 0.01 / 4 ** (bits - 1))
    assert abs(sd / expect - 1) < 0.05
    assert abs(w.mean() * math.sqrt(d_in)) < 0.02


def test_vectors_and_x_distribution():
    h = 2048
    g = gen.gen_vector(gen.sub_seed(0, 0, 258), gen.T_GATEVEC, h * 64, 1 / math.sqrt(h))
    assert abs(g.std() * math.sqrt(h) - 1) < 0.02
    x = gen.gen_x(1000, 8, 4096)
    assert x.shape == (8, 4096)
    assert abs(x.mean()) < 0.03 and abs(x.std() - 1) < 0.02
    assert np.array_equal(gen.bf16_round(x), x)
    # x differs per seed, equal for equal seed
    assert np.array_equal(gen.gen_x(5, 2, 64), gen.gen_x(5, 2, 64))
    assert not np.array_equal(gen.gen_x(5, 2, 64), gen.gen_x(6, 2, 64))


def test_sub_seeds_distinct():
    seen = set()
    for layer in range(6):
        for slot in range(515):
            seen.add(gen.sub_seed(0, layer, slot))
    assert len(seen) == 6 * 515


def test_generated_layer_shapes():
    sh = gen.MoEShape(hidden=256, n_experts=16, inter=128, top_k=2, shared_inter=128,
                      router_bits=16, expert_bits=4, shared_bits=4)
    lw = gen.GeneratedLayer(sh, 0, 0)
    e = lw.expert(3)
    assert e["gate"][0].shape == (128, 256) and e["gate"][1].shape == (128, 4)
    assert e["down"][0].shape == (256, 128) and e["down"][1].shape == (256, 2)
    kind, wr = lw.router()
    assert kind == "dense" and wr.shape == (16, 256)
    assert abs(wr.std() * 16 - 1) < 0.05
    assert lw.gatevec().shape == (256,)
    # determinism and independence across experts
    assert np.array_equal(gen.GeneratedLayer(sh, 0, 0).expert(3)["up"][0], e["up"][0])
    assert not np.array_equal(lw.expert(4)["up"][0], e["up"][0])
