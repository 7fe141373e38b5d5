"""Seeded synthetic weights and activations, the oracle's own implementation.

Test infrastructure only (see the package docstring). The GPU library carries
its own implementation of the same published generator; nothing is shared.

Generator definition
--------------------
The pages describe the workloads (a 35B-A3B-shaped and a 397B-A17B-shaped
MoE, group-affine 2/3/4/6/8-bit experts, bf16 scales and biases) but publish
no weights, so the inputs are synthetic. They come from one counter-based
generator, splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used as a stateless hash:

* ``mix64(s)`` is the first splitmix64 output from state ``s``:
  ``z = s + 0x9E3779B97F4A7C15``; ``z = (z ^ z>>30) * 0xBF58476D1CE4E5B9``;
  ``z = (z ^ z>>27) * 0x94D049BB133111EB``; return ``z ^ z>>31`` (mod 2^64).
* sub-seed of (layer, slot): ``mix64(seed ^ mix64(layer * 2^20 + slot))``
  with slot = expert id ``0..E-1``, ``E`` = shared expert, ``E+1`` = router,
  ``E+2`` = shared-expert gate vector.
* a draw: ``mix64(sub ^ (stream * 2^48 + index))`` with
  ``stream = 3 * tensor + field``; tensor gate 0, up 1, down 2, router 3,
  gate vector 4, x 5; field code 0, scale 1, bias 2. ``index`` is row-major
  inside the tensor: ``row * K + col`` for codes and vector values,
  ``row * (K / 64) + group`` for scales; a bias uses the three draws
  ``3*i, 3*i+1, 3*i+2`` of its stream, a vector value the three draws
  ``3*i .. 3*i+2`` of the code stream.
* code ``c = draw >> (64 - b)``: uniform on ``[0, 2^b - 1]``.
* scale ``s = bf16(f32(U * C))`` with ``U = 0.5 + ((draw >> 40) + 0.5) * 2^-24``
  (uniform on [0.5, 1.5)) and ``C = 1 / (2^(b-1) * sqrt(d_in))`` in fp64,
  d_in the matrix's input dimension. At b = 4 this is the tiny workload's
  ``[0.5, 1.5] / (8 sqrt(d_in))``; for other widths the ``2^(b-1)`` keeps
  the dequantised weight spread independent of b.
* bias ``beta = bf16(f32((0.1 * s) * z - m_b * s))``, ``m_b = (2^b - 1) / 2``,
  evaluated in that order in fp64 with no fused multiply-add, with ``s`` the
  bf16 scale and ``z`` an Irwin-Hall(12) normal: the twelve 16-bit lanes
  ``L_i`` of three draws give ``z = sum((L_i + 0.5) / 2^16) - 6``, computed
  exactly as ``(sum L_i + 6 - 6 * 2^16) / 2^16``. Mean 0, variance 1, bounded
  by +-6: a Gaussian shape with no transcendental function, so two
  implementations agree bit for bit.
* bf16 vectors (shared-expert gate vector, a bf16 router, x rows):
  ``v = bf16(f32(z * sigma))`` with z as above, sigma = ``1 / sqrt(H)`` for
  the gate vector and a bf16 router, 1 for x.
* x rows: sub-seed ``mix64(seed_x ^ mix64(XTAG))``, tensor 5, index
  ``t * H + j``.
* every fp64 -> f32 and f32 -> bf16 conversion rounds to nearest even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Tuple

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# tensor ids and fields of the draw stream
T_GATE, T_UP, T_DOWN, T_ROUTER, T_GATEVEC, T_X = 0, 1, 2, 3, 4, 5
# dense (non-expert) projections of a layer: query, key, value, attention
# output, lm_head; their sub-seed uses the slot DENSE_SLOT of the layer
T_Q, T_K, T_V, T_O, T_LM = 6, 7, 8, 9, 10
DENSE_SLOT = (1 << 20) - 1
F_CODE, F_SCALE, F_BIAS = 0, 1, 2
GROUP = 64
# tag of the x-row sub-seed ("x_rows" in ASCII)
XTAG = 0x785F726F7773


def mix64(x) -> np.ndarray:
    """First splitmix64 output from state(s) ``x`` (uint64, wraps mod 2^64)."""
    z = np.atleast_1d(np.asarray(x, dtype=np.uint64))
    with np.errstate(over="ignore"):
        z = z + np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def sub_seed(seed: int, layer: int, slot: int) -> int:
    inner = int(mix64((layer << 20) + slot)[0])
    return int(mix64((seed & MASK64) ^ inner)[0])


def x_sub_seed(seed_x: int) -> int:
    return int(mix64((seed_x & MASK64) ^ int(mix64(XTAG)[0]))[0])


def draws(sub: int, tensor: int, field: int, idx: np.ndarray) -> np.ndarray:
    stream = 3 * tensor + field
    ctr = np.uint64(stream << 48) + idx.astype(np.uint64)
    return mix64(np.uint64(sub) ^ ctr)


# ---------------------------------------------------------------- bf16 helpers
def f64_to_bf16_bits(x) -> np.ndarray:
    """fp64 -> f32 (round to nearest even) -> bf16 (round to nearest even)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Value of ``bf16(f32(x))`` as fp64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


# ------------------------------------------------------------- draw decoders
def irwin_hall(d3: np.ndarray) -> np.ndarray:
    """z from three draws per value, shape [..., 3] uint64 -> fp64 [...]."""
    s = np.zeros(d3.shape[:-1], dtype=np.int64)
    for j in range(3):
        d = d3[..., j]
        for sh in (0, 16, 32, 48):
            s += ((d >> np.uint64(sh)) & np.uint64(0xFFFF)).astype(np.int64)
    return (s + 6 - 6 * 65536).astype(np.float64) / 65536.0


def scale_const(bits: int, d_in: int) -> float:
    return 1.0 / (2.0 ** (bits - 1) * math.sqrt(d_in))


def gen_codes(sub: int, tensor: int, rows: int, k: int, bits: int) -> np.ndarray:
    d = draws(sub, tensor, F_CODE, np.arange(rows * k, dtype=np.uint64))
    return (d >> np.uint64(64 - bits)).astype(np.uint8).reshape(rows, k)


def gen_scales(sub: int, tensor: int, rows: int, k: int, bits: int) -> np.ndarray:
    ng = k // GROUP
    d = draws(sub, tensor, F_SCALE, np.arange(rows * ng, dtype=np.uint64))
    u = 0.5 + ((d >> np.uint64(40)).astype(np.float64) + 0.5) * 2.0 ** -24
    return bf16_round(u * scale_const(bits, k)).reshape(rows, ng)


def gen_biases(sub: int, tensor: int, s: np.ndarray, bits: int) -> np.ndarray:
    rows, ng = s.shape
    d = draws(sub, tensor, F_BIAS, np.arange(3 * rows * ng, dtype=np.uint64))
    z = irwin_hall(d.reshape(rows, ng, 3))
    m_b = (2.0 ** bits - 1.0) / 2.0
    t = 0.1 * s
    t = t * z
    return bf16_round(t - m_b * s)


def gen_vector(sub: int, tensor: int, n: int, sigma: float) -> np.ndarray:
    d = draws(sub, tensor, F_CODE, np.arange(3 * n, dtype=np.uint64))
    return bf16_round(irwin_hall(d.reshape(n, 3)) * sigma)


def gen_x(seed_x: int, t: int, h: int) -> np.ndarray:
    """x rows [t, h] as fp64 holding bf16 values, ~N(0, 1) (Irwin-Hall)."""
    return gen_vector(x_sub_seed(seed_x), T_X, t * h, 1.0).reshape(t, h)


# ------------------------------------------------------------------- shapes
@dataclass(frozen=True)
class MoEShape:
    """One MoE FFN layer: H hidden, E routed experts of intermediate I, top-k,
    one shared expert of intermediate I_s with a bf16 sigmoid gate vector.
    ``router_bits`` 16 means a dense bf16 router, else affine codes."""

    hidden: int
    n_experts: int
    inter: int
    top_k: int
    shared_inter: int
    router_bits: int
    expert_bits: int
    shared_bits: int
    group: int = GROUP
    eps: float = 1e-6


QMat = Tuple[np.ndarray, np.ndarray, np.ndarray]  # codes [R,K] u8, scale [R,K/64], bias [R,K/64]


def gen_qmat(sub: int, tensor: int, rows: int, k: int, bits: int) -> QMat:
    c = gen_codes(sub, tensor, rows, k, bits)
    s = gen_scales(sub, tensor, rows, k, bits)
    b = gen_biases(sub, tensor, s, bits)
    return c, s, b


def dense_matrix(seed: int, layer: int, tensor: int, rows: int, k: int, bits: int) -> QMat:
    """A dense projection's packed-as-arrays matrix [rows, k] (codes, scales,
    biases) from the sub-seed of (layer, DENSE_SLOT) and its tensor id."""
    return gen_qmat(sub_seed(seed, layer, DENSE_SLOT), tensor, rows, k, bits)


class GeneratedLayer:
    """Weights of one layer, regenerated on demand from (seed, layer)."""

    def __init__(self, shape: MoEShape, seed: int, layer: int):
        self.shape, self.seed, self.layer = shape, seed, layer
        self._cache: Dict[object, object] = {}

    def _sub(self, slot: int) -> int:
        return sub_seed(self.seed, self.layer, slot)

    def _ffn(self, slot: int, inter: int, bits: int) -> Dict[str, QMat]:
        h = self.shape.hidden
        sub = self._sub(slot)
        return {
            "gate": gen_qmat(sub, T_GATE, inter, h, bits),
            "up": gen_qmat(sub, T_UP, inter, h, bits),
            "down": gen_qmat(sub, T_DOWN, h, inter, bits),
        }

    def expert(self, e: int) -> Dict[str, QMat]:
        key = ("e", e)
        if key not in self._cache:
            sh = self.shape
            self._cache[key] = self._ffn(e, sh.inter, sh.expert_bits)
        return self._cache[key]

    def shared(self) -> Dict[str, QMat]:
        if "s" not in self._cache:
            sh = self.shape
            self._cache["s"] = self._ffn(sh.n_experts, sh.shared_inter, sh.shared_bits)
        return self._cache["s"]

    def router(self):
        """('dense', W [E,H]) for a bf16 router, else ('q', (codes, s, b))."""
        if "r" not in self._cache:
            sh = self.shape
            sub = self._sub(sh.n_experts + 1)
            if sh.router_bits == 16:
                w = gen_vector(sub, T_ROUTER, sh.n_experts * sh.hidden, 1.0 / math.sqrt(sh.hidden))
                self._cache["r"] = ("dense", w.reshape(sh.n_experts, sh.hidden))
            else:
                self._cache["r"] = ("q", gen_qmat(sub, T_ROUTER, sh.n_experts, sh.hidden, sh.router_bits))
        return self._cache["r"]

    def gatevec(self) -> np.ndarray:
        if "g" not in self._cache:
            sh = self.shape
            sub = self._sub(sh.n_experts + 2)
            self._cache["g"] = gen_vector(sub, T_GATEVEC, sh.hidden, 1.0 / math.sqrt(sh.hidden))
        return self._cache["g"]

    def drop_cache(self) -> None:
        self._cache.clear()


class ExplicitLayer:
    """A layer given by arrays (for tests that build special weights).

    experts: list of dicts {gate, up, down} -> QMat; shared: same dict;
    router: ('dense', W) or ('q', QMat); gatevec: fp64 [H]."""

    def __init__(self, shape: MoEShape, experts, shared, router, gatevec):
        self.shape = shape
        self._experts, self._shared, self._router, self._gatevec = experts, shared, router, gatevec

    def expert(self, e: int):
        return self._experts[e]

    def shared(self):
        return self._shared

    def router(self):
        return self._router

    def gatevec(self):
        return self._gatevec
