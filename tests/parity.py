"""Comparison of GPU results with the oracle, per the pass criteria:

* routing: the selected ids, as ordered lists (descending logit), must equal
  the oracle's. Rows whose oracle gap between the k-th and (k+1)-th logit is
  below 1e-5 are reported, not failed, when their id sets differ (a different
  but equally valid selection; such rows are left out of the output
  comparison). Inside the selection two ids may trade places only where the
  oracle's logits of the two differ by less than 1e-5 (reported as order
  ties).
* routing weights: |w - w_ref| <= 1e-6 for every selected expert (matched by
  id), w the GPU's fp32 renormalised weight and w_ref the oracle's fp64 one.
* output: max |y - y_ref| <= 4e-3 * max |y_ref| over the T x H outputs of the
  layer, with y the GPU's bf16 output and y_ref the oracle's fp64 value
  before rounding;
* output, element by element: the GPU's bf16 value must be the correct
  rounding (to nearest even) of some value within e = 1e-5 * |y_ref| +
  2e-6 * max|y_ref| of y_ref, i.e. lie between bf16(y_ref - e) and
  bf16(y_ref + e). Where y_ref is not near a rounding midpoint this is
  bf16(y_ref) exactly; near a midpoint either neighbour passes; for elements
  near zero (h and the experts' sum cancelling) the absolute part allows the
  few ulps an fp32 sum of order-1 terms leaves. This bounds the compute error
  some 2000 times below the 4e-3 budget, which bf16 rounding of the output
  alone nearly uses up.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from oracle import gen as ogen
from oracle.gen import MoEShape

TIE_GAP = 1e-5
REL_TOL = 4e-3
W_TOL = 1e-6
EL_REL = 1e-5
EL_ABS = 2e-6


def oracle_shape(kw: dict) -> MoEShape:
    return MoEShape(hidden=kw["hidden"], n_experts=kw["n_experts"], inter=kw["inter"], top_k=kw["top_k"],
                    shared_inter=kw["shared_inter"], router_bits=kw["router_bits"], expert_bits=kw["expert_bits"],
                    shared_bits=kw["shared_bits"], eps=kw.get("rms_eps", 1e-6))


def _ordered_key(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers in the order of the values (one step = one ulp)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def ulp_check(y_bits: np.ndarray, y_ref: np.ndarray):
    """Element-wise check of the GPU's bf16 output against the exact fp64 value.

    Returns (n_bad, n_off, max_ulps, worst): elements outside
    [bf16(y_ref - e), bf16(y_ref + e)]; elements that differ from bf16(y_ref);
    the largest such difference in ulps; and a description of the first bad
    element (or "")."""
    ref_bits = ogen.f64_to_bf16_bits(y_ref)
    e = EL_REL * np.abs(y_ref) + EL_ABS * np.abs(y_ref).max()
    g = _ordered_key(y_bits)
    lo = _ordered_key(ogen.f64_to_bf16_bits(y_ref - e))
    hi = _ordered_key(ogen.f64_to_bf16_bits(y_ref + e))
    d = g - _ordered_key(ref_bits)
    bad = (g < lo) | (g > hi)
    worst = ""
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        yg = float(ogen.bf16_bits_to_f64(y_bits[i]))
        worst = (f"first bad {i}: y_ref={float(y_ref[i]):.9g} gpu={yg:.9g} "
                 f"bf16(y_ref)={float(ogen.bf16_bits_to_f64(ref_bits[i])):.9g} e={float(e[i]):.3g} "
                 f"max|y_ref|={float(np.abs(y_ref).max()):.4g}")
    return int(bad.sum()), int((d != 0).sum()), int(np.abs(d).max()), worst


def _step(bits: np.ndarray, direction: int) -> np.ndarray:
    """The bf16 neighbour of each pattern, one ulp up (+1) or down (-1) in value."""
    k = _ordered_key(bits) + direction
    return np.where(k >= 0, k, (-k) | 0x8000).astype(np.uint16)


@dataclass
class LayerCheck:
    ok: bool
    ratio: float  # max|y - y_ref| / max|y_ref| over compared rows
    ties: List[int] = field(default_factory=list)
    id_mismatch: List[int] = field(default_factory=list)
    order_ties: List[int] = field(default_factory=list)
    max_w_err: float = 0.0
    ulp_bad: int = 0
    ulp_off: int = 0
    ulp_max: int = 0
    ulp_worst: str = ""

    def __str__(self):
        return (f"ok={self.ok} err/max={self.ratio:.3e} ties={self.ties} id_mismatch={self.id_mismatch} "
                f"order_ties={self.order_ties} max_w_err={self.max_w_err:.2e} elements: bad={self.ulp_bad} "
                f"off={self.ulp_off} max_ulps={self.ulp_max} {self.ulp_worst}")


def check_layer(y_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, ref: dict) -> LayerCheck:
    """y_bits: uint16 [T, H] GPU output; ids/w: GPU routing [T, k]; ref: oracle layer_forward result."""
    y = ogen.bf16_bits_to_f64(y_bits)
    t_rows = y.shape[0]
    ties, bad, keep, order_ties = [], [], [], []
    max_w_err = 0.0
    for t in range(t_rows):
        gi, ri = [int(v) for v in ids[t]], [int(v) for v in ref["ids"][t]]
        same = set(gi) == set(ri)
        if ref["gap"][t] < TIE_GAP:
            ties.append(t)
            if not same:
                continue
        if not same:
            bad.append(t)
            continue
        lam = ref["logits"][t]
        if gi != ri:
            # positions may differ only between ids whose oracle logits are within TIE_GAP
            if all(g == r or abs(lam[g] - lam[r]) < TIE_GAP for g, r in zip(gi, ri)):
                order_ties.append(t)
            else:
                bad.append(t)
                continue
        wref = dict(zip(ri, ref["w"][t]))
        max_w_err = max(max_w_err, max(abs(float(w[t][i]) - float(wref[g])) for i, g in enumerate(gi)))
        keep.append(t)
    if not keep:
        return LayerCheck(ok=not bad, ratio=0.0, ties=ties, id_mismatch=bad, order_ties=order_ties,
                          max_w_err=max_w_err)
    yr = ref["y"][keep]
    ratio = float(np.abs(y[keep] - yr).max() / np.abs(yr).max())
    nbad, noff, nmax, worst = ulp_check(y_bits[keep], yr)
    ok = (not bad) and ratio <= REL_TOL and max_w_err <= W_TOL and nbad == 0
    return LayerCheck(ok=ok, ratio=ratio, ties=ties, id_mismatch=bad, order_ties=order_ties, max_w_err=max_w_err,
                      ulp_bad=nbad, ulp_off=noff, ulp_max=nmax, ulp_worst=worst)
