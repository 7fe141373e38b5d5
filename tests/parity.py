"""Comparison of GPU results with the oracle, per the pass criteria:

* routing: the selected id sets must be equal, except rows whose oracle gap
  between the k-th and (k+1)-th logit is below 1e-5, which are reported
  (those rows are then left out of the output comparison, since a different
  but equally valid selection changes them);
* output: max |y - y_ref| <= 4e-3 * max |y_ref| over the T x H outputs of the
  layer, with y the GPU's bf16 output and y_ref the oracle's fp64 value
  before rounding.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from oracle import gen as ogen
from oracle.gen import MoEShape

TIE_GAP = 1e-5
REL_TOL = 4e-3


def oracle_shape(kw: dict) -> MoEShape:
    return MoEShape(hidden=kw["hidden"], n_experts=kw["n_experts"], inter=kw["inter"], top_k=kw["top_k"],
                    shared_inter=kw["shared_inter"], router_bits=kw["router_bits"], expert_bits=kw["expert_bits"],
                    shared_bits=kw["shared_bits"], eps=kw.get("rms_eps", 1e-6))


@dataclass
class LayerCheck:
    ok: bool
    ratio: float  # max|y - y_ref| / max|y_ref| over compared rows
    ties: List[int] = field(default_factory=list)
    id_mismatch: List[int] = field(default_factory=list)
    max_w_err: float = 0.0

    def __str__(self):
        return (f"ok={self.ok} err/max={self.ratio:.3e} ties={self.ties} id_mismatch={self.id_mismatch} "
                f"max_w_err={self.max_w_err:.2e}")


def check_layer(y_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, ref: dict) -> LayerCheck:
    """y_bits: uint16 [T, H] GPU output; ids/w: GPU routing [T, k]; ref: oracle layer_forward result."""
    y = ogen.bf16_bits_to_f64(y_bits)
    t_rows = y.shape[0]
    ties, bad, keep = [], [], []
    max_w_err = 0.0
    for t in range(t_rows):
        same = set(ids[t].tolist()) == set(ref["ids"][t].tolist())
        if ref["gap"][t] < TIE_GAP:
            ties.append(t)
            if not same:
                continue
        if not same:
            bad.append(t)
            continue
        keep.append(t)
        order_g = np.argsort(ids[t])
        order_r = np.argsort(ref["ids"][t])
        max_w_err = max(max_w_err, float(np.abs(w[t][order_g] - ref["w"][t][order_r]).max()))
    if not keep:
        return LayerCheck(ok=not bad, ratio=0.0, ties=ties, id_mismatch=bad, max_w_err=max_w_err)
    yr = ref["y"][keep]
    ratio = float(np.abs(y[keep] - yr).max() / np.abs(yr).max())
    return LayerCheck(ok=(not bad) and ratio <= REL_TOL, ratio=ratio, ties=ties, id_mismatch=bad,
                      max_w_err=max_w_err)
