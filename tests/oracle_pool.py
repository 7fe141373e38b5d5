"""Oracle runs spread over worker processes (test infrastructure).

Token rows are independent in the method, so the oracle's layer chain of
each row (h_{l+1} = bf16(y_l)) is computed in its own process and the
per-layer results are stacked back into the [T, ...] form layer_forward
returns. The workers import only oracle/ and numpy; they are started with
the "spawn" method, so they share nothing with a parent that uses the GPU.
"""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Sequence

import numpy as np


def _row_chain(args):
    """One row through `layers` in order: the oracle's own chain."""
    shape_kw, seed, layers, x_row, chain = args
    from oracle import gen as ogen
    from oracle.moe import layer_forward

    sh = ogen.MoEShape(**shape_kw)
    h = ogen.bf16_round(np.asarray(x_row, dtype=np.float64)[None, :])
    out = []
    for i, l in enumerate(layers):
        hin = h if chain or i == 0 else ogen.bf16_round(np.asarray(x_row, dtype=np.float64)[None, :])
        r = layer_forward(ogen.GeneratedLayer(sh, seed, l), hin)
        r["h"] = hin
        out.append(r)
        h = ogen.bf16_round(r["y"])
    return out


def _workers(n: int) -> int:
    return max(1, min(n, 8, os.cpu_count() or 1))


def oracle_rows(shape, seed: int, layers: Sequence[int], x: np.ndarray, chain: bool = True) -> List[Dict]:
    """Per layer of `layers`, the oracle's layer_forward result for all rows of x.

    chain=True: each row runs the oracle chain through the layers in order
    (layer i's input is bf16 of layer i-1's output); chain=False: every
    listed layer gets x itself. ``shape`` is an oracle MoEShape."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    kw = dict(hidden=shape.hidden, n_experts=shape.n_experts, inter=shape.inter, top_k=shape.top_k,
              shared_inter=shape.shared_inter, router_bits=shape.router_bits, expert_bits=shape.expert_bits,
              shared_bits=shape.shared_bits, eps=shape.eps)
    jobs = [(kw, seed, list(layers), x[t], chain) for t in range(x.shape[0])]
    if len(jobs) == 1:
        per_row = [_row_chain(jobs[0])]
    else:
        with ProcessPoolExecutor(_workers(len(jobs)), mp_context=mp.get_context("spawn")) as ex:
            per_row = list(ex.map(_row_chain, jobs))
    out = []
    for i in range(len(layers)):
        rows = [per_row[t][i] for t in range(x.shape[0])]
        out.append({k: np.concatenate([r[k] for r in rows]) if np.ndim(rows[0][k]) else np.array([r[k] for r in rows])
                    for k in rows[0]})
    return out


def oracle_pairs(shape, seed: int, pairs: Sequence) -> List[Dict]:
    """layer_forward of each (layer, x_row) pair, one worker process per pair."""
    kw = dict(hidden=shape.hidden, n_experts=shape.n_experts, inter=shape.inter, top_k=shape.top_k,
              shared_inter=shape.shared_inter, router_bits=shape.router_bits, expert_bits=shape.expert_bits,
              shared_bits=shape.shared_bits, eps=shape.eps)
    jobs = [(kw, seed, [l], np.asarray(xr, dtype=np.float64).reshape(-1), False) for l, xr in pairs]
    with ProcessPoolExecutor(_workers(len(jobs)), mp_context=mp.get_context("spawn")) as ex:
        return [r[0] for r in ex.map(_row_chain, jobs)]
