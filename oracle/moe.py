"""The MoE FFN decode step, written out plainly in fp64 (test infrastructure only).

Sources (web pages; section names as printed on them):

* PureDrive-35B-A3B-MLX model card, "Summary": 40 MoE layers, 256 routed
  experts with top-8 selection plus one shared expert; 6-bit routed experts,
  8-bit shared expert and other weights. "FAQ": all 8 routed experts run (no
  top-k reduction).
* flash-moe news page (ja.news.hada.io topic 27758), "FMA-optimised dequant
  kernel": the dequantised weight is ``code * scale + bias`` (group affine)
  and the product ``(code*scale + bias)*x`` equals
  ``fma(code, scale*x, bias*x)``; "Metal Compute Shaders": SwiGLU, RMS
  normalisation, and an MoE combine + residual + gate kernel; "Deferred GPU
  Expert Compute": combine, norm and residual run on the GPU and the result
  goes straight to the next layer; "Model architecture": a 512-expert,
  hidden-4096 shape.

Where the pages are silent the readings taken are:

* SwiGLU is ``silu(W_gate u) * (W_up u)`` with ``silu(g) = g / (1 + e^-g)``;
* RMSNorm has weight 1 and eps 1e-6 and is applied to the layer input; the
  residual is the un-normalised input;
* routing weights are the softmax of the router logits, restricted to the k
  selected experts and renormalised to sum to 1 (equal, in exact arithmetic,
  to the softmax over the selected logits alone); ties in the top-k go to the
  lower expert index; ids are listed by descending logit;
* the shared expert's output is scaled by ``sigmoid(gvec . u)`` at the
  combine, with ``gvec`` a bf16 vector;
* the layer output is kept in fp64 (not rounded); a stack hands the bf16
  rounding (nearest even) of it to the next layer as that layer's input.
"""

from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .gen import MoEShape, bf16_round


def dequant(codes: np.ndarray, scale: np.ndarray, bias: np.ndarray, group: int = 64) -> np.ndarray:
    """Dense fp64 matrix ``W[i, j] = codes[i, j] * scale[i, j // group] + bias[i, j // group]``.

    Group-affine dequantisation along the input dimension (flash-moe news page,
    "FMA-optimised dequant kernel"). With codes < 2^8 and bf16 scale/bias every
    entry is exact in fp64."""
    c = codes.astype(np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float64), group, axis=1)
    b = np.repeat(np.asarray(bias, dtype=np.float64), group, axis=1)
    return c * s + b


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """``u = h / sqrt(mean(h^2) + eps)`` with weight 1 (RMS normalisation,
    flash-moe news page, "Metal Compute Shaders")."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h) + eps)


def route(logits: np.ndarray, k: int):
    """Top-k of the router logits with renormalised softmax weights.

    Returns ``(ids, weights, gap)``: ids of the k largest logits in descending
    order (ties to the lower index), their softmax probabilities renormalised
    to sum 1, and ``gap = logit_(k) - logit_(k+1)`` (inf when k == E).
    Full top-k as on the PureDrive model card ("FAQ"); the weighting is the
    reading stated in the module docstring."""
    lam = np.asarray(logits, dtype=np.float64)
    e = lam.shape[0]
    p = np.exp(lam - lam.max())
    p = p / p.sum()
    order = np.lexsort((np.arange(e), -lam))  # primary: logit descending; then index ascending
    ids = order[:k]
    gap = lam[order[k - 1]] - lam[order[k]] if k < e else np.inf
    w = p[ids] / p[ids].sum()
    return ids.astype(np.int64), w, float(gap)


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def sigmoid(x: float) -> float:
    with np.errstate(over="ignore"):
        return float(1.0 / (1.0 + np.exp(-x)))


def expert_ffn(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, u: np.ndarray) -> np.ndarray:
    """One expert: ``W_down (silu(W_gate u) * (W_up u))`` (SwiGLU, flash-moe news
    page, "Metal Compute Shaders")."""
    return wd @ (silu(wg @ u) * (wu @ u))


def shared_gate(gvec: np.ndarray, u: np.ndarray) -> float:
    """Sigmoid gate of the shared expert, ``1 / (1 + exp(-gvec . u))``."""
    return sigmoid(float(np.dot(gvec, u)))


def _dense_ffn(q: Dict[str, tuple], group: int):
    return tuple(dequant(*q[m], group=group) for m in ("gate", "up", "down"))


class _DenseCache:
    """Dequantises each matrix of a layer once per layer_forward call."""

    def __init__(self, weights, group: int):
        self.w, self.group, self.c = weights, group, {}

    def expert(self, e: int):
        if e not in self.c:
            self.c[e] = _dense_ffn(self.w.expert(e), self.group)
        return self.c[e]

    def shared(self):
        if "s" not in self.c:
            self.c["s"] = _dense_ffn(self.w.shared(), self.group)
        return self.c["s"]

    def router(self):
        if "r" not in self.c:
            kind, val = self.w.router()
            self.c["r"] = val if kind == "dense" else dequant(*val, group=self.group)
        return self.c["r"]


def layer_forward(weights, h: np.ndarray, shape: Optional[MoEShape] = None):
    """One MoE FFN layer on T independent rows.

    ``h`` is [T, H] (bf16 values held in fp64). For each row t:
    ``u = rmsnorm(h_t)``; logits ``W_r u``; ``(ids, w, gap) = route``;
    ``y_t = h_t + sum_i w_i * expert(ids_i)(u) + sigmoid(gvec . u) * shared(u)``
    (the combine + residual + gate step, flash-moe news page, "Metal Compute
    Shaders"). Rows share nothing but weights. Returns a dict with ``y`` [T,H]
    fp64 (not rounded), ``ids`` [T,k], ``w`` [T,k], ``gap`` [T], ``logits``
    [T,E] and ``sgate`` [T]."""
    sh = shape if shape is not None else weights.shape
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    t_rows = h.shape[0]
    dense = _DenseCache(weights, sh.group)
    wr = dense.router()
    gvec = np.asarray(weights.gatevec(), dtype=np.float64)
    ys, ids_all, w_all, gaps, logit_all, sg = [], [], [], [], [], []
    for t in range(t_rows):
        u = rmsnorm(h[t], sh.eps)
        lam = wr @ u
        ids, w, gap = route(lam, sh.top_k)
        y = h[t].copy()
        for i in range(sh.top_k):
            y = y + w[i] * expert_ffn(*dense.expert(int(ids[i])), u)
        sgate = shared_gate(gvec, u)
        y = y + sgate * expert_ffn(*dense.shared(), u)
        ys.append(y)
        ids_all.append(ids)
        w_all.append(w)
        gaps.append(gap)
        logit_all.append(lam)
        sg.append(sgate)
    return {
        "y": np.stack(ys),
        "ids": np.stack(ids_all),
        "w": np.stack(w_all),
        "gap": np.array(gaps),
        "logits": np.stack(logit_all),
        "sgate": np.array(sg),
    }


def stack_forward(layers: List, x: np.ndarray, shape: Optional[MoEShape] = None):
    """A stack of MoE layers: ``h_0 = x``; ``h_{l+1} = bf16(layer_l(h_l))``.

    The hidden state crosses each layer boundary as bf16 (round to nearest
    even), which is how the combine hands its result to the next layer.
    Returns per-layer results (each with the fp64 ``y`` before rounding and
    the layer's bf16 input ``h``)."""
    h = bf16_round(np.atleast_2d(np.asarray(x, dtype=np.float64)))
    out = []
    for lw in layers:
        r = layer_forward(lw, h, shape)
        r["h"] = h
        out.append(r)
        h = bf16_round(r["y"])
    return out
