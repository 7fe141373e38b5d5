"""Dense group-affine matrix-vector products of the non-expert projections,
written out plainly in fp64 (test infrastructure only).

Sources (web pages; section names as printed on them):

* PureDrive-35B-A3B-MLX model card, "Summary": the attention projections,
  the shared expert, the embedding and lm_head are 8-bit.
* Qwen3.5-397B on M5 Max news page, "効果的な最適化" (effective
  optimisations): a fused Q/K/V projection kernel reads the input vector once
  instead of three times.
* flash-moe news page, "FMA-optimised dequant kernel": the weights are group
  affine, ``code * scale + bias``.

What is computed: for matrices W_m [rows_m, K] sharing one input x [T, K],
``y_m[t, r] = sum_c W_m[r, c] * x[t, c]`` with W dequantised in groups of 64
along K. The fused Q/K/V projection is this with three matrices; the
attention output projection and lm_head are the one-matrix case. Each
product is computed on its own in fp64; reading x once is an implementation
property the definition does not depend on.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .gen import QMat
from .moe import dequant


def gemv(mats: Sequence[QMat], x: np.ndarray, group: int = 64) -> List[np.ndarray]:
    """``[x @ W_m^T for m]``: fp64 [T, rows_m] for each packed-as-arrays matrix
    ``(codes, scale, bias)`` of shape [rows_m, K], with x [T, K] (bf16 values
    held in fp64)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    out = []
    for codes, scale, bias in mats:
        w = dequant(codes, scale, bias, group)
        if w.shape[1] != x.shape[1]:
            raise ValueError(f"matrix has {w.shape[1]} columns, x has {x.shape[1]}")
        out.append(x @ w.T)
    return out
