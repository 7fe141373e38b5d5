"""Grouped-query decode attention over a bf16 key/value cache, written out
plainly in fp64 (test infrastructure only).

Sources (web pages; section names as printed on them):

* PureDrive-35B-A3B-MLX model card, "How it works": a custom GQA attention
  kernel reads K/V once for all 8 query heads of a KV head and all verify
  rows, split along the keys ("flash-decoding" style) with split points and
  summation order that depend only on the row's position, so each verify
  row is bit-identical to a one-row decode at that position; "Beyond this
  checkpoint": the kernel is built for 16 query heads, 2 KV heads, head
  dimension 256; "Hardware": the bf16 KV cache takes about 20 KB per token.
* flash-moe news page, "Metal Compute Shaders": GPU attention as Q @ K^T,
  softmax, scores @ V.

What is computed, for verify rows i = 0..T-1 at positions p0 + i (the rows'
own keys and values already in the cache) and query head h:
    s_j   = (q[i, h] . K[h // g, j]) / sqrt(d),      j = 0 .. p0 + i
    o[i, h] = sum_j softmax(s)_j V[h // g, j]
with g = n_q / n_kv query heads per KV head. Rows past a row's own position
are not visible to it (causal). Readings where the pages are silent: the
scale is 1/sqrt(d); q is given (bf16, after any normalisation or rotary
embedding, which are not part of this step); the output is not rounded.
"""

from __future__ import annotations

import numpy as np


def gqa_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, p0: int) -> np.ndarray:
    """q [T, n_q, d], k_cache / v_cache [n_kv, S, d] (values held in fp64),
    p0 the position of row 0 (row i sees keys 0..p0+i, all < S).
    Returns o [T, n_q, d] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    t_rows, n_q, d = q.shape
    n_kv, s_len, _ = k_cache.shape
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    if p0 < 0 or p0 + t_rows > s_len:
        raise ValueError("positions beyond the cache")
    g = n_q // n_kv
    o = np.zeros((t_rows, n_q, d))
    for i in range(t_rows):
        n = p0 + i + 1  # visible keys
        for h in range(n_q):
            kv = h // g
            s = k_cache[kv, :n] @ q[i, h] / np.sqrt(d)
            p = np.exp(s - s.max())
            p /= p.sum()
            o[i, h] = p @ v_cache[kv, :n]
    return o
