"""One decode step of a Gated DeltaNet layer's recurrence, written out plainly
in fp64 (test infrastructure only).

Sources:

* PureDrive-35B-A3B-MLX model card, "Summary": 30 of the 40 layers of the
  35B-A3B model are Gated DeltaNet layers; "How it works": the runtime retunes
  its GDN recurrence kernels; credits: Gated DeltaNet (Yang et al., ICLR 2025).
* flash-moe news page, "Accelerate BLAS活用" (use of Accelerate BLAS): the
  GatedDeltaNet recurrence is computed with cblas_sscal, cblas_sgemv and
  cblas_sger (a scaling of the state, matrix-vector products and a rank-one
  update); "Model architecture": 45 GatedDeltaNet layers of the 397B model.

The pages name only those BLAS calls. The recurrence is the gated delta rule
of Yang, Kautz & Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with
Delta Rule" (ICLR 2025): with a state S in R^{d_v x d_k} per value head,
    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,
and alpha_t in (0, 1] the decay gate, beta_t in [0, 1] the writing strength.
As the BLAS calls order it (the same matrix, regrouped):
    S <- alpha S                 (sscal)
    u  = S k                     (sgemv)
    S <- S + beta (v - u) k^T    (sger)
    o  = S q                     (sgemv)
Readings where the pages are silent: q and k arrive already normalised (the
projections, short convolution and normalisation before the recurrence are
not part of this step); value head h uses key/query head h // (n_v / n_k);
a call of T rows applies the step to each row in order and leaves the state
after the last row; the state is fp32 in the kernels and fp64 here.
"""

from __future__ import annotations

import numpy as np


def gdn_step(state: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray,
             beta: np.ndarray):
    """One token through the recurrence of every value head.

    state [n_v, d_v, d_k]; q, k [n_k, d_k]; v [n_v, d_v]; alpha, beta [n_v].
    Returns (new_state, o [n_v, d_v]); the input state is not modified."""
    s = np.array(state, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_v = s.shape[0]
    n_k = k.shape[0]
    if n_v % n_k:
        raise ValueError("n_v must be a multiple of n_k")
    g = n_v // n_k
    o = np.zeros((n_v, s.shape[1]))
    for h in range(n_v):
        kh, qh = k[h // g], q[h // g]
        s[h] *= alpha[h]
        u = s[h] @ kh
        s[h] += beta[h] * np.outer(v[h] - u, kh)
        o[h] = s[h] @ qh
    return s, o


def gdn_rows(state, q, k, v, alpha, beta):
    """T rows in order: q, k [T, n_k, d_k]; v [T, n_v, d_v]; alpha, beta [T, n_v].
    Returns (state after the last row, o [T, n_v, d_v])."""
    outs = []
    s = state
    for t in range(np.asarray(q).shape[0]):
        s, o = gdn_step(s, q[t], k[t], v[t], alpha[t], beta[t])
        outs.append(o)
    return s, np.stack(outs)
