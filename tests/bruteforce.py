"""Independent brute-force forms used to pin the fp64 oracle (test-only).

These are deliberately different computations from the oracle's two-pass
definition:

* ``visible_mask`` enumerates the visible set of every (query, key) pair with
  Python loops (causal, optional sliding window, optional sink tokens; the
  "Sliding-window beats linear attention" review, sec. 1).
* ``closed_form`` evaluates the expanded matrix identity
      O = (P o (1 + S)) V - rowsum(P o S) o (P V),   S = R K^T (unscaled),
  which equals the definition o_i = sum_j p_ij (1 + rho_i.(k_j - kbar_i)) v_j
  because rho_i.kbar_i = sum_j p_ij rho_i.k_j (Parallax: the probe reads the
  key/value covariance as a correction on softmax attention; review page
  "Parallax: Parameterized Local Linear Attention for Language Modeling",
  sec. 1 and sec. 3).
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp, softmax


def visible_mask(L: int, window: int = 0, n_sink: int = 0) -> np.ndarray:
    """Boolean [L, L] mask, entry (i, j) true when query i may read key j."""
    m = np.zeros((L, L), dtype=bool)
    for i in range(L):
        for j in range(L):
            if j > i:
                continue
            in_window = window <= 0 or (i - j) < window
            is_sink = j < n_sink
            m[i, j] = in_window or is_sink
    return m


def closed_form(q, k, v, r, scale=None, window=0, n_sink=0):
    """Matrix closed form on [B,H,L,d] float64 arrays -> (O, LSE)."""
    q, k, v, r = (np.asarray(x, dtype=np.float64) for x in (q, k, v, r))
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    mask = visible_mask(L, window, n_sink)
    O = np.zeros_like(q)
    LSE = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            Z = scale * q[b, h] @ k[b, h].T
            Z = np.where(mask, Z, -np.inf)
            P = softmax(Z, axis=1)
            S = r[b, h] @ k[b, h].T
            PS = P * S
            PV = P @ v[b, h]
            O[b, h] = (P + PS) @ v[b, h] - PS.sum(axis=1, keepdims=True) * PV
            LSE[b, h] = logsumexp(Z, axis=1)
    return O, LSE
