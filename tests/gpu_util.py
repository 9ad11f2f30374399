"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same bf16 values, compare.

Tolerances: O max abs error <= 2e-2 (with rel-L2 reported) and LSE max abs
error <= 1e-3, both against the fp64 oracle evaluated on the exact bf16 inputs
the GPU consumed."""
from __future__ import annotations

import math

import numpy as np
import torch

O_TOL = 2e-2
LSE_TOL = 1e-3


def say(msg: str):
    print(msg, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, what: str, o_tol=O_TOL, lse_tol=LSE_TOL):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    assert np.isfinite(o_gpu).all(), what + ": non-finite O"
    err_o = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    den = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o_gpu - o_ref)) / den if den > 0 else 0.0
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), what + ": LSE finiteness differs"
    assert np.array_equal(lse_gpu[~fin], lse_ref[~fin]), what + ": LSE infinities differ"
    err_lse = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
    say("[parity] %s: max|dO|=%.3e relL2=%.3e max|dLSE|=%.3e" % (what, err_o, rel_l2, err_lse))
    assert err_o <= o_tol, "%s: max|dO| %.3e > %.1e" % (what, err_o, o_tol)
    assert err_lse <= lse_tol, "%s: max|dLSE| %.3e > %.1e" % (what, err_lse, lse_tol)
    return err_o, rel_l2, err_lse


def oracle_rows(orc, q, k, v, r, b, h, rows, scale, window=0, n_sink=0):
    """Oracle on selected rows of one (b, h) slice of device tensors [B,H,L,d]."""
    rows = np.asarray(rows, dtype=np.int64)
    last = int(rows.max()) + 1
    idx = torch.as_tensor(rows, device=q.device)
    K = f64(k[b, h, :last])
    V = f64(v[b, h, :last])
    Q = f64(q[b, h].index_select(0, idx))
    R = f64(r[b, h].index_select(0, idx))
    return orc.rows(Q, R, rows, K, V, scale, window, n_sink)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
