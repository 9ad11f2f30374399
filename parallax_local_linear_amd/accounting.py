"""Algorithmic work and traffic of the workloads (measurement accounting only).

Prefill counts 8d FLOP per visible (query, key) pair: four products of 2d
FLOP each -- the two score products q.k and rho.k, and the two value products
p v and p s v.  Exponentials, masked-out work and rescaling are not counted.
Algorithmic HBM bytes are the inputs read once and the outputs written once.
Decode counts the same 8d FLOP per cached key; its bytes are dominated by the
K and V caches.

The backward counts 16d FLOP per visible pair: eight products of 2d FLOP --
the three score products q.k, rho.k and dO.v (recomputed once), dv, the two
terms of dk (from q and from rho), dq and drho.  A second recomputation of
the scores, which the query kernel does, is not counted.
"""
from __future__ import annotations

from .workloads import Decode, Prefill


def visible_pairs(L: int, window: int = 0, n_sink: int = 0) -> int:
    """Number of (i, j) pairs with key j visible from query i, for one (b, h)."""
    if window <= 0 or window >= L:
        return L * (L + 1) // 2
    w = window
    total = w * (w + 1) // 2 + (L - w) * w        # row i sees min(i + 1, w) window keys
    for j in range(min(n_sink, L)):               # sink j seen again once it left the window
        first = j + w
        if first < L:
            total += L - first
    return total


def prefill_pairs(cfg: Prefill) -> int:
    return cfg.B * cfg.H * visible_pairs(cfg.L, cfg.window, cfg.n_sink)


def prefill_flops(cfg: Prefill) -> int:
    return 8 * cfg.d * prefill_pairs(cfg)


def prefill_bwd_flops(cfg: Prefill) -> int:
    return 16 * cfg.d * prefill_pairs(cfg)


def prefill_bytes(cfg: Prefill) -> int:
    """q, k, v, r read once (bf16) + o (fp32) and lse (fp32) written once."""
    n = cfg.B * cfg.H * cfg.L
    return n * cfg.d * 2 * 4 + n * cfg.d * 4 + n * 4


def decode_bytes(cfg: Decode) -> int:
    """K and V caches (bf16) once + q, r (bf16) + o (fp32) and lse (fp32)."""
    bh = cfg.B * cfg.H
    return bh * cfg.Lmax * cfg.d * 2 * 2 + bh * cfg.d * 2 * 2 + bh * cfg.d * 4 + bh * 4


def decode_flops(cfg: Decode) -> int:
    return 8 * cfg.d * cfg.B * cfg.H * cfg.Lmax
