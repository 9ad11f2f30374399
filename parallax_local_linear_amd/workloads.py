"""Seeded synthetic workloads (shapes and input draws only).

This module holds no arithmetic of the attention method: it fixes the five
workload shapes and draws their inputs, and both the GPU path and the CPU
oracle consume what it returns.

Inputs are i.i.d. standard normal draws from torch's generator on the given
device, seeded with the workload's number and drawn in the order q, k, v, r,
then scaled (prefill 0.6B-like only: by d^-1/4) and rounded to bf16.  The
pages measure on pretraining corpora and recall suites that are not
available; these Gaussian tensors stand in for them with the same shapes.
Shapes follow the pages' settings: 0.6B and 1.7B pretraining scale (review
page "Parallax: Parameterized Local Linear Attention for Language Modeling",
sec. 3), a sliding window of 128 keys ("Simple linear attention language
models balance the recall-throughput tradeoff" review, proposed method) and
4 attention sinks ("Sliding-window beats linear attention" review, sec. 3),
and a KV-cache decode step (tilnote note on Parallax).
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    seed: int
    B: int
    H: int
    L: int
    d: int
    scale_inputs: float = 1.0
    window: int = 0
    n_sink: int = 0


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    seed: int
    B: int
    H: int
    Lmax: int
    d: int
    num_splits: int = 16


@dataclasses.dataclass(frozen=True)
class Based:
    """Based linear attention layer: dk query/key features, dv value features."""
    name: str
    seed: int
    B: int
    H: int
    L: int
    dk: int
    dv: int
    scale: float


TINY = Prefill("tiny", 1, 1, 2, 256, 64)
PREFILL_06B = Prefill("prefill_0.6b", 2, 4, 16, 2048, 64, scale_inputs=64 ** -0.25)
PREFILL_17B = Prefill("prefill_1.7b_long", 3, 2, 16, 8192, 128)
LOCAL = Prefill("local_swa128_sink4", 4, 1, 16, 16384, 64, window=128, n_sink=4)
DECODE = Decode("decode_4k", 5, 64, 16, 4096, 128, num_splits=16)

# The 1.7B-like layer shape (16 heads, 8192 tokens, 128 value features) with
# Based's 16 query/key features; x = q.k / sqrt(16).
BASED = Based("based_1.7b_long", 6, 2, 16, 8192, 16, 128, 0.25)

PREFILLS = (TINY, PREFILL_06B, PREFILL_17B, LOCAL)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(cfg: Prefill, device="cpu", dtype=torch.bfloat16):
    """(q, k, v, r) of shape [B,H,L,d]; fp32 draws, scaled, then cast to dtype."""
    g = _gen(device, cfg.seed)
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    out = []
    for _ in range(4):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if cfg.scale_inputs != 1.0:
            x = x * cfg.scale_inputs
        out.append(x.to(dtype))
    return tuple(out)


def prefill_grad(cfg: Prefill, device="cpu", dtype=torch.bfloat16):
    """Output gradient dO for the backward of a prefill workload: i.i.d.
    N(0, 1) of shape [B,H,L,d], seeded with 1000 + the workload's number."""
    g = _gen(device, 1000 + cfg.seed)
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def decode_inputs(cfg: Decode, device="cpu", dtype=torch.bfloat16):
    """(q [B,H,d], k_cache [B,H,Lmax,d], v_cache, r [B,H,d]), drawn in that order."""
    g = _gen(device, cfg.seed)
    q = torch.randn((cfg.B, cfg.H, cfg.d), generator=g, device=device).to(dtype)
    k = torch.randn((cfg.B, cfg.H, cfg.Lmax, cfg.d), generator=g, device=device).to(dtype)
    v = torch.randn((cfg.B, cfg.H, cfg.Lmax, cfg.d), generator=g, device=device).to(dtype)
    r = torch.randn((cfg.B, cfg.H, cfg.d), generator=g, device=device).to(dtype)
    return q, k, v, r


def based_inputs(cfg: Based, device="cpu", dtype=torch.bfloat16):
    """(q [B,H,L,dk], k [B,H,L,dk], v [B,H,L,dv]), N(0,1), drawn in that order."""
    g = _gen(device, cfg.seed)
    q = torch.randn((cfg.B, cfg.H, cfg.L, cfg.dk), generator=g, device=device).to(dtype)
    k = torch.randn((cfg.B, cfg.H, cfg.L, cfg.dk), generator=g, device=device).to(dtype)
    v = torch.randn((cfg.B, cfg.H, cfg.L, cfg.dv), generator=g, device=device).to(dtype)
    return q, k, v


def rising_inputs(B: int, H: int, L: int, d: int, seed: int, device="cpu",
                  dtype=torch.bfloat16):
    """(q, k, v, r) whose attention scores rise along the sequence: with u a
    seeded random unit vector, q_i = 3u + 0.1 z, k_j = (46 (d/64)^1/2 j / L) u
    + 0.1 z, v ~ N(0, 1), r ~ 0.25 N(0, 1) (z i.i.d. N(0, 1)).  A row's later
    keys then score about 25 log2 units above its first ones."""
    g = _gen(device, seed)
    u = torch.randn(d, generator=g, device=device)
    u = u / u.norm()
    ramp = 46.0 * (d / 64) ** 0.5 * torch.arange(L, dtype=torch.float32, device=device) / L
    shape = (B, H, L, d)
    q = 3.0 * u + 0.1 * torch.randn(shape, generator=g, device=device)
    k = ramp[:, None] * u + 0.1 * torch.randn(shape, generator=g, device=device)
    v = torch.randn(shape, generator=g, device=device)
    r = 0.25 * torch.randn(shape, generator=g, device=device)
    return tuple(x.to(dtype) for x in (q, k, v, r))


def random_tensor(shape, seed: int, device="cpu", scale: float = 1.0, dtype=torch.bfloat16):
    """One seeded N(0, scale^2) tensor (edge-case tests)."""
    g = _gen(device, seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * scale).to(dtype)
