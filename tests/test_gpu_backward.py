"""GPU parity of the prefill backward against the fp64 oracle (MI355X only).

The forward for training (o, lse and the saved sbar, pv) and the backward
(dq, dk, dv, drho) run through the C ABI; the oracle's backward runs on the
same bf16 inputs and output gradient.  Whole gradients are compared at sizes
the oracle finishes in seconds (several tiles, ragged tails, windows,
sinks, the chunked sink path), and whole (b, h) slices at the full workload
sizes in the launch configuration the benchmark times.

Tolerance.  The accumulating products take bfloat16 operands (q, k, v, rho,
dO as given; the weights p t, dS and scale dZ rounded to bfloat16, relative
rounding at most 2^-9 ~ 2e-3 each), with float32 sums.  A gradient element
is a sum of many such terms of both signs, so its error is a small multiple
of 2^-9 times the size of the terms, which the size of the largest gradient
element bounds.  The bar: max |g - g_ref| <= 2e-2 * max |g_ref| + 1e-4 and
||g - g_ref|| <= 1e-2 ||g_ref|| + 1e-4 sqrt(n), per gradient and per case.
The absolute floor covers gradients that are exactly zero but come out of
float32 sums whose terms cancel (dq, dk and drho of a row that sees a single
key): terms like G_i = dO_i . pv_i reach about 4 sqrt(d) ~ 45, and times
|q| up to about 4 with a few roundings of 2^-24 each gives 1e-5 .. 1e-4.
"""
import numpy as np
import pytest
import torch

from gpu_util import default_scale, f64, say
from parallax_local_linear_amd import (parallax_attn_bwd, parallax_attn_fwd,
                                       parallax_attn_fwd_train, workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_TOL = 2e-2
L2_TOL = 1e-2
ABS_FLOOR = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def rand(shape, seed, scale=1.0):
    return workloads.random_tensor(shape, seed, device="cpu", scale=scale)


def compare_grads(got, ref, what):
    """got, ref: sequences of (name, array) with matching shapes."""
    worst = 0.0
    for (name, g), r in zip(got, ref):
        g = np.asarray(g, dtype=np.float64)
        r = np.asarray(r, dtype=np.float64)
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        assert np.isfinite(g).all(), "%s: non-finite %s" % (what, name)
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        den = float(np.linalg.norm(r))
        rel = float(np.linalg.norm(g - r)) / den if den > 0 else float(np.linalg.norm(g))
        say("[parity] %s %s: max|err|=%.3e (%.2e of max|ref| %.3e) relL2=%.3e"
            % (what, name, err, err / scale if scale else 0.0, scale, rel))
        assert err <= MAX_TOL * scale + ABS_FLOOR, \
            "%s %s: max|err| %.3e > %.0e * max|ref| %.3e + %.0e" % (what, name, err, MAX_TOL,
                                                                  scale, ABS_FLOOR)
        assert np.linalg.norm(g - r) <= L2_TOL * den + ABS_FLOOR * np.sqrt(r.size), \
            "%s %s: relL2 %.3e > %.0e" % (what, name, rel, L2_TOL)
        worst = max(worst, rel)
    return worst


def nan_grads(q):
    return tuple(torch.full(q.shape, float("nan"), device=DEV) for _ in range(4))


def run_gpu(q, k, v, r, do, scale, window, n_sink):
    o, lse, sbar, pv = parallax_attn_fwd_train(q, k, v, r, softmax_scale=scale, window=window,
                                               n_sink=n_sink)
    grads = parallax_attn_bwd(q, k, v, r, do, o, lse, sbar, pv, softmax_scale=scale,
                              window=window, n_sink=n_sink, grads=nan_grads(q))
    torch.cuda.synchronize()
    return grads


def full_check(orc, q, k, v, r, do, window=0, n_sink=0, scale=None, what=""):
    d = q.shape[-1]
    scale = default_scale(d) if scale is None else scale
    say("[case] %s shape=%s window=%d n_sink=%d" % (what, tuple(q.shape), window, n_sink))
    grads = run_gpu(*(x.to(DEV) for x in (q, k, v, r, do)), scale, window, n_sink)
    ref = orc.bwd(f64(q), f64(k), f64(v), f64(r), f64(do), scale=scale, window=window,
                  n_sink=n_sink)
    return compare_grads(list(zip(("dq", "dk", "dv", "dr"), (f64(g) for g in grads))), ref, what)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_train_outputs(orc, d):
    """o and lse equal the inference forward bit for bit; pv and sbar match the
    oracle: pv is the oracle with rho = 0, and sbar = rho . kbar with kbar the
    oracle with rho = 0 and v = k."""
    q, k, v, r = (rand((2, 2, 300, d), 10 + t + d) for t in range(4))
    for window, n_sink in ((0, 0), (64, 3)):
        qd, kd, vd, rd = (x.to(DEV) for x in (q, k, v, r))
        o, lse, sbar, pv = parallax_attn_fwd_train(qd, kd, vd, rd, window=window, n_sink=n_sink)
        o2, lse2 = parallax_attn_fwd(qd, kd, vd, rd, window=window, n_sink=n_sink)
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        zero = np.zeros(q.shape)
        pv_ref, _ = orc.fwd(f64(q), f64(k), f64(v), zero, window=window, n_sink=n_sink)
        kbar, _ = orc.fwd(f64(q), f64(k), f64(k), zero, window=window, n_sink=n_sink)
        sbar_ref = np.sum(f64(r) * kbar, axis=-1)
        e_pv = float(np.max(np.abs(f64(pv) - pv_ref)))
        e_s = float(np.max(np.abs(f64(sbar) - sbar_ref)))
        say("[parity] fwd_train d=%d W=%d S=%d: max|dpv|=%.3e max|dsbar|=%.3e"
            % (d, window, n_sink, e_pv, e_s))
        assert e_pv <= 2e-2 and e_s <= 2e-2 * max(1.0, float(np.max(np.abs(sbar_ref))))


def test_tiny_workload(orc):
    cfg = workloads.TINY
    q, k, v, r = workloads.prefill_inputs(cfg)
    do = rand(q.shape, 77)
    full_check(orc, q, k, v, r, do, what="tiny")


def test_tiny_probe_zero(orc):
    """rho = 0 (the oracle is pinned to softmax attention's autograd there)."""
    cfg = workloads.TINY
    q, k, v, _ = workloads.prefill_inputs(cfg)
    do = rand(q.shape, 78)
    full_check(orc, q, k, v, torch.zeros_like(q), do, what="tiny rho=0")


SMALL = [
    # (B, H, L, d, window, n_sink)
    (1, 2, 256, 64, 0, 0),
    (1, 1, 300, 128, 0, 0),
    (2, 1, 129, 128, 0, 0),
    (1, 1, 1, 64, 0, 0),
    (1, 1, 1, 128, 0, 0),
    (1, 1, 65, 128, 0, 0),
    (1, 1, 33, 64, 0, 0),
    (1, 2, 1000, 128, 0, 0),
    (1, 2, 1000, 64, 0, 0),
    (1, 2, 300, 128, 128, 4),
    (1, 1, 700, 64, 37, 70),
    (1, 1, 700, 128, 100, 200),
    (1, 1, 1000, 64, 64, 4),
    (1, 1, 1500, 128, 128, 4),
    (1, 1, 500, 64, 600, 0),
    (1, 1, 500, 128, 0, 5),
    (1, 1, 400, 64, 1, 0),
    (1, 1, 400, 128, 1, 3),
]


@pytest.mark.parametrize("B,H,L,d,window,n_sink", SMALL)
def test_small_shapes(orc, B, H, L, d, window, n_sink):
    seed = B * 1000003 + H * 10007 + L * 101 + d + window * 7 + n_sink
    q, k, v, r, do = (rand((B, H, L, d), seed + t) for t in range(5))
    full_check(orc, q, k, v, r, do, window=window, n_sink=n_sink,
               what="small B%d H%d L%d d%d" % (B, H, L, d))


def test_custom_scale(orc):
    q, k, v, r, do = (rand((1, 2, 400, 64), 950 + t, scale=0.5) for t in range(5))
    full_check(orc, q, k, v, r, do, scale=0.3, what="custom scale 0.3")


def test_strided_inputs_match_contiguous():
    """[B, L, H, d] storage viewed as [B, H, L, d] gives the same bits."""
    B, H, L, d = 1, 3, 333, 128
    base = [rand((B, L, H, d), 1300 + t).to(DEV) for t in range(5)]
    views = [x.permute(0, 2, 1, 3) for x in base]
    conts = [x.contiguous() for x in views]
    a = run_gpu(*views, default_scale(d), 100, 0)
    b = run_gpu(*conts, default_scale(d), 100, 0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_deterministic():
    """Causal: identical bits on repeated calls (no atomics on this path)."""
    q, k, v, r, do = (rand((2, 2, 700, 128), 1400 + t).to(DEV) for t in range(5))
    a = run_gpu(q, k, v, r, do, default_scale(128), 0, 0)
    b = run_gpu(q, k, v, r, do, default_scale(128), 0, 0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("cfg", [workloads.PREFILL_06B, workloads.PREFILL_17B, workloads.LOCAL],
                         ids=lambda c: c.name)
def test_full_size_slices(orc, cfg):
    """The benchmark workloads at full size; whole (b, h) slices against the oracle."""
    say("[case] full size backward %s" % cfg.name)
    q, k, v, r = workloads.prefill_inputs(cfg, device=DEV)
    do = workloads.prefill_grad(cfg, device=DEV)
    scale = default_scale(cfg.d)
    grads = run_gpu(q, k, v, r, do, scale, cfg.window, cfg.n_sink)
    for g in grads:
        assert torch.isfinite(g).all()
    pairs = [(0, 0), (cfg.B - 1, cfg.H - 1)]
    for b, h in pairs:
        sl = [f64(x[b:b + 1, h:h + 1]) for x in (q, k, v, r, do)]
        ref = orc.bwd(*sl, scale=scale, window=cfg.window, n_sink=cfg.n_sink)
        got = [(n, f64(g[b:b + 1, h:h + 1])) for n, g in zip(("dq", "dk", "dv", "dr"), grads)]
        compare_grads(got, ref, "%s b=%d h=%d" % (cfg.name, b, h))
