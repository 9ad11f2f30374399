"""Pins of the fp64 CPU oracle against facts outside the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` handle and raises AssertionError
when the oracle disagrees with the fact it is pinned to.  The same functions
run on the unmodified oracle (all must pass) and on builds with a planted
mistake (at least one must fail), so a plausible slip anywhere in the oracle
-- a dropped term, a wrong sign, an index or mask off by one, a transposed
operand -- is caught.

Facts used (none of them re-types the oracle's own two-pass algorithm):
  * the matrix closed form with brute-force mask enumeration (bruteforce.py);
  * rho = 0 reduces to softmax attention: torch's scaled_dot_product_attention
    and torch.logsumexp in fp64 on the CPU (library routines);
  * rho = Sigma_kk^-1 (q - kbar) reproduces the intercept of the weighted
    least-squares local linear fit (the LLA estimator that Parallax
    parameterises), solved by numpy.linalg.lstsq;
  * closed forms: a single visible key gives o = v, lse = scale q.k;
  * invariants: key translation, value affinity, linearity in rho;
  * a hand-worked example with exact rational results (tests/golden);
  * backward: central differences of the (pinned) forward, torch's autograd
    of softmax attention at rho = 0, and exact identities (key translation,
    value shift, linearity in V, affinity in rho);
  * Walsh-Hadamard output projection: scipy.linalg.hadamard and the
    popcount closed form of the Sylvester matrix, orthogonality (norms kept,
    the transform its own inverse), and the closed form of a constant row;
  * Based linear attention: the state-space recurrence of the explicit
    feature map, the weight as a function of x recovered from outputs (a
    polynomial of degree two matching exp's value and first two derivatives
    at 0), softmax attention as its small-x limit, and closed forms (equal
    weights give prefix means, one key gives its value).
Sources: review page "Parallax: Parameterized Local Linear Attention for
Language Modeling", sec. 1-3; tilnote note on Parallax, section on Local
Linear Attention as the starting point; "Sliding-window beats linear
attention" review, sec. 1 (windows and sinks); "Rethinking Attention Output
Projection: Structured Hadamard Transforms for Efficient Transformers"
review, sec. 2; "Simple linear attention language models balance the
recall-throughput tradeoff" review, "Proposed method".
"""
from __future__ import annotations

import json
import os

import numpy as np

from bruteforce import closed_form, visible_mask

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL = 1e-11


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * scale


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a) == np.isfinite(b)), what + ": finiteness differs"
    fin = np.isfinite(b)
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]) / (1.0 + np.abs(b[fin])))
        assert err <= tol, "%s: max rel err %.3e > %.1e" % (what, err, tol)


MASKS = [(0, 0), (1, 0), (3, 0), (5, 2), (2, 4), (0, 3), (64, 0)]


def pin_closed_form(orc):
    """Oracle == matrix closed form (brute-force masks), several masks and d."""
    for d, L in ((3, 9), (8, 17)):
        for seed, (window, n_sink) in enumerate(MASKS):
            q, k, v, r = (_rand((2, 2, L, d), 100 * seed + t + d) for t in range(4))
            o, lse = orc.fwd(q, k, v, r, window=window, n_sink=n_sink)
            o2, lse2 = closed_form(q, k, v, r, window=window, n_sink=n_sink)
            _close(o, o2, what="O closed form W=%d S=%d" % (window, n_sink))
            _close(lse, lse2, what="LSE closed form W=%d S=%d" % (window, n_sink))


def pin_softmax_special_case(orc):
    """rho = 0 gives exactly softmax attention (torch SDPA, fp64, CPU)."""
    import torch
    import torch.nn.functional as F
    for seed, (window, n_sink) in enumerate(MASKS):
        B, H, L, d = 1, 2, 13, 8
        q, k, v = (_rand((B, H, L, d), 7 + 3 * seed + t) for t in range(3))
        r = np.zeros_like(q)
        scale = 1.0 / np.sqrt(d)
        o, lse = orc.fwd(q, k, v, r, scale=scale, window=window, n_sink=n_sink)
        mask = torch.from_numpy(visible_mask(L, window, n_sink))
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        scores = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        scores = scores.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1)
        _close(o, ref.numpy(), what="O vs SDPA W=%d S=%d" % (window, n_sink))
        _close(lse, ref_lse.numpy(), what="LSE vs logsumexp W=%d S=%d" % (window, n_sink))


def _softmax_weights(q, K, scale, vis):
    z = scale * (K[vis] @ q)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def pin_local_linear_fit(orc):
    """With rho = Sigma_kk^-1 (q - kbar) the output is the weighted LLS intercept.

    The local linear estimate at the query point fits v ~ a + B (k - q) with
    the softmax weights and reports a; the probe form sum p (1 + rho.(k-kbar)) v
    equals it for this rho.  Checked on rows with more visible keys than d.
    """
    for (window, n_sink) in ((0, 0), (9, 2)):
        B, H, L, d = 1, 1, 16, 3
        q, k, v = (_rand((B, H, L, d), 31 + t + window) for t in range(3))
        scale = 1.0 / np.sqrt(d)
        mask = visible_mask(L, window, n_sink)
        r = np.zeros_like(q)
        rows = [i for i in range(L) if mask[i].sum() >= d + 2]
        for i in rows:
            vis = mask[i]
            K = k[0, 0]
            p = _softmax_weights(q[0, 0, i], K, scale, vis)
            Kv = K[vis]
            kbar = p @ Kv
            cov = (Kv - kbar).T @ ((Kv - kbar) * p[:, None])
            r[0, 0, i] = np.linalg.solve(cov, q[0, 0, i] - kbar)
        o, _ = orc.fwd(q, k, v, r, scale=scale, window=window, n_sink=n_sink)
        for i in rows:
            vis = mask[i]
            K = k[0, 0]
            p = _softmax_weights(q[0, 0, i], K, scale, vis)
            X = np.concatenate([np.ones((vis.sum(), 1)), K[vis] - q[0, 0, i]], axis=1)
            w = np.sqrt(p)[:, None]
            coef, *_ = np.linalg.lstsq(X * w, v[0, 0][vis] * w, rcond=None)
            _close(o[0, 0, i], coef[0], tol=1e-9, what="LLS intercept row %d" % i)


def pin_single_key(orc):
    """One visible key: o = v_j and lse = scale * q.k_j (row 0; window 1)."""
    B, H, L, d = 2, 1, 6, 5
    q, k, v, r = (_rand((B, H, L, d), 50 + t) for t in range(4))
    scale = 0.37
    o, lse = orc.fwd(q, k, v, r, scale=scale)
    _close(o[:, :, 0], v[:, :, 0], what="row 0 output")
    _close(lse[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), what="row 0 lse")
    o, lse = orc.fwd(q, k, v, r, scale=scale, window=1)
    _close(o, v, what="window 1 output")
    _close(lse, scale * np.sum(q * k, axis=-1), what="window 1 lse")


def pin_key_translation(orc):
    """k_j -> k_j + u: o unchanged, lse shifted by scale * q.u."""
    B, H, L, d = 1, 2, 11, 4
    q, k, v, r = (_rand((B, H, L, d), 60 + t) for t in range(4))
    u = _rand((d,), 99) * 3.0
    scale = 0.5
    for (window, n_sink) in ((0, 0), (3, 2)):
        o, lse = orc.fwd(q, k, v, r, scale=scale, window=window, n_sink=n_sink)
        o2, lse2 = orc.fwd(q, k + u, v, r, scale=scale, window=window, n_sink=n_sink)
        _close(o2, o, tol=1e-10, what="translated keys output")
        _close(lse2, lse + scale * (q @ u), tol=1e-10, what="translated keys lse")


def pin_value_affine(orc):
    """v_j -> v_j + w gives o + w; constant values give constant outputs."""
    B, H, L, d = 1, 1, 10, 6
    q, k, v, r = (_rand((B, H, L, d), 70 + t) for t in range(4))
    w = _rand((d,), 77)
    o, _ = orc.fwd(q, k, v, r)
    o2, _ = orc.fwd(q, k, v + w, r)
    _close(o2, o + w, tol=1e-10, what="value shift")
    o3, _ = orc.fwd(q, k, np.ones_like(v), r, window=4, n_sink=1)
    _close(o3, np.ones_like(v), tol=1e-10, what="constant values")


def pin_rho_linearity(orc):
    """o is affine in rho: o(a rho) = o(0) + a (o(rho) - o(0))."""
    B, H, L, d = 1, 1, 9, 4
    q, k, v, r = (_rand((B, H, L, d), 80 + t) for t in range(4))
    o0, _ = orc.fwd(q, k, v, np.zeros_like(r))
    o1, _ = orc.fwd(q, k, v, r)
    oa, _ = orc.fwd(q, k, v, -2.5 * r)
    _close(oa, o0 - 2.5 * (o1 - o0), tol=1e-10, what="rho linearity")


def pin_masks(orc):
    """Window >= L equals causal; sinks without a window change nothing."""
    B, H, L, d = 1, 1, 12, 4
    q, k, v, r = (_rand((B, H, L, d), 90 + t) for t in range(4))
    base = orc.fwd(q, k, v, r)
    for window, n_sink in ((L, 0), (L + 5, 3), (0, 4)):
        o, lse = orc.fwd(q, k, v, r, window=window, n_sink=n_sink)
        _close(o, base[0], what="mask W=%d S=%d vs causal" % (window, n_sink))
        _close(lse, base[1], what="mask lse W=%d S=%d vs causal" % (window, n_sink))


def pin_golden(orc):
    """Hand-worked uniform-weight example (tests/golden/uniform_weights.json)."""
    with open(os.path.join(GOLDEN, "uniform_weights.json")) as f:
        g = json.load(f)
    shape = (1, 1, g["L"], g["d"])
    q, k, v, r = (np.array(g[n], dtype=np.float64).reshape(shape) for n in "qkvr")
    for case in g["cases"]:
        o, lse = orc.fwd(q, k, v, r, scale=g["scale"], window=case["window"],
                         n_sink=case["n_sink"])
        _close(o[0, 0], np.array(case["o"], dtype=np.float64), tol=1e-14,
               what="golden O W=%d S=%d" % (case["window"], case["n_sink"]))
        _close(lse[0, 0], np.log(np.array(case["lse_n_visible"], dtype=np.float64)),
               tol=1e-14, what="golden LSE W=%d S=%d" % (case["window"], case["n_sink"]))


def pin_decode(orc):
    """A decode row equals the prefill row at position seqlen-1; seqlen 0 is empty."""
    B, H, Lmax, d = 3, 2, 9, 4
    k, v = (_rand((B, H, Lmax, d), 110 + t) for t in range(2))
    q, r = (_rand((B, H, d), 120 + t) for t in range(2))
    seqlens = [9, 4, 0]
    o, lse = orc.decode(q, r, k, v, seqlens=seqlens, scale=0.4)
    for b, n in enumerate(seqlens):
        if n == 0:
            assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b])), "empty decode row"
            continue
        qq = np.zeros((1, H, n, d))
        rr = np.zeros((1, H, n, d))
        qq[0, :, n - 1] = q[b]
        rr[0, :, n - 1] = r[b]
        o2, lse2 = closed_form(qq, k[b:b + 1, :, :n], v[b:b + 1, :, :n], rr, scale=0.4)
        _close(o[b], o2[0, :, n - 1], what="decode row b=%d" % b)
        _close(lse[b], lse2[0, :, n - 1], what="decode lse b=%d" % b)


def pin_decode_general(orc):
    """General decode: a row with a window and sinks equals the prefill row at
    position seqlen-1 (matrix closed form), and grouped kv heads equal the
    plain decode with each kv head repeated for its query heads."""
    B, Hq, Hkv, Lmax, d = 3, 4, 2, 40, 5
    k, v = (_rand((B, Hkv, Lmax, d), 130 + t) for t in range(2))
    q, r = (_rand((B, Hq, d), 140 + t) for t in range(2))
    seqlens = [40, 17, 0]
    g = Hq // Hkv
    for window, n_sink in ((0, 0), (6, 2), (3, 0), (1, 4)):
        o, lse = orc.decode_ext(q, r, k, v, seqlens=seqlens, scale=0.45, window=window,
                                n_sink=n_sink)
        o_rep, lse_rep = orc.decode_ext(q, r, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1),
                                        seqlens=seqlens, scale=0.45, window=window, n_sink=n_sink)
        _close(o, o_rep, what="grouped kv heads vs repeated W=%d S=%d" % (window, n_sink))
        _close(lse, lse_rep, what="grouped kv lse vs repeated W=%d S=%d" % (window, n_sink))
        for b, n in enumerate(seqlens):
            if n == 0:
                assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b])), "empty decode row"
                continue
            for h in range(Hq):
                qq = np.zeros((1, 1, n, d))
                rr = np.zeros((1, 1, n, d))
                qq[0, 0, n - 1] = q[b, h]
                rr[0, 0, n - 1] = r[b, h]
                kk = k[b:b + 1, h // g:h // g + 1, :n]
                vv = v[b:b + 1, h // g:h // g + 1, :n]
                o2, lse2 = closed_form(qq, kk, vv, rr, scale=0.45, window=window, n_sink=n_sink)
                _close(o[b, h], o2[0, 0, n - 1], what="decode row b=%d h=%d W=%d S=%d"
                       % (b, h, window, n_sink))
                _close(lse[b, h], lse2[0, 0, n - 1], what="decode lse b=%d h=%d" % (b, h))


def _weighted_fit_intercept(q, K, V, scale, vis, ridge=0.0):
    """Intercept a of min sum_j p_j |v_j - a - B (k_j - q)|^2 + ridge |B|^2 (numpy lstsq)."""
    p = _softmax_weights(q, K, scale, vis)
    Kv, Vv = K[vis], V[vis]
    X = np.concatenate([np.ones((len(p), 1)), Kv - q], axis=1) * np.sqrt(p)[:, None]
    Y = Vv * np.sqrt(p)[:, None]
    if ridge > 0:
        d = K.shape[1]
        X = np.concatenate([X, np.concatenate([np.zeros((d, 1)), np.sqrt(ridge) * np.eye(d)],
                                              axis=1)])
        Y = np.concatenate([Y, np.zeros((d, V.shape[1]))])
    coef, *_ = np.linalg.lstsq(X, Y, rcond=None)
    return coef[0]


def pin_lla_conjugate_gradient(orc):
    """Exact LLA by CG equals the weighted least-squares intercept (numpy lstsq),
    with and without a ridge, and the Parallax form with the CG probe gives the
    same output."""
    L, d = 24, 4
    rng_q, rng_k, rng_v = (_rand((L, d), 700 + t) for t in range(3))
    scale = 0.5
    for window, n_sink, ridge in ((0, 0, 0.0), (12, 2, 0.0), (0, 0, 0.3), (7, 1, 0.05)):
        mask = visible_mask(L, window, n_sink)
        rows = [i for i in range(L) if mask[i].sum() >= d + 2 or ridge > 0]
        o, rho, iters = orc.lla_rows(rng_q[rows], rows, rng_k, rng_v, scale, window, n_sink,
                                     ridge=ridge)
        assert np.all(iters <= 4 * d)
        for n, i in enumerate(rows):
            ref = _weighted_fit_intercept(rng_q[i], rng_k, rng_v, scale, mask[i], ridge)
            _close(o[n], ref, tol=1e-9, what="LLA CG intercept row %d W=%d S=%d ridge=%g"
                   % (i, window, n_sink, ridge))
        r_full = np.zeros((1, 1, L, d))
        r_full[0, 0, rows] = rho
        o_plx, _ = orc.fwd(rng_q[None, None], rng_k[None, None], rng_v[None, None], r_full,
                           scale=scale, window=window, n_sink=n_sink)
        _close(o_plx[0, 0, rows], o, tol=1e-10, what="Parallax with the LLA probe")


def pin_projection(orc):
    """Fused projections equal numpy's matmul x @ w.T; an identity block of w
    copies the matching columns of x."""
    x = _rand((37, 64), 801)
    w = _rand((40, 64), 802)
    _close(orc.project(x, w), x @ w.T, tol=1e-12, what="projection vs numpy matmul")
    eye = np.zeros((16, 64))
    eye[:, 8:24] = np.eye(16)
    _close(orc.project(x, eye), x[:, 8:24], tol=0.0, what="projection with an identity block")


# ---------------------------------------------------------------------------
# Backward.  The loss is Lambda = sum dO . o (so dO is dLambda/do); lse takes
# no part in it.  The pins below use the forward oracle (itself pinned above)
# through finite differences, torch's autograd of softmax attention, and four
# exact identities of the method.

BWD_MASKS = [(0, 0), (3, 1), (2, 3), (1, 0)]


def _loss(orc, q, k, v, r, dout, **kw):
    o, _ = orc.fwd(q, k, v, r, nthreads=1, **kw)
    return float(np.sum(o * dout))


def pin_bwd_finite_differences(orc):
    """Every gradient element equals the central difference of the forward.

    h = 1e-5 in fp64: the truncation error (h^2 times a third derivative of
    order one) and the rounding error (1e-16 / h) both stay below 1e-8.
    """
    B, H, L, d = 1, 2, 7, 4
    for seed, (window, n_sink) in enumerate(BWD_MASKS):
        ins = [_rand((B, H, L, d), 200 + 10 * seed + t) for t in range(5)]
        q, k, v, r, dout = ins
        kw = dict(scale=0.6, window=window, n_sink=n_sink)
        grads = orc.bwd(q, k, v, r, dout, nthreads=1, **kw)
        h = 1e-5
        for x_idx, (name, g) in enumerate(zip("qkvr", grads)):
            fd = np.zeros_like(g)
            for e in np.ndindex(*g.shape):
                xs = [a.copy() for a in (q, k, v, r)]
                xs[x_idx][e] += h
                up = _loss(orc, *xs, dout, **kw)
                xs[x_idx][e] -= 2 * h
                dn = _loss(orc, *xs, dout, **kw)
                fd[e] = (up - dn) / (2 * h)
            _close(g, fd, tol=1e-7, what="d%s vs finite differences W=%d S=%d"
                   % (name, window, n_sink))


def pin_bwd_directional(orc):
    """Directional derivatives on larger slices (several tiles of keys)."""
    B, H, L, d = 2, 1, 33, 16
    for seed, (window, n_sink) in enumerate(((0, 0), (8, 2), (5, 0))):
        q, k, v, r, dout = (_rand((B, H, L, d), 300 + 10 * seed + t) for t in range(5))
        kw = dict(scale=d ** -0.5, window=window, n_sink=n_sink)
        grads = orc.bwd(q, k, v, r, dout, **kw)
        h = 1e-5
        for x_idx, (name, g) in enumerate(zip("qkvr", grads)):
            u = _rand(g.shape, 400 + 10 * seed + x_idx)
            xs = [a.copy() for a in (q, k, v, r)]
            xs[x_idx] += h * u
            up = _loss(orc, *xs, dout, **kw)
            xs[x_idx] -= 2 * h * u
            dn = _loss(orc, *xs, dout, **kw)
            fd = (up - dn) / (2 * h)
            got = float(np.sum(g * u))
            assert abs(got - fd) <= 1e-7 * (1.0 + abs(fd)), \
                "d%s along a direction: %.12g vs %.12g (W=%d S=%d)" % (name, got, fd, window, n_sink)


def pin_bwd_softmax_case(orc):
    """rho = 0: dq, dk, dv equal torch's autograd of softmax attention (fp64)."""
    import torch
    import torch.nn.functional as F
    B, H, L, d = 1, 2, 13, 8
    for seed, (window, n_sink) in enumerate(MASKS):
        q, k, v, dout = (_rand((B, H, L, d), 500 + 5 * seed + t) for t in range(4))
        scale = d ** -0.5
        dq, dk, dv, _ = orc.bwd(q, k, v, np.zeros_like(q), dout, scale=scale,
                                window=window, n_sink=n_sink)
        mask = torch.from_numpy(visible_mask(L, window, n_sink))
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        o.backward(torch.from_numpy(dout))
        for name, a, t in (("dq", dq, tq), ("dk", dk, tk), ("dv", dv, tv)):
            _close(a, t.grad.numpy(), what="%s vs autograd SDPA W=%d S=%d" % (name, window, n_sink))


def pin_bwd_identities(orc):
    """Four exact identities of the method.

    * Translating every key by u leaves o unchanged (the scores move by
      scale q.u for all keys of a row, and k_j - kbar is unchanged), so the
      key gradients of a slice sum to zero.
    * sum_j p_j (1 + c_j) = 1, so adding w to every value adds w to every
      output: the value gradients sum to the output gradients.
    * o is linear in V, so sum_j dv_j . v_j = sum_i dO_i . o_i.
    * o is affine in rho, so sum_i drho_i . rho_i = sum_i dO_i . (o_i - o_i|rho=0).
    """
    B, H, L, d = 1, 3, 64, 8
    for seed, (window, n_sink) in enumerate(((0, 0), (16, 4), (7, 0))):
        q, k, v, r, dout = (_rand((B, H, L, d), 600 + 10 * seed + t) for t in range(5))
        kw = dict(scale=0.4, window=window, n_sink=n_sink)
        dq, dk, dv, dr = orc.bwd(q, k, v, r, dout, **kw)
        o, _ = orc.fwd(q, k, v, r, **kw)
        o0, _ = orc.fwd(q, k, v, np.zeros_like(r), **kw)
        tag = " W=%d S=%d" % (window, n_sink)
        mag = np.abs(dk).sum(axis=2)
        assert np.all(np.abs(dk.sum(axis=2)) <= 1e-11 * (1.0 + mag)), "sum of dk" + tag
        _close(dv.sum(axis=2), dout.sum(axis=2), tol=1e-11, what="sum of dv" + tag)
        _close(np.sum(dv * v, axis=(2, 3)), np.sum(dout * o, axis=(2, 3)), tol=1e-11,
               what="dv . v" + tag)
        _close(np.sum(dr * r, axis=(2, 3)), np.sum(dout * (o - o0), axis=(2, 3)), tol=1e-11,
               what="drho . rho" + tag)


# ---------------------------------------------------------------------------
# Walsh-Hadamard output projection and Based linear attention.

def pin_hadamard_library(orc):
    """sqrt(n) times the transform of the identity is scipy.linalg.hadamard(n);
    entry (k, c) has the sign (-1)^popcount(k & c)."""
    from scipy.linalg import hadamard
    for n in (1, 2, 4, 8, 16, 64, 256, 512):
        h = orc.hadamard(np.eye(n)) * np.sqrt(n)
        _close(h, hadamard(n).astype(np.float64), tol=1e-12, what="H_%d vs scipy" % n)
    n = 128
    h = orc.hadamard(np.eye(n)) * np.sqrt(n)
    kk, cc = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    sign = 1.0 - 2.0 * (np.vectorize(lambda a: bin(a).count("1"))(kk & cc) % 2)
    _close(h, sign, tol=1e-12, what="H_128 vs popcount signs")


def pin_hadamard_orthogonal(orc):
    """Without the affine map the transform keeps every row's l2 norm and is its
    own inverse (the normalised Sylvester matrix is symmetric and orthogonal)."""
    y = _rand((6, 2048), 901)
    t = orc.hadamard(y)
    _close(np.linalg.norm(t, axis=1), np.linalg.norm(y, axis=1), tol=1e-12, what="norms kept")
    _close(orc.hadamard(t), y, tol=1e-12, what="transform twice is the identity")


def pin_hadamard_affine(orc):
    """A constant row c maps to c sqrt(n) at feature 0 and 0 elsewhere, so the
    output is alpha_0 c sqrt(n) + beta_0 at 0 and beta elsewhere; for any
    input, alpha and beta act on the transformed features."""
    n = 256
    alpha, beta = _rand(n, 902) + 2.0, _rand(n, 903)
    c = 0.75
    out = orc.hadamard(np.full((1, n), c), alpha, beta)[0]
    want = beta.copy()
    want[0] += alpha[0] * c * np.sqrt(n)
    _close(out, want, tol=1e-12, what="constant row")
    y = _rand((5, n), 904)
    _close(orc.hadamard(y, alpha, beta), alpha * orc.hadamard(y) + beta, tol=1e-12,
           what="affine map after the transform")


def _based_features(u, scale):
    """phi(u) = [1, sqrt(scale) u, (scale / sqrt 2) vec(u u^T)], so that
    phi(q) . phi(k) = 1 + x + x^2 / 2 with x = scale q . k."""
    quad = np.einsum("...a,...b->...ab", u, u).reshape(u.shape[:-1] + (-1,))
    one = np.ones(u.shape[:-1] + (1,))
    return np.concatenate([one, np.sqrt(scale) * u, scale / np.sqrt(2.0) * quad], axis=-1)


def pin_based_recurrence(orc):
    """The causal sum equals linear attention's recurrence on the explicit
    feature map: state S_i = S_{i-1} + phi(k_i) [v_i, 1]^T, o_i = phi(q_i) S_i
    split into numerator and denominator."""
    for (dk, dv, L, scale) in [(4, 3, 9, 0.5), (3, 5, 17, 0.9)]:
        q, k, v = (_rand((1, 2, L, dd), 910 + dd + t) for t, dd in enumerate((dk, dk, dv)))
        o = orc.based(q, k, v, scale=scale)
        for h in range(2):
            fq, fk = _based_features(q[0, h], scale), _based_features(k[0, h], scale)
            vv = np.concatenate([v[0, h], np.ones((L, 1))], axis=1)
            state = np.zeros((fq.shape[1], dv + 1))
            for i in range(L):
                state += np.outer(fk[i], vv[i])
                num = fq[i] @ state
                _close(o[0, h, i], num[:dv] / num[dv], tol=1e-12,
                       what="recurrence dk=%d row %d" % (dk, i))


def pin_based_taylor_weight(orc):
    """The weight of a key as a function of x = scale q.k, read off outputs
    (key 0 at x = 0 with value 0, key 1 at x with value 1: o_1 = w / (1 + w)),
    is a polynomial of degree two with exp's value, slope and curvature at 0,
    i.e. the second-order Taylor polynomial of exp."""
    scale, h = 0.5, 0.25
    xs = h * np.arange(-3, 4)
    ws = []
    for x in xs:
        q = np.array([[[[1.0, 2.0], [1.0, 2.0]]]])
        kx = x / (scale * 5.0)
        k = np.array([[[[0.0, 0.0], [kx, 2.0 * kx]]]])
        v = np.array([[[[0.0], [1.0]]]])
        o = orc.based(q, k, v, scale=scale)[0, 0, 1, 0]
        ws.append(o / (1.0 - o))
    ws = np.array(ws)
    c = 3  # index of x = 0
    _close(ws[c], 1.0, tol=1e-12, what="w(0)")
    _close((ws[c + 1] - ws[c - 1]) / (2 * h), 1.0, tol=1e-11, what="slope at 0")
    _close((ws[c + 1] - 2 * ws[c] + ws[c - 1]) / h ** 2, 1.0, tol=1e-10, what="curvature at 0")
    third = ws[3:] - 3 * ws[2:-1] + 3 * ws[1:-2] - ws[:-3]
    _close(third, np.zeros_like(third), tol=1e-12, what="third differences vanish")


def pin_based_closed_forms(orc):
    """q = 0 gives equal weights, so o_i is the mean of v_0..v_i; row 0 sees
    only its own key, so o_0 = v_0; o is affine in the values."""
    B, H, L, dk, dv = 1, 2, 11, 4, 6
    k, v = _rand((B, H, L, dk), 920), _rand((B, H, L, dv), 921)
    o = orc.based(np.zeros((B, H, L, dk)), k, v)
    means = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    _close(o, means, tol=1e-12, what="prefix means")
    q = _rand((B, H, L, dk), 922)
    o = orc.based(q, k, v)
    _close(o[:, :, 0], v[:, :, 0], tol=1e-12, what="row 0")
    shift = _rand(dv, 923)
    _close(orc.based(q, k, 2.5 * v + shift), 2.5 * o + shift, tol=1e-12, what="value affine")


def pin_based_softmax_limit(orc):
    """For small x the weight 1 + x + x^2/2 is exp(x) (1 - r) with
    |r| <= |x|^3 e^|x| / 6, so the output stays within
    2 max|r| / (1 - max|r|) * max|v - o| of softmax attention (the Parallax
    oracle at rho = 0)."""
    B, H, L, d = 1, 2, 40, 8
    q, k = (_rand((B, H, L, d), 930 + t, scale=0.3) for t in range(2))
    v = _rand((B, H, L, d), 932)
    scale = d ** -0.5
    o = orc.based(q, k, v, scale=scale)
    o_sm, _ = orc.fwd(q, k, v, np.zeros_like(q), scale=scale)
    xmax = float(np.max(np.abs(scale * np.einsum("bhid,bhjd->bhij", q, k))))
    rmax = xmax ** 3 * np.exp(xmax) / 6.0
    bound = 2.0 * rmax / (1.0 - rmax) * 2.0 * float(np.max(np.abs(v)))
    err = float(np.max(np.abs(o - o_sm)))
    assert err <= bound, "softmax limit: %.3e > %.3e" % (err, bound)


ALL_PINS = [pin_closed_form, pin_softmax_special_case, pin_local_linear_fit,
            pin_single_key, pin_key_translation, pin_value_affine, pin_rho_linearity,
            pin_masks, pin_golden, pin_decode, pin_decode_general, pin_lla_conjugate_gradient,
            pin_projection,
            pin_bwd_finite_differences, pin_bwd_directional, pin_bwd_softmax_case,
            pin_bwd_identities,
            pin_hadamard_library, pin_hadamard_orthogonal, pin_hadamard_affine,
            pin_based_recurrence, pin_based_taylor_weight, pin_based_closed_forms,
            pin_based_softmax_limit]
