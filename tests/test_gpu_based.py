"""GPU parity of Based linear attention (prefill and decode) against the fp64
oracle (MI355X only).

The oracle sums w_ij v_j / sum w_ij pairwise with w_ij = 1 + x + x^2/2.  The
prefill instead carries a state: phi(q) and the prefix state S reach the
matrix cores as bf16 (relative rounding 2^-8 each), phi(k), v and the
in-segment weights as f16, all sums in fp32.  The numerator's error is then
at most about 2^-7 sum_f |phi_f(q)| |S_fc| <= 2^-7 sum_j wt_ij |v_jc| and the
normaliser's 2^-7 sum_j wt_ij, where wt_ij = sum_f |phi_f(q_i) phi_f(k_j)|
= 1 + s a + (s^2/2) a^2 with a = sum_t |q_it k_jt|.  So per element

    |o - o_ref| <= 2^-7 (sum_j wt_ij |v_jc| + |o_ref| sum_j wt_ij) / sum_j w_ij.

The decode works in fp32 on the state the prefill returned; its bar is the
same (the state carries the prefill's rounding)."""
import numpy as np
import pytest
import torch

from gpu_util import f64, say
from parallax_local_linear_amd import (based_state_shape, parallax_based_decode,
                                       parallax_based_fwd, workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def bound_rows(q, k, v, rows, scale, ref_rows):
    """The per-element bar above for rows `rows` of one (b, h) slice (fp64)."""
    out = np.zeros_like(ref_rows)
    for n, i in enumerate(rows):
        x = scale * (k[: i + 1] @ q[i])
        w = 1.0 + x + 0.5 * x * x
        a = np.abs(k[: i + 1]) @ np.abs(q[i])
        wt = 1.0 + scale * a + 0.5 * (scale * a) ** 2
        out[n] = 2.0 ** -7 * (wt @ np.abs(v[: i + 1]) + np.abs(ref_rows[n]) * wt.sum()) / w.sum()
    return out


def check_rows(o_gpu, ref, q, k, v, rows, scale, what):
    got = np.asarray(o_gpu, dtype=np.float64)
    assert np.isfinite(got).all(), what + ": non-finite output"
    bound = bound_rows(q, k, v, rows, scale, ref)
    err = np.abs(got - ref)
    worst = float(np.max(err / bound))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say("[parity] %s: max|err|=%.3e relL2=%.3e worst err/bound=%.3f" % (what, float(err.max()),
                                                                        rel, worst))
    assert worst <= 1.0, what


def run(orc, B, H, L, dv, seed, strided=False):
    scale = 0.25
    q, k = (workloads.random_tensor((B, H, L, 16), seed + t) for t in range(2))
    v = workloads.random_tensor((B, H, L, dv), seed + 2)
    if strided:
        # token-major storage [B, L, H, d] viewed as [B, H, L, d]
        qd, kd, vd = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3).to(DEV)
                      for t in (q, k, v))
    else:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, state = parallax_based_fwd(qd, kd, vd, scale=scale, return_state=True)
    torch.cuda.synchronize()
    ref = orc.based(f64(q), f64(k), f64(v), scale=scale)
    og = f64(o)
    for b in range(B):
        for h in range(H):
            check_rows(og[b, h], ref[b, h], f64(q)[b, h], f64(k)[b, h], f64(v)[b, h],
                       np.arange(L), scale, "based B=%d H=%d L=%d dv=%d (%d,%d)%s"
                       % (B, H, L, dv, b, h, " strided" if strided else ""))
    return q, k, v, o, state


@pytest.mark.parametrize("B,H,L,dv", [
    (1, 2, 300, 128),    # one ragged segment
    (2, 3, 1100, 64),    # three segments, ragged
    (1, 2, 512, 128),    # exactly one segment
    (1, 1, 1537, 128),   # four segments, one-token tail
    (1, 1, 1, 128),      # a single token
    (1, 1, 257, 64),     # one token past an output tile
])
def test_based_prefill(orc, B, H, L, dv):
    say("[case] based prefill B=%d H=%d L=%d dv=%d" % (B, H, L, dv))
    run(orc, B, H, L, dv, 8000 + L + dv)


def test_based_prefill_strided(orc):
    say("[case] based prefill strided")
    run(orc, 2, 2, 700, 128, 8100, strided=True)


def test_based_final_state_and_decode(orc):
    """Prefill of L-1 tokens returns the state; two decode steps then give
    rows L-1 and L of the oracle on the whole sequence."""
    B, H, L, dv = 2, 2, 1030, 128
    scale = 0.25
    say("[case] based prefill + decode B=%d H=%d L=%d" % (B, H, L))
    q, k = (workloads.random_tensor((B, H, L + 1, 16), 8200 + t) for t in range(2))
    v = workloads.random_tensor((B, H, L + 1, dv), 8202)
    _, state = parallax_based_fwd(q[:, :, : L - 1].to(DEV), k[:, :, : L - 1].to(DEV),
                                  v[:, :, : L - 1].to(DEV), scale=scale, return_state=True)
    assert tuple(state.shape) == (B, H) + based_state_shape(dv)
    outs = []
    for t in (L - 1, L):
        outs.append(parallax_based_decode(q[:, :, t].contiguous().to(DEV),
                                          k[:, :, t].contiguous().to(DEV),
                                          v[:, :, t].contiguous().to(DEV), state, scale=scale))
    torch.cuda.synchronize()
    ref = orc.based(f64(q), f64(k), f64(v), scale=scale)
    for n, t in enumerate((L - 1, L)):
        for b in range(B):
            for h in range(H):
                check_rows(f64(outs[n])[b, h][None], ref[b, h, t][None], f64(q)[b, h],
                           f64(k)[b, h], f64(v)[b, h], [t], scale,
                           "based decode step %d (%d,%d)" % (t, b, h))


def test_based_decode_from_zero_state(orc):
    """A zero state starts a sequence: the first output is v_0, then rows 1, 2."""
    B, H, dv = 3, 2, 64
    scale = 0.25
    q, k = (workloads.random_tensor((B, H, 3, 16), 8300 + t) for t in range(2))
    v = workloads.random_tensor((B, H, 3, dv), 8302)
    state = torch.zeros((B, H) + based_state_shape(dv), dtype=torch.float32, device=DEV)
    outs = [parallax_based_decode(q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
                                  v[:, :, t].contiguous().to(DEV), state, scale=scale)
            for t in range(3)]
    torch.cuda.synchronize()
    ref = orc.based(f64(q), f64(k), f64(v), scale=scale)
    for t in range(3):
        err = float(np.max(np.abs(f64(outs[t]) - ref[:, :, t])))
        say("[parity] based decode from zero, step %d: max|err|=%.3e" % (t, err))
        assert err <= 1e-5 * max(1.0, float(np.max(np.abs(ref[:, :, t]))))


def test_based_full_size(orc):
    """The bench workload (2 x 16 heads x 8192 tokens, dk 16, dv 128): two whole
    (b, h) slices against the oracle, the rest finite."""
    cfg = workloads.BASED
    say("[case] based full size B=%d H=%d L=%d dv=%d" % (cfg.B, cfg.H, cfg.L, cfg.dv))
    q, k, v = workloads.based_inputs(cfg, device=DEV)
    o = parallax_based_fwd(q, k, v, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 511, 512, 513, 4095, 4096, 8190, 8191],
                                     rng.integers(0, cfg.L, 40)]))
    for (b, h) in ((0, 0), (1, 15)):
        Q, K, V = f64(q[b, h]), f64(k[b, h]), f64(v[b, h])
        ref = orc.based(Q[None, None], K[None, None], V[None, None], scale=cfg.scale)[0, 0]
        check_rows(f64(o[b, h])[rows], ref[rows], Q, K, V, rows, cfg.scale,
                   "based full size (%d,%d) sampled rows" % (b, h))


@pytest.mark.parametrize("window,n_sink", [(64, 0), (128, 4)])
def test_based_softmax_half(orc, window, n_sink):
    """The other half of the Based hybrid, small-window softmax attention, is
    the Parallax prefill at rho = 0 (the oracle's rho = 0 case is pinned to
    torch's scaled_dot_product_attention): windows of 64 and 128 keys."""
    from gpu_util import compare
    from parallax_local_linear_amd import parallax_attn_fwd
    B, H, L, d = 1, 2, 700, 64
    say("[case] based softmax half W=%d S=%d" % (window, n_sink))
    q, k, v = (workloads.random_tensor((B, H, L, d), 8400 + t) for t in range(3))
    r = torch.zeros_like(q)
    o, lse = parallax_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), r.to(DEV), window=window,
                               n_sink=n_sink)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.fwd(f64(q), f64(k), f64(v), f64(r), window=window, n_sink=n_sink)
    compare(f64(o), f64(lse), o_ref, lse_ref, "softmax half W=%d S=%d" % (window, n_sink))
