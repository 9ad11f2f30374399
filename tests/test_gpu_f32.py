"""GPU parity of the fp32 prefill (parallax_attn_fwd_f32) against the fp64
oracle on the same fp32 values, unrounded (MI355X only).

The tiny reference workload is specified in fp32; the matrix-core prefill
takes bf16 inputs, whose rounding alone moves o by about 0.07 there.  This
path keeps the fp32 values.  Bar: max |dO| <= 1e-3 and max |dLSE| <= 1e-4.
Derivation: the scores are fp32 dot products of d terms (relative error
about d * 2^-24, at most 8e-6 at d = 128), exponentials and sums are fp32;
a relative error e of the weights moves o by about e * R * |v| with R the
spread of the probe scores (below about 70 for N(0,1) inputs at d = 128),
so about 6e-4 at worst, and the LSE by about e * |scale q.k| (below 1e-4)."""
import numpy as np
import pytest
import torch

from gpu_util import f64, say
from parallax_local_linear_amd import parallax_attn_fwd_f32, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL, LSE_TOL = 1e-3, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def check(orc, q, k, v, r, what, window=0, n_sink=0, scale=None):
    o, lse = parallax_attn_fwd_f32(q.to(DEV), k.to(DEV), v.to(DEV), r.to(DEV), window=window,
                                   n_sink=n_sink, softmax_scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.fwd(f64(q), f64(k), f64(v), f64(r), scale=scale, window=window,
                             n_sink=n_sink)
    eo = float(np.max(np.abs(f64(o) - o_ref)))
    el = float(np.max(np.abs(f64(lse) - lse_ref)))
    say("[parity] %s: max|dO|=%.3e max|dLSE|=%.3e" % (what, eo, el))
    assert np.isfinite(f64(o)).all() and np.isfinite(f64(lse)).all(), what
    assert eo <= O_TOL and el <= LSE_TOL, what
    return o, lse


def draws(B, H, L, d, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return tuple(scale * torch.randn((B, H, L, d), generator=g, dtype=torch.float32)
                 for _ in range(4))


def test_tiny_workload_fp32(orc):
    """B=1 H=2 L=256 d=64, the fp32 draws themselves."""
    say("[case] fp32 tiny workload")
    q, k, v, r = workloads.prefill_inputs(workloads.TINY, dtype=torch.float32)
    check(orc, q, k, v, r, "fp32 tiny")


def test_tiny_probe_zero_is_softmax_fp32(orc):
    say("[case] fp32 tiny, rho = 0")
    q, k, v, _ = workloads.prefill_inputs(workloads.TINY, dtype=torch.float32)
    check(orc, q, k, v, torch.zeros_like(q), "fp32 tiny rho=0")


@pytest.mark.parametrize("B,H,L,d,window,n_sink", [
    (1, 2, 300, 128, 0, 0), (2, 1, 200, 64, 37, 3), (1, 1, 1, 128, 0, 0),
    (1, 2, 190, 64, 64, 0), (1, 1, 129, 128, 1, 5)])
def test_shapes_fp32(orc, B, H, L, d, window, n_sink):
    say("[case] fp32 B=%d H=%d L=%d d=%d W=%d S=%d" % (B, H, L, d, window, n_sink))
    q, k, v, r = draws(B, H, L, d, 100 + L + d + window)
    check(orc, q, k, v, r, "fp32 L=%d d=%d W=%d S=%d" % (L, d, window, n_sink), window=window,
          n_sink=n_sink)


def test_strided_inputs_fp32(orc):
    """Views with row and head strides larger than their widths."""
    say("[case] fp32 strided views")
    B, H, L, d = 1, 2, 150, 64
    g = torch.Generator().manual_seed(7)
    big = torch.randn((B, L, H, 4 * d + 16), generator=g, dtype=torch.float32).to(DEV)
    q, k, v, r = (big[..., i * d:(i + 1) * d].permute(0, 2, 1, 3) for i in range(4))
    o, lse = parallax_attn_fwd_f32(q, k, v, r)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.fwd(f64(q), f64(k), f64(v), f64(r))
    eo = float(np.max(np.abs(f64(o) - o_ref)))
    say("[parity] fp32 strided: max|dO|=%.3e" % eo)
    assert eo <= O_TOL
    assert float(np.max(np.abs(f64(lse) - lse_ref))) <= LSE_TOL
