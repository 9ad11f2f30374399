"""GPU parity of the fused input projections [Q | K | V | R] = X W^T (MI355X only).

Compared with the fp64 oracle on the same bf16 operands.  The kernel sums in
fp32 and rounds the result to bf16 (relative rounding <= 2^-9), so the bar
per element is |y - y_ref| <= 2^-8 |y_ref| + 1e-4 sum_t |x_it w_nt| (the
second term covers fp32 accumulation over K terms)."""
import numpy as np
import pytest
import torch

from gpu_util import f64, say
from parallax_local_linear_amd import (parallax_attn_fwd, parallax_qkvr_project, split_qkvr,
                                       workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def check(orc, y, x, w, what):
    ref = orc.project(f64(x), f64(w))
    mag = orc.project(np.abs(f64(x)), np.abs(f64(w)))
    got = f64(y)
    assert np.isfinite(got).all(), what + ": non-finite output"
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * mag
    worst = float(np.max(err / bound)) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say("[parity] %s: max|err|=%.3e relL2=%.3e worst err/bound=%.3f" % (what, float(err.max()),
                                                                        rel, worst))
    assert worst <= 1.0, what


@pytest.mark.parametrize("M,N,K", [(300, 520, 96), (1, 8, 32), (513, 1024, 256),
                                   (256, 256, 2048), (77, 4 * 16 * 64, 1024)])
def test_projection_shapes(orc, M, N, K):
    say("[case] projection M=%d N=%d K=%d" % (M, N, K))
    x = workloads.random_tensor((M, K), 1000 + M + K)
    w = workloads.random_tensor((N, K), 2000 + N + K, scale=K ** -0.5)
    y = parallax_qkvr_project(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    check(orc, y, x, w, "projection M=%d N=%d K=%d" % (M, N, K))


def test_projection_strided(orc):
    """Row strides larger than the row widths, for x, w and the output."""
    M, N, K = 200, 264, 128
    xb = workloads.random_tensor((M, K + 64), 3001).to(DEV)
    wb = workloads.random_tensor((N, K + 32), 3002, scale=K ** -0.5).to(DEV)
    yb = torch.full((M, N + 40), float("nan"), dtype=torch.bfloat16, device=DEV)
    x, w, y = xb[:, 16:16 + K], wb[:, 8:8 + K], yb[:, 8:8 + N]
    parallax_qkvr_project(x, w, out=y)
    torch.cuda.synchronize()
    check(orc, y, x, w, "projection strided")
    assert torch.isnan(yb[:, :8]).all() and torch.isnan(yb[:, 8 + N:]).all()


@pytest.mark.parametrize("K", [32, 96])
def test_projection_odd_k_ignores_row_padding(orc, K):
    """K % 64 == 32: the last 64-k stage reads 32 k past K of every row (row
    padding here, NaN) and must not use it."""
    M, N = 300, 264
    say("[case] projection odd K=%d with NaN row padding" % K)
    xb = torch.full((M, K + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    wb = torch.full((N, K + 32), float("nan"), dtype=torch.bfloat16, device=DEV)
    x, w = xb[:, :K], wb[:, :K]
    x.copy_(workloads.random_tensor((M, K), 3101 + K).to(DEV))
    w.copy_(workloads.random_tensor((N, K), 3102 + K, scale=K ** -0.5).to(DEV))
    y = parallax_qkvr_project(x, w)
    torch.cuda.synchronize()
    check(orc, y, x, w, "projection odd K=%d" % K)


def test_projection_full_size_sampled(orc):
    """The 1.7B-like layer: 2 x 8192 tokens, width 2048, 4 x 16 heads x 128;
    sampled token rows against the oracle."""
    cfg = workloads.PREFILL_17B
    M, K, N = cfg.B * cfg.L, cfg.H * cfg.d, 4 * cfg.H * cfg.d
    say("[case] projection full size M=%d N=%d K=%d" % (M, N, K))
    g = torch.Generator(device=DEV).manual_seed(4242)
    x = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device=DEV) * K ** -0.5).to(torch.bfloat16)
    y = parallax_qkvr_project(x, w)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    rows = torch.tensor([0, 1, 255, 256, 4095, 8191, 8192, 12345, M - 257, M - 1], device=DEV)
    check(orc, y.index_select(0, rows), x.index_select(0, rows), w, "projection full size rows")


def test_attention_reads_projection_views():
    """Prefill on the strided views of the projection output equals the prefill
    on contiguous copies of the same values, bit for bit."""
    B, L, H, d, K = 2, 300, 3, 64, 192
    x = workloads.random_tensor((B * L, K), 5001).to(DEV)
    w = workloads.random_tensor((4 * H * d, K), 5002, scale=K ** -0.5).to(DEV)
    y = parallax_qkvr_project(x, w)
    views = split_qkvr(y, B, L, H, d)
    o1, l1 = parallax_attn_fwd(*views, window=100, n_sink=2)
    o2, l2 = parallax_attn_fwd(*(t.contiguous() for t in views), window=100, n_sink=2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
