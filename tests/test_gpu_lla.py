"""Exact Local Linear Attention through the Parallax kernel (MI355X only).

Parallax is LLA with a learned probe in place of LLA's per-token solve
(review page "Parallax: Parameterized Local Linear Attention for Language
Modeling", sec. 1-3).  Fed the probe that the solve gives, rho_i =
(Sigma_i + ridge I)^-1 (q_i - kbar_i) (the oracle's conjugate-gradient LLA,
ridge 0.1: rows that see fewer than d + 1 keys have a singular Sigma_i),
the prefill kernel computes LLA's output.  The probe reaches the kernel
rounded to bf16, so the kernel is compared with the oracle on that rounded
probe (the usual 2e-2 / 1e-3 bar), and its distance to exact LLA is
reported.  Inputs are scaled by 0.3 so that the softmax weights are spread
over many keys and the local covariance is well conditioned."""
import numpy as np
import pytest
import torch

from gpu_util import compare, f64, say
from parallax_local_linear_amd import parallax_attn_fwd, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


@pytest.mark.parametrize("d,L,window,n_sink", [(64, 400, 0, 0), (128, 300, 0, 0),
                                               (64, 500, 160, 4)])
def test_parallax_kernel_computes_lla(orc, d, L, window, n_sink):
    say("[case] LLA through the kernel d=%d L=%d W=%d S=%d" % (d, L, window, n_sink))
    q, k, v = (workloads.random_tensor((1, 1, L, d), 900 + d + t, scale=0.3) for t in range(3))
    scale = d ** -0.5
    Q, K, V = f64(q)[0, 0], f64(k)[0, 0], f64(v)[0, 0]
    rows = np.arange(L)
    o_lla, rho, iters = orc.lla_rows(Q, rows, K, V, scale, window, n_sink, ridge=0.1)
    say("[info] CG iterations: min %d median %d max %d" % (iters.min(), np.median(iters),
                                                           iters.max()))
    r = torch.from_numpy(rho).to(torch.bfloat16)[None, None]
    o, lse = parallax_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), r.to(DEV), window=window,
                               n_sink=n_sink)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.fwd(f64(q), f64(k), f64(v), f64(r), window=window, n_sink=n_sink)
    compare(f64(o), f64(lse), o_ref, lse_ref, "kernel with the LLA probe d=%d" % d)
    dist = float(np.max(np.abs(f64(o)[0, 0] - o_lla)))
    rel = float(np.linalg.norm(f64(o)[0, 0] - o_lla) / np.linalg.norm(o_lla))
    say("[report] kernel vs exact LLA (probe rounded to bf16): max|dO|=%.3e relL2=%.3e"
        % (dist, rel))
    assert rel <= 2e-2
