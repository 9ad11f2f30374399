"""One attention layer through the library, end to end (MI355X only):

    [q | k | v | rho] = x [W_Q; W_K; W_V; W_R]^T     (parallax_qkvr_project)
    o = Parallax attention over the strided views     (parallax_attn_fwd)
    y = alpha * (O H_n / sqrt(n)) + beta              (parallax_hadamard_out)

against the same chain of oracle functions in fp64.  The oracle rounds its
projection to bf16 as the library stores it (round to nearest even), so
both sides feed the attention the same values except where the fp32 and
fp64 sums round differently (one bf16 ulp).

Bars: the attention's output O within its own 2e-2 of the oracle's; and,
since the output projection is linear, the GPU's y within bf16 rounding of
the oracle's y moved by the propagated attention error e = alpha (dO H /
sqrt n) (dO = O_gpu - O_oracle, transformed by the oracle):
|y - y_ref| <= 2^-8 (|y_ref| + |e|) + |e| + (the fp32 error of the
transform's butterflies) per element; relative l2 error of y at most
1e-2."""
import numpy as np
import pytest
import torch

from gpu_util import f64, say
from parallax_local_linear_amd import (parallax_attn_fwd, parallax_hadamard_out,
                                       parallax_qkvr_project, split_qkvr, workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def bf16_round(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("B,L,H,d,window,n_sink", [(2, 300, 4, 64, 0, 0), (1, 520, 8, 128, 128, 4)])
def test_layer_end_to_end(orc, B, L, H, d, window, n_sink):
    say("[case] layer B=%d L=%d H=%d d=%d W=%d S=%d" % (B, L, H, d, window, n_sink))
    n = H * d
    x = workloads.random_tensor((B * L, n), 9100 + d)
    w = workloads.random_tensor((4 * n, n), 9101 + d, scale=n ** -0.5)
    alpha = (1.0 + 0.1 * workloads.random_tensor((n,), 9102, dtype=torch.float32))
    beta = 0.1 * workloads.random_tensor((n,), 9103, dtype=torch.float32)
    # library
    yproj = parallax_qkvr_project(x.to(DEV), w.to(DEV))
    q, k, v, r = split_qkvr(yproj, B, L, H, d)
    o, _ = parallax_attn_fwd(q, k, v, r, window=window, n_sink=n_sink)
    y = parallax_hadamard_out(o, alpha.to(DEV), beta.to(DEV))
    torch.cuda.synchronize()
    # oracle chain
    P = bf16_round(orc.project(f64(x), f64(w)))              # [B*L, 4n]
    parts = [P[:, j * n:(j + 1) * n].reshape(B, L, H, d).transpose(0, 2, 1, 3) for j in range(4)]
    o_ref, _ = orc.fwd(*parts, window=window, n_sink=n_sink)  # [B, H, L, d]
    Y = o_ref.transpose(0, 2, 1, 3).reshape(B * L, n)
    y_ref = orc.hadamard(Y, f64(alpha), f64(beta))
    got = f64(y).reshape(B * L, n)
    d_o = f64(o) - o_ref
    e_o = float(np.abs(d_o).max())
    assert e_o <= 2e-2, "attention stage: max|dO| %.3e" % e_o
    e = f64(alpha) * orc.hadamard(d_o.transpose(0, 2, 1, 3).reshape(B * L, n))
    # plus the fp32 butterflies' own error: (log2 n + 2) 2^-24 |alpha| sum|O| / sqrt n
    rows = np.abs(f64(o)).transpose(0, 2, 1, 3).reshape(B * L, n).sum(axis=1, keepdims=True)
    fp32 = 2 * (np.log2(n) + 2) * 2.0 ** -24 * np.abs(f64(alpha)) * rows / np.sqrt(n)
    bound = 2.0 ** -8 * (np.abs(y_ref) + np.abs(e)) + np.abs(e) + fp32
    err = np.abs(got - y_ref)
    worst = float(np.max(err / bound))
    rel = float(np.linalg.norm(got - y_ref) / np.linalg.norm(y_ref))
    say("[parity] layer: attention max|dO|=%.3e; y max|err|=%.3e relL2=%.3e worst err/bound=%.3f"
        % (e_o, float(err.max()), rel, worst))
    assert np.isfinite(got).all()
    assert rel <= 1e-2 and worst <= 1.0
