"""GPU parity of the Walsh-Hadamard output projection (MI355X only).

y = alpha * (O H_n / sqrt(n)) + beta on the concatenated heads of an fp32
attention output, rounded to bf16, against the fp64 oracle on the same fp32
values.  Bar per element, from the arithmetic: the kernel's fp32 butterflies
(log2 n additions on the path of every output, each adding a relative error
of at most 2^-24 of a partial sum bounded by sum|x|) and the fp32 affine map
stay within e = (log2 n + 2) 2^-24 (|alpha| sum|x| / sqrt(n) + |beta|); the
bf16 rounding adds at most 2^-8 of the value.  The test allows
|y - y_ref| <= 2^-8 |y_ref| + 2 e."""
import numpy as np
import pytest
import torch

from gpu_util import f64, say
from parallax_local_linear_amd import parallax_hadamard_out, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def concat_heads(o):
    """[B, H, L, d] -> [B*L, H*d] rows ordered (b, l) (the page's Y)."""
    B, H, L, d = o.shape
    return np.ascontiguousarray(np.transpose(o, (0, 2, 1, 3)).reshape(B * L, H * d))


def check(orc, y, o, alpha, beta, what):
    Y = concat_heads(f64(o))
    a = None if alpha is None else f64(alpha)
    b = None if beta is None else f64(beta)
    ref = orc.hadamard(Y, a, b)
    n = Y.shape[1]
    got = f64(y).reshape(ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite output"
    e = (np.log2(n) + 2) * 2.0 ** -24 * (
        np.abs(a if a is not None else 1.0) * np.abs(Y).sum(axis=1, keepdims=True) / np.sqrt(n)
        + np.abs(b if b is not None else 0.0))
    bound = 2.0 ** -8 * np.abs(ref) + 2 * e
    err = np.abs(got - ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say("[parity] %s: max|err|=%.3e relL2=%.3e worst err/bound=%.3f" % (what, float(err.max()),
                                                                        rel, worst))
    assert worst <= 1.0, what


@pytest.mark.parametrize("B,H,L,d,affine", [
    (1, 4, 37, 64, True),      # n = 256, 16 tokens per wavefront, ragged
    (2, 4, 50, 128, False),    # n = 512
    (1, 16, 33, 64, True),     # n = 1024
    (2, 16, 77, 128, True),    # n = 2048, 154 tokens: ragged last workgroup
    (1, 32, 19, 128, False),   # n = 4096, one token per wavefront
    (3, 16, 1, 128, True),     # decode: one token per sequence
])
def test_hadamard_shapes(orc, B, H, L, d, affine):
    say("[case] hadamard B=%d H=%d L=%d d=%d affine=%s" % (B, H, L, d, affine))
    n = H * d
    o = workloads.random_tensor((B, H, L, d), 7000 + n + L, dtype=torch.float32).to(DEV)
    alpha = beta = None
    if affine:
        alpha = (1.0 + workloads.random_tensor((n,), 7001, dtype=torch.float32)).to(DEV)
        beta = workloads.random_tensor((n,), 7002, scale=0.1, dtype=torch.float32).to(DEV)
    y = parallax_hadamard_out(o, alpha, beta)
    torch.cuda.synchronize()
    assert y.shape == (B, L, n)
    check(orc, y, o, alpha, beta, "hadamard n=%d d=%d L=%d" % (n, d, L))


def test_hadamard_strided_input_and_output(orc):
    """o as a permuted view of a [B, L, H, d] buffer (the token-major layout),
    output rows wider than n; the padding columns stay untouched."""
    B, H, L, d = 2, 8, 45, 128
    n = H * d
    buf = workloads.random_tensor((B, L, H, d), 7100, dtype=torch.float32).to(DEV)
    o = buf.permute(0, 2, 1, 3)
    big = torch.full((B * L, n + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = big[:, 32:32 + n]
    parallax_hadamard_out(o, out=out)
    torch.cuda.synchronize()
    check(orc, out, o, None, None, "hadamard strided")
    assert torch.isnan(big[:, :32]).all() and torch.isnan(big[:, 32 + n:]).all()


def test_hadamard_full_size(orc):
    """The 1.7B-like layer (2 x 8192 tokens, 16 heads x 128): sampled tokens
    against the oracle, and on every token the two properties that hold at
    any size: the l2 norm is kept (alpha = 1, beta = 0) and applying the
    transform to its own output gives back the input."""
    B, H, L, d = 2, 16, 8192, 128
    n = H * d
    say("[case] hadamard full size B=%d H=%d L=%d d=%d" % (B, H, L, d))
    g = torch.Generator(device=DEV).manual_seed(7200)
    o = torch.randn((B, H, L, d), generator=g, device=DEV)
    y = parallax_hadamard_out(o)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 2, 7, 8, 4095, 8191, 8192, 12000, 2 * L - 1], device=DEV)
    yr = y.view(B * L, n).index_select(0, rows)
    o_rows = o.permute(0, 2, 1, 3).reshape(B * L, n).index_select(0, rows)
    check(orc, yr, o_rows.view(len(rows), 1, n // d, d).permute(0, 2, 1, 3), None, None,
          "hadamard full size rows")
    # norms: |y| = |o| up to the bf16 rounding of y (relative 2^-8 per element)
    n_in = o.permute(0, 2, 1, 3).reshape(B * L, n).double().norm(dim=1)
    n_out = y.view(B * L, n).double().norm(dim=1)
    worst = float(((n_out - n_in).abs() / n_in).max())
    say("[property] full size: max relative change of the row norm %.3e" % worst)
    assert worst <= 2.0 ** -8
    # the transform is its own inverse: H(H(o)) = o up to two bf16 roundings
    back = parallax_hadamard_out(y.float().view(B, L, H, d).permute(0, 2, 1, 3))
    torch.cuda.synchronize()
    err = (back.view(B * L, n).float() - o.permute(0, 2, 1, 3).reshape(B * L, n)).norm(dim=1)
    rel = float((err.double() / n_in).max())
    say("[property] full size: H(H(o)) vs o, max relative row error %.3e" % rel)
    assert rel <= 2 * 2.0 ** -8
