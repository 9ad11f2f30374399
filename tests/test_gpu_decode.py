"""GPU parity of the split-KV decode kernel against the fp64 oracle (MI355X only)."""
import pytest
import torch

from gpu_util import compare, default_scale, f64, say
from parallax_local_linear_amd import parallax_attn_decode, parallax_attn_fwd, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SPLITS = (1, 2, 4, 8, 16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def rand(shape, seed, scale=1.0):
    return workloads.random_tensor(shape, seed, device="cpu", scale=scale)


@pytest.mark.parametrize("d", (64, 128))
@pytest.mark.parametrize("splits", SPLITS)
def test_decode_small(orc, d, splits):
    B, H, Lmax = 5, 2, 300
    seqlens = [300, 1, 0, 17, 299]
    q, r = (rand((B, H, d), 10 * d + t) for t in range(2))
    k, v = (rand((B, H, Lmax, d), 20 * d + t) for t in range(2))
    say("[case] decode d=%d splits=%d seqlens=%s" % (d, splits, seqlens))
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    o, lse = parallax_attn_decode(q.to(DEV), r.to(DEV), k.to(DEV), v.to(DEV), sl,
                                  num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode(f64(q), f64(r), f64(k), f64(v), seqlens=seqlens)
    compare(f64(o), f64(lse), o_ref, lse_ref, "decode d=%d splits=%d" % (d, splits))
    assert torch.all(o[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_decode_without_seqlens_and_clamping(orc):
    B, H, Lmax, d = 3, 4, 513, 128
    q, r = (rand((B, H, d), 40 + t) for t in range(2))
    k, v = (rand((B, H, Lmax, d), 50 + t) for t in range(2))
    o, lse = parallax_attn_decode(q.to(DEV), r.to(DEV), k.to(DEV), v.to(DEV))
    o_ref, lse_ref = orc.decode(f64(q), f64(r), f64(k), f64(v))
    compare(f64(o), f64(lse), o_ref, lse_ref, "decode seqlens=None")
    # out-of-range lengths are clamped to [0, Lmax]
    sl = torch.tensor([10 ** 6, -7, 5], dtype=torch.int32, device=DEV)
    o, lse = parallax_attn_decode(q.to(DEV), r.to(DEV), k.to(DEV), v.to(DEV), sl)
    o_ref, lse_ref = orc.decode(f64(q), f64(r), f64(k), f64(v), seqlens=[Lmax, 0, 5])
    compare(f64(o), f64(lse), o_ref, lse_ref, "decode clamped seqlens")


def test_decode_matches_last_prefill_row():
    """A decode step at length n equals row n-1 of the prefill over the same keys."""
    B, H, n, d = 2, 3, 700, 128
    q, k, v, r = (rand((B, H, n, d), 60 + t).to(DEV) for t in range(4))
    o_p, lse_p = parallax_attn_fwd(q, k, v, r)
    o_d, lse_d = parallax_attn_decode(q[:, :, -1].contiguous(), r[:, :, -1].contiguous(), k, v)
    err = float((o_p[:, :, -1] - o_d).abs().max())
    say("[invariant] decode vs last prefill row: max|dO|=%.3e" % err)
    assert err <= 2e-2
    assert float((lse_p[:, :, -1] - lse_d).abs().max()) <= 1e-3


def test_split_invariance():
    cfg = workloads.Decode("split", 7, 8, 4, 2048, 128)
    q, k, v, r = workloads.decode_inputs(cfg, device=DEV)
    outs = [parallax_attn_decode(q, r, k, v, num_splits=s) for s in SPLITS]
    for s, (o, lse) in zip(SPLITS[1:], outs[1:]):
        e_o = float((o - outs[0][0]).abs().max())
        e_l = float((lse - outs[0][1]).abs().max())
        say("[invariant] splits %d vs 1: max|dO|=%.3e max|dLSE|=%.3e" % (s, e_o, e_l))
        assert e_o <= 1e-4 and e_l <= 1e-5


def test_decode_deterministic():
    cfg = workloads.Decode("det", 8, 4, 4, 1024, 128)
    q, k, v, r = workloads.decode_inputs(cfg, device=DEV)
    a = parallax_attn_decode(q, r, k, v)
    b = parallax_attn_decode(q, r, k, v)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_full_size_all_heads(orc):
    """The benchmark decode workload (64 x 16 heads, 4096 cached tokens) in
    the launch the benchmark times: every one of the 1024 heads against the
    oracle (compared eight sequences at a time to bound host memory)."""
    cfg = workloads.DECODE
    say("[case] full size %s" % cfg.name)
    q, k, v, r = workloads.decode_inputs(cfg, device=DEV)
    o, lse = parallax_attn_decode(q, r, k, v, num_splits=cfg.num_splits)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    scale = default_scale(cfg.d)
    for b0 in range(0, cfg.B, 8):
        sl = slice(b0, b0 + 8)
        o_ref, lse_ref = orc.decode(f64(q[sl]), f64(r[sl]), f64(k[sl]), f64(v[sl]), scale=scale)
        compare(f64(o[sl]), f64(lse[sl]), o_ref, lse_ref,
                "decode full b=%d..%d (all %d heads)" % (b0, b0 + 7, cfg.H))
