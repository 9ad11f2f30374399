"""GPU parity of the prefill kernel against the fp64 oracle (MI355X only).

Every case compares the HIP path element by element with the oracle run on
the same bf16 inputs: whole outputs at sizes the oracle finishes in seconds
(several tiles plus ragged tails), sampled rows at the full workload sizes
in the same launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

from gpu_util import compare, default_scale, f64, oracle_rows, say
from parallax_local_linear_amd import (parallax_attn_fwd, parallax_attn_fwd_workspace_size,
                                       workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def rand(shape, seed, scale=1.0):
    return workloads.random_tensor(shape, seed, device="cpu", scale=scale)


def nan_outputs(q):
    """Output buffers pre-filled with NaN, so a row the kernel never writes shows up."""
    B, H, L, d = q.shape
    return (torch.full((B, H, L, d), float("nan"), device=DEV),
            torch.full((B, H, L), float("nan"), device=DEV))


def full_check(orc, q, k, v, r, window=0, n_sink=0, scale=None, what=""):
    d = q.shape[-1]
    scale = default_scale(d) if scale is None else scale
    say("[case] %s shape=%s window=%d n_sink=%d" % (what, tuple(q.shape), window, n_sink))
    qd, kd, vd, rd = (x.to(DEV) for x in (q, k, v, r))
    o0, l0 = nan_outputs(qd)
    o, lse = parallax_attn_fwd(qd, kd, vd, rd, softmax_scale=scale, window=window, n_sink=n_sink,
                               out=o0, lse=l0)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.fwd(f64(q), f64(k), f64(v), f64(r), scale=scale, window=window,
                             n_sink=n_sink)
    return compare(f64(o), f64(lse), o_ref, lse_ref, what), o, lse


def test_tiny_workload(orc):
    """B=1 H=2 L=256 d=64, fp32 draws rounded to bf16; plus the unrounded error (reported)."""
    cfg = workloads.TINY
    q32, k32, v32, r32 = workloads.prefill_inputs(cfg, dtype=torch.float32)
    q, k, v, r = (x.to(torch.bfloat16) for x in (q32, k32, v32, r32))
    _, o, _ = full_check(orc, q, k, v, r, what="tiny")
    o_fp32_ref, _ = orc.fwd(f64(q32), f64(k32), f64(v32), f64(r32))
    say("[report] tiny vs oracle on the unrounded fp32 inputs: max|dO|=%.3e"
        % float(np.max(np.abs(f64(o) - o_fp32_ref))))


def test_tiny_probe_zero_is_softmax(orc):
    """rho = 0: the kernel must reduce to softmax attention (oracle pinned to SDPA)."""
    cfg = workloads.TINY
    q, k, v, _ = workloads.prefill_inputs(cfg)
    full_check(orc, q, k, v, torch.zeros_like(q), what="tiny rho=0")


SMALL = [
    # (B, H, L, d, window, n_sink)
    (1, 2, 1000, 64, 0, 0),
    (1, 2, 1000, 128, 0, 0),
    (2, 1, 129, 64, 0, 0),
    (1, 1, 1, 64, 0, 0),
    (1, 1, 1, 128, 0, 0),
    (1, 1, 63, 128, 0, 0),
    (1, 1, 65, 64, 0, 0),
    (3, 1, 200, 128, 0, 0),
    (1, 2, 300, 64, 1, 0),
    (1, 2, 300, 128, 128, 4),
    (1, 1, 700, 64, 37, 70),
    (1, 1, 700, 128, 200, 130),
    (1, 1, 500, 64, 600, 0),
    (1, 1, 500, 64, 0, 5),
    (1, 1, 257, 128, 64, 4),
    (1, 1, 1000, 64, 1, 64),
    (1, 2, 1500, 64, 128, 4),
]


# Causal tiles end with a few steps after the main loop (their remaining
# full stages and the diagonal), taken as whole groups of six plus a partial
# group.  These lengths give tiles with each possible count, from the stage
# schedule (128-row tiles, fully visible stages first): with 32-key stages
# (d = 128) 2 to 9 steps (2: L=257, 3: 289, 4: 129, 5: 161, 6: 193, 7: 225,
# 8: 449, 9: 481); with 64-key stages (d = 64) 2 to 7 steps (2: L=129,
# 3: 193, 4: 257, 5: 321, 6: 385, 7: 449).
TAIL_LENGTHS = {128: [129, 161, 193, 225, 257, 289, 449, 481],
                64: [129, 193, 257, 321, 385, 449]}


@pytest.mark.parametrize("d", [64, 128])
def test_causal_tail_step_counts(orc, d):
    for i, L in enumerate(TAIL_LENGTHS[d]):
        q, k, v, r = (rand((1, 1, L, d), 60 + 4 * i + j) for j in range(4))
        full_check(orc, q, k, v, r, what="causal tail L=%d d=%d" % (L, d))


@pytest.mark.parametrize("B,H,L,d,window,n_sink", SMALL)
def test_small_shapes(orc, B, H, L, d, window, n_sink):
    seed = B * 1000003 + H * 10007 + L * 101 + d + window * 7 + n_sink
    q, k, v, r = (rand((B, H, L, d), seed + t) for t in range(4))
    full_check(orc, q, k, v, r, window=window, n_sink=n_sink,
               what="small B%d H%d L%d d%d" % (B, H, L, d))


def test_window_one_returns_values(orc):
    """Window 1 and no sinks: each row sees only itself, so o = v (up to f16 rounding of v)."""
    q, k, v, r = (rand((1, 2, 333, 128), 900 + t) for t in range(4))
    o, lse = parallax_attn_fwd(*(x.to(DEV) for x in (q, k, v, r)), window=1)
    np.testing.assert_allclose(f64(o), f64(v), atol=1e-6, rtol=2 ** -10)


def test_scaled_inputs_and_custom_scale(orc):
    q, k, v, r = (rand((1, 2, 400, 64), 950 + t, scale=0.5) for t in range(4))
    full_check(orc, q, k, v, r, scale=0.3, what="custom scale 0.3")


@pytest.mark.parametrize("d", [64, 128])
def test_scores_rising_late(orc, d):
    """Keys whose scores grow along the sequence (about 25 log2 units from the
    first to the last key): each row's softmax offset, fixed from its first
    stage plus a margin of 3, is overtaken by more than 5 for most rows, so
    the workgroups recompute with the exact row max.  The data is checked to
    have that property before the kernel is compared with the oracle."""
    L = 512
    g = torch.Generator().manual_seed(4321 + d)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    ramp = 46.0 * (d / 64) ** 0.5 * torch.arange(L, dtype=torch.float32) / L
    q = (3.0 * u + 0.1 * torch.randn(1, 1, L, d, generator=g)).to(torch.bfloat16)
    k = (ramp[:, None] * u + 0.1 * torch.randn(1, 1, L, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(1, 1, L, d, generator=g).to(torch.bfloat16)
    # Probe scores |rho . k| stay below about 60 here: the O error of the f16
    # value path grows with them, and this case is about the offsets.
    r = (0.25 * torch.randn(1, 1, L, d, generator=g)).to(torch.bfloat16)
    scale = default_scale(d)
    x = (f64(q)[0, 0] @ f64(k)[0, 0].T) * scale * np.log2(np.e)
    rows = np.arange(32, L)
    first = x[rows, :32].max(axis=1)
    last = np.array([x[i, :i + 1].max() for i in rows])
    assert (last > first + 3 + 5).mean() > 0.5, "the data must overtake the first-stage offsets"
    full_check(orc, q, k, v, r, what="scores rising late d=%d" % d)


@pytest.mark.parametrize("cfg", [workloads.PREFILL_06B, workloads.PREFILL_17B, workloads.LOCAL],
                         ids=lambda c: c.name)
def test_full_size_whole_slices(orc, cfg):
    """The benchmark workloads at full size, in the launch the benchmark
    times: every output is finite (a skipped tile would leave NaN rows), and
    every row of five (b, h) slices -- the first, the last and three seeded
    others -- equals the oracle."""
    say("[case] full size %s" % cfg.name)
    q, k, v, r = workloads.prefill_inputs(cfg, device=DEV)
    scale = default_scale(cfg.d)
    o0, l0 = nan_outputs(q)
    o, lse = parallax_attn_fwd(q, k, v, r, softmax_scale=scale, window=cfg.window,
                               n_sink=cfg.n_sink, out=o0, lse=l0)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(cfg.seed)
    BH = cfg.B * cfg.H
    picks = {0, BH - 1}
    while len(picks) < min(5, BH):
        picks.add(int(rng.integers(0, BH)))
    rows = list(range(cfg.L))
    for x in sorted(picks):
        b, h = x // cfg.H, x % cfg.H
        o_ref, lse_ref = oracle_rows(orc, q, k, v, r, b, h, rows, scale, cfg.window, cfg.n_sink)
        compare(f64(o[b, h]), f64(lse[b, h]), o_ref, lse_ref,
                "%s b=%d h=%d (all %d rows)" % (cfg.name, b, h, cfg.L))


def test_constant_values_give_constant_output():
    """Weights 1 + rho.(k - kbar) sum to one under p, so v = 1 everywhere gives o = 1."""
    q, k, r = (rand((2, 2, 777, 128), 1000 + t) for t in range(3))
    v = torch.ones_like(q)
    o, _ = parallax_attn_fwd(*(x.to(DEV) for x in (q, k, v, r)), window=100, n_sink=3)
    err = float((o - 1).abs().max())
    say("[invariant] constant values: max|o-1|=%.3e" % err)
    assert err <= 2e-2


def test_deterministic():
    q, k, v, r = (rand((2, 4, 1100, 128), 1100 + t).to(DEV) for t in range(4))
    o1, l1 = parallax_attn_fwd(q, k, v, r)
    o2, l2 = parallax_attn_fwd(q, k, v, r)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_strided_layouts_match_contiguous():
    """[B, L, H, d] storage (viewed as [B, H, L, d]) and a strided output give identical bits."""
    B, H, L, d = 2, 3, 517, 64
    base = [rand((B, L, H, d), 1200 + t).to(DEV) for t in range(4)]
    views = [x.permute(0, 2, 1, 3) for x in base]
    conts = [x.contiguous() for x in views]
    o1, l1 = parallax_attn_fwd(*conts, window=64, n_sink=2)
    big = torch.full((B, H, L, 2 * d), float("nan"), device=DEV)
    out = big[..., :d]
    o2, l2 = parallax_attn_fwd(*views, window=64, n_sink=2, out=out)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isnan(big[..., d:]).all()


def test_64bit_offsets(orc):
    """More than 2^31 elements per tensor (windowed so it stays fast): rows at the far end."""
    B, H, L, d = 1, 2, (1 << 23) + 1000, 128
    window, n_sink = 128, 4
    say("[case] 64-bit offsets B=%d H=%d L=%d d=%d" % (B, H, L, d))
    q, k, v, r = (workloads.random_tensor((B, H, L, d), 1300 + t, device=DEV) for t in range(4))
    o, lse = parallax_attn_fwd(q, k, v, r, window=window, n_sink=n_sink)
    torch.cuda.synchronize()
    scale = default_scale(d)
    for i in (L - 1, L - 200, L // 2, 5):
        # The visible set of row i is the sinks plus the last `window` keys; give the
        # oracle exactly that context, re-indexed so that it keeps the same visible set.
        lo = max(n_sink, i - window + 1)
        keys = list(range(min(n_sink, i + 1))) + list(range(lo, i + 1))
        keys = sorted(set(keys))
        idx = torch.as_tensor(keys, device=DEV)
        K = f64(k[0, 1].index_select(0, idx))
        V = f64(v[0, 1].index_select(0, idx))
        pos = len(keys) - 1
        o_ref, lse_ref = orc.rows(f64(q[0, 1, i:i + 1]), f64(r[0, 1, i:i + 1]), [pos], K, V,
                                  scale, 0, 0)
        compare(f64(o[0, 1, i:i + 1]), f64(lse[0, 1, i:i + 1]), o_ref, lse_ref,
                "64-bit offsets row %d" % i)


def test_key_slice_past_31_bit_offsets(orc):
    """K rows spaced 2^14 elements apart over 65616 rows (a slice of more than
    2^31 bytes): the general kernel then builds buffer resources per stage
    instead of one per tensor.  At d = 64 a stage is two 32-key V^T images,
    the second of which does not exist for the last stage when the sequence
    ends in its first half (65616 = 1025 * 64 + 16).  Rows across the
    sequence against the oracle with their full causal context."""
    B, H, L, d, ld = 1, 1, 65616, 64, 1 << 14
    say("[case] 31-bit key slice B=%d H=%d L=%d d=%d row stride %d" % (B, H, L, d, ld))
    q, v, r = (workloads.random_tensor((B, H, L, d), 1400 + t, device=DEV) for t in range(3))
    kbuf = torch.zeros((L, ld), dtype=torch.bfloat16, device=DEV)
    kbuf[:, :d] = workloads.random_tensor((L, d), 1403, device=DEV)
    k = kbuf[:, :d].unsqueeze(0).unsqueeze(0)
    assert k.stride() == (L * ld, L * ld, ld, 1)
    o, lse = parallax_attn_fwd(q, k, v, r)
    torch.cuda.synchronize()
    scale = default_scale(d)
    K, V = f64(k[0, 0]), f64(v[0, 0])
    for i in (0, 31, 32, 63, 64, 127, 40000, L - 81, L - 17, L - 16, L - 1):
        o_ref, lse_ref = orc.rows(f64(q[0, 0, i:i + 1]), f64(r[0, 0, i:i + 1]), [i],
                                  K[:i + 1], V[:i + 1], scale, 0, 0)
        compare(f64(o[0, 0, i:i + 1]), f64(lse[0, 0, i:i + 1]), o_ref, lse_ref,
                "31-bit key slice row %d" % i)
    del kbuf


def test_many_slices(orc):
    """B*H above 65535 (the prepass's grid then loops over slices): short
    sequences, every output finite, and whole slices on both sides of that
    bound against the oracle."""
    B, H, L, d = 2, 33000, 40, 64
    say("[case] many slices B=%d H=%d L=%d d=%d" % (B, H, L, d))
    q, k, v, r = (workloads.random_tensor((B, H, L, d), 1400 + t, device=DEV) for t in range(4))
    o0, l0 = nan_outputs(q)
    o, lse = parallax_attn_fwd(q, k, v, r, out=o0, lse=l0)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    scale = default_scale(d)
    for b, h in ((0, 0), (0, 32999), (1, 32534), (1, 32535), (1, 32999)):
        rows = list(range(L))
        o_ref, lse_ref = oracle_rows(orc, q, k, v, r, b, h, rows, scale)
        compare(f64(o[b, h]), f64(lse[b, h]), o_ref, lse_ref, "many slices b=%d h=%d" % (b, h))


def test_side_stream_with_internal_workspace():
    """A prefill on a side stream whose workspace the binding allocates and
    frees, followed at once by an allocation and fill on the current stream:
    the freed workspace must not be handed to that fill while the prefill
    still reads it, so the result equals a current-stream run bit for bit."""
    B, H, L, d = 2, 16, 4096, 128
    q, k, v, r = (workloads.random_tensor((B, H, L, d), 1500 + t, device=DEV) for t in range(4))
    o_ref, l_ref = parallax_attn_fwd(q, k, v, r)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    o, lse = parallax_attn_fwd(q, k, v, r, stream=side)
    junk = torch.empty(parallax_attn_fwd_workspace_size(B, H, L, d), dtype=torch.uint8,
                       device=DEV)
    junk.fill_(0x55)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


# Windows of at most 128 keys with at most 32 sinks take the windowed kernel:
# 64-row tiles streamed in runs through a ring of key stages.  The first two
# cases have more tiles than the chip has workgroup slots, so workgroups run
# several consecutive tiles (2 at d = 64, 3 at d = 128).
WINDOW_CASES = [
    # (B, H, L, d, window, n_sink)
    (1, 8, 5000, 64, 128, 4),
    (1, 8, 5000, 128, 128, 4),
    (2, 3, 777, 64, 1, 0),
    (1, 2, 1000, 64, 16, 31),
    (1, 2, 1000, 128, 33, 32),
    (1, 2, 1000, 64, 100, 1),
    (1, 2, 1000, 128, 127, 0),
    (1, 1, 65, 64, 64, 4),
    (1, 1, 31, 128, 128, 4),
    (3, 2, 300, 64, 128, 32),
    (1, 2, 1000, 64, 128, 1),
    (1, 2, 700, 128, 128, 32),
    # 16 sinks: the largest count whose sink stage takes half the work; 17
    # takes the general stage loop
    (1, 4, 2000, 64, 128, 16),
    (1, 4, 2000, 64, 128, 17),
    # runs of 5 tiles (the staggered start and the row streams over several
    # tiles) ending in a ragged tile
    (1, 16, 8200, 64, 128, 4),
]


@pytest.mark.parametrize("B,H,L,d,window,n_sink", WINDOW_CASES)
def test_window_kernel_shapes(orc, B, H, L, d, window, n_sink):
    seed = 31 * L + 7 * d + window + 1000 * n_sink + B + 10 * H
    q, k, v, r = (rand((B, H, L, d), seed + t) for t in range(4))
    full_check(orc, q, k, v, r, window=window, n_sink=n_sink,
               what="window kernel B%d H%d L%d d%d" % (B, H, L, d))


@pytest.mark.parametrize("d", [64, 128])
def test_window_kernel_rising_scores(orc, d):
    """Keys whose scores rise along the sequence make most wavefronts of the
    windowed kernel recompute their rows with exact offsets, after the first
    pass took the window's common-case schedule."""
    q, k, v, r = workloads.rising_inputs(1, 2, 1000, d, seed=91 + d)
    full_check(orc, q, k, v, r, window=128, n_sink=4, what="window kernel rising d%d" % d)


@pytest.mark.parametrize("rising", [False, True], ids=["normal", "rising"])
def test_recompute_counter(orc, rising):
    """The workspace's counter (4 bytes after the V image) holds the number of
    128-row query tiles that took the exact second pass: most tiles for keys
    whose scores rise along the sequence, about none for N(0,1) inputs; the
    outputs match the oracle either way."""
    B, H, L, d = 1, 2, 1024, 128
    if rising:
        q, k, v, r = workloads.rising_inputs(B, H, L, d, seed=77)
    else:
        q, k, v, r = (rand((B, H, L, d), 7700 + t) for t in range(4))
    n_tiles = B * H * (L // 128)
    image = B * H * (L // 32) * 32 * d * 2
    ws = torch.full((parallax_attn_fwd_workspace_size(B, H, L, d),), 0xAB, dtype=torch.uint8,
                    device=DEV)
    o, lse = parallax_attn_fwd(*(x.to(DEV) for x in (q, k, v, r)), workspace=ws)
    torch.cuda.synchronize()
    count = int(ws[image:image + 4].view(torch.int32).item())
    say("[counter] %s: %d of %d tiles recomputed" % ("rising" if rising else "normal", count,
                                                      n_tiles))
    if rising:
        assert n_tiles // 2 <= count <= n_tiles
    else:
        assert 0 <= count <= 1
    o_ref, lse_ref = orc.fwd(f64(q), f64(k), f64(v), f64(r))
    compare(f64(o), f64(lse), o_ref, lse_ref, "recompute counter %s" % rising)
