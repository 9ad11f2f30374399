"""GPU parity of the general decode (paged cache, grouped kv heads, window and
sinks) against the fp64 oracle (MI355X only).

The oracle computes each row on the logical contiguous cache
[B, Hkv, Lmax, d]; the GPU reads the same values scattered over a page pool
through a shuffled block table.  Tolerances as for the plain decode: O max
abs error <= 2e-2, LSE <= 1e-3 (the decode runs in fp32; with Hq / Hkv >= 4
the weights and values reach the matrix cores as float16, as in the
prefill)."""
import numpy as np
import pytest
import torch

from gpu_util import compare, f64, say
from parallax_local_linear_amd import (parallax_attn_decode, parallax_attn_decode_paged,
                                       parallax_attn_decode_paged_workspace_size, workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def rand(shape, seed, scale=1.0):
    return workloads.random_tensor(shape, seed, device="cpu", scale=scale)


def to_pages(cache, page_size, seed, spare=3):
    """[B, Hkv, Lmax, d] -> (pool [P, page_size, Hkv, d], block_table [B, max_pages]) with
    the pages of all sequences shuffled over the pool (plus a few unused pages)."""
    B, Hkv, Lmax, d = cache.shape
    max_pages = -(-Lmax // page_size)
    n_pages = B * max_pages + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * max_pages]
    pool = torch.zeros((n_pages, page_size, Hkv, d), dtype=cache.dtype)
    padded = torch.zeros((B, Hkv, max_pages * page_size, d), dtype=cache.dtype)
    padded[:, :, :Lmax] = cache
    pages = padded.view(B, Hkv, max_pages, page_size, d).permute(0, 2, 3, 1, 4)
    pool[torch.as_tensor(perm)] = pages.reshape(B * max_pages, page_size, Hkv, d)
    table = torch.as_tensor(perm.reshape(B, max_pages), dtype=torch.int32)
    return pool, table


def run_case(orc, B, Hq, Hkv, Lmax, d, seqlens, window, n_sink, page_size, splits, seed,
             workspace=None):
    say("[case] paged decode B=%d Hq=%d Hkv=%d Lmax=%d d=%d page=%s W=%d S=%d splits=%d"
        % (B, Hq, Hkv, Lmax, d, page_size, window, n_sink, splits))
    q, r = (rand((B, Hq, d), seed + t) for t in range(2))
    k, v = (rand((B, Hkv, Lmax, d), seed + 10 + t) for t in range(2))
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV) if seqlens is not None else None
    if page_size is None:
        kc = k.to(DEV).permute(0, 2, 1, 3)
        vc = v.to(DEV).permute(0, 2, 1, 3)
        table = None
    else:
        kp, table = to_pages(k, page_size, seed)
        vp, _ = to_pages(v, page_size, seed)
        kc, vc, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    o, lse = parallax_attn_decode_paged(q.to(DEV), r.to(DEV), kc, vc, table, sl, window=window,
                                        n_sink=n_sink, num_splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.decode_ext(f64(q), f64(r), f64(k), f64(v), seqlens=seqlens,
                                    window=window, n_sink=n_sink)
    compare(f64(o), f64(lse), o_ref, lse_ref,
            "paged decode Hq=%d Hkv=%d d=%d page=%s W=%d S=%d" % (Hq, Hkv, d, page_size,
                                                                  window, n_sink))
    return o, lse


CASES = [
    # (B, Hq, Hkv, Lmax, d, seqlens, window, n_sink, page_size, splits)
    (5, 4, 4, 300, 128, [300, 1, 0, 17, 299], 0, 0, 16, 16),
    (5, 4, 1, 300, 64, [300, 1, 0, 17, 299], 0, 0, 64, 8),
    (3, 8, 2, 513, 128, [513, 200, 64], 0, 0, 256, 4),
    (3, 8, 2, 513, 128, [513, 200, 64], 128, 4, 32, 16),
    (4, 6, 3, 700, 64, [700, 130, 71, 5], 37, 70, 16, 16),
    (4, 6, 3, 700, 128, [700, 130, 71, 5], 1, 3, 64, 2),
    (2, 4, 2, 257, 128, [257, 256], 600, 0, 128, 1),
    (3, 8, 8, 400, 128, [400, 399, 1], 64, 0, None, 16),
    (3, 8, 2, 400, 64, None, 100, 2, None, 4),
    # matrix-core path (Hq / Hkv >= 4): 16 heads per kv head (MQA), a group
    # of 6 (columns 6..7 of its tile unused), and 20 heads (16 + 4 columns
    # in two workgroups per kv head)
    (2, 16, 1, 300, 128, [300, 77], 0, 0, 32, 16),
    (2, 12, 2, 300, 64, [300, 5], 50, 3, 16, 4),
    (1, 20, 1, 700, 128, None, 0, 0, None, 8),
]


@pytest.mark.parametrize("B,Hq,Hkv,Lmax,d,seqlens,window,n_sink,page_size,splits", CASES)
def test_paged_decode(orc, B, Hq, Hkv, Lmax, d, seqlens, window, n_sink, page_size, splits):
    seed = B * 7919 + Hq * 104729 + Lmax + d + window * 13 + n_sink + (page_size or 0)
    run_case(orc, B, Hq, Hkv, Lmax, d, seqlens, window, n_sink, page_size, splits, seed)


GROUPED = [c for c in CASES if c[1] // c[2] >= 4]


@pytest.mark.parametrize("B,Hq,Hkv,Lmax,d,seqlens,window,n_sink,page_size,splits", GROUPED)
def test_grouped_without_key_splits(orc, B, Hq, Hkv, Lmax, d, seqlens, window, n_sink,
                                    page_size, splits):
    """The grouped cases through parallax_attn_decode_paged (no workspace, so
    one workgroup per kv head and column group); the cases above take the
    workspace entry, which splits these small calls' keys over 8 workgroups."""
    seed = B * 7919 + Hq * 104729 + Lmax + d + window * 13 + n_sink + (page_size or 0) + 1
    run_case(orc, B, Hq, Hkv, Lmax, d, seqlens, window, n_sink, page_size, splits, seed,
             workspace=False)


def test_workspace_reused_by_a_smaller_call(orc):
    """One caller workspace, two calls in a row (the second smaller, over
    stale partial states of the first): both match the oracle."""
    ws = torch.empty(parallax_attn_decode_paged_workspace_size(3, 16, 128), dtype=torch.uint8,
                     device=DEV)
    run_case(orc, 3, 16, 1, 900, 128, [900, 450, 2], 0, 0, 64, 16, 4242, workspace=ws)
    run_case(orc, 2, 8, 2, 333, 128, [1, 333], 0, 0, None, 16, 4343, workspace=ws)


def test_plain_case_matches_contiguous_decode(orc):
    """Hkv = Hq, no window, contiguous: the same values as parallax_attn_decode."""
    B, H, Lmax, d = 4, 4, 777, 128
    q, r = (rand((B, H, d), 300 + t).to(DEV) for t in range(2))
    k, v = (rand((B, H, Lmax, d), 310 + t).to(DEV) for t in range(2))
    sl = torch.tensor([777, 500, 3, 0], dtype=torch.int32, device=DEV)
    o1, l1 = parallax_attn_decode(q, r, k, v, sl)
    o2, l2 = parallax_attn_decode_paged(q, r, k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3),
                                        None, sl)
    torch.cuda.synchronize()
    err = float((o1 - o2).abs().max())
    say("[parity] paged vs contiguous decode kernel: max|dO|=%.3e" % err)
    assert err <= 1e-5
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2))
    assert float((l1[fin] - l2[fin]).abs().max()) <= 1e-5


def test_bad_block_table_entries_are_clamped(orc):
    """Out-of-range page indices read a page of the pool instead of faulting."""
    B, Hq, Hkv, Lmax, d, page = 2, 2, 1, 64, 64, 16
    q, r = (rand((B, Hq, d), 400 + t).to(DEV) for t in range(2))
    pool_k, pool_v = (rand((8, page, Hkv, d), 410 + t).to(DEV) for t in range(2))
    table = torch.tensor([[0, 1, 2, 3], [10 ** 6, -5, 7, 6]], dtype=torch.int32, device=DEV)
    o, lse = parallax_attn_decode_paged(q, r, pool_k, pool_v, table)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("Hkv", [16, 4, 1])
def test_full_size_paged_gqa(orc, Hkv):
    """The decode workload's size (B=64, 16 query heads, 4096 tokens, d=128) in
    64-token pages, with 16, 4 or 1 kv heads (with 1, 64 kv heads serve 16
    query heads each, in four workgroups of 4 per kv head); sampled (b, h)
    rows against the oracle."""
    cfg = workloads.DECODE
    B, Hq, Lmax, d, page = cfg.B, cfg.H, cfg.Lmax, cfg.d, 64
    say("[case] full-size paged decode Hkv=%d" % Hkv)
    g = torch.Generator(device=DEV).manual_seed(777 + Hkv)
    q = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    r = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    n_pages = B * Lmax // page
    kp = torch.randn((n_pages, page, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vp = torch.randn((n_pages, page, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(Hkv))
    table = perm.view(B, Lmax // page).to(torch.int32).to(DEV)
    seqlens = torch.full((B,), Lmax, dtype=torch.int32)
    seqlens[1::3] = torch.randint(1, Lmax, (len(seqlens[1::3]),),
                                  generator=torch.Generator().manual_seed(5))
    o, lse = parallax_attn_decode_paged(q, r, kp, vp, table, seqlens.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for b in (0, 1, 31, 63):
        n = int(seqlens[b])
        pages = table[b].cpu()[: -(-n // page)]
        kb = kp.index_select(0, pages.to(DEV)).reshape(-1, Hkv, d)[:n].permute(1, 0, 2)
        vb = vp.index_select(0, pages.to(DEV)).reshape(-1, Hkv, d)[:n].permute(1, 0, 2)
        o_ref, lse_ref = orc.decode_ext(f64(q[b:b + 1]), f64(r[b:b + 1]), f64(kb)[None],
                                        f64(vb)[None])
        compare(f64(o[b:b + 1]), f64(lse[b:b + 1]), o_ref, lse_ref,
                "full-size paged decode Hkv=%d b=%d n=%d" % (Hkv, b, n))


@pytest.mark.parametrize("bad", ["dtype", "shape", "strided"])
def test_paged_rejects_bad_outputs(bad):
    """A caller-supplied out / lse is checked before the launch: the kernel
    writes B*Hq*d and B*Hq fp32 values through their pointers."""
    B, Hq, Hkv, L, d = 2, 4, 2, 64, 128
    q, r = (rand((B, Hq, d), 7 + t).to(DEV) for t in range(2))
    k, v = (rand((B, L, Hkv, d), 9 + t).to(DEV) for t in range(2))
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    if bad == "dtype":
        out = out.to(torch.bfloat16)
    elif bad == "shape":
        lse = torch.empty((B, Hq - 1), dtype=torch.float32, device=DEV)
    else:
        out = torch.empty((B, Hq, 2 * d), dtype=torch.float32, device=DEV)[..., :d]
    with pytest.raises((TypeError, ValueError)):
        parallax_attn_decode_paged(q, r, k, v, out=out, lse=lse)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (16, 1)])
def test_workspace_entry_through_the_c_abi(Hq, Hkv):
    """parallax_attn_decode_paged_ws called directly: with fewer than four
    query heads per kv head it leaves the workspace alone and gives the plain
    entry's bits; with sixteen it splits the keys, within the decode's
    tolerance of the plain entry."""
    from parallax_local_linear_amd import binding
    lib = binding.load_library()
    B, L, d, page = 3, 640, 128, 64
    say("[case] C-ABI workspace decode Hq=%d Hkv=%d" % (Hq, Hkv))
    q, r = (rand((B, Hq, d), 900 + t).to(DEV) for t in range(2))
    n_pages = B * L // page
    kp, vp = (rand((n_pages, page, Hkv, d), 910 + t).to(DEV) for t in range(2))
    table = torch.arange(n_pages, dtype=torch.int32).flip(0).view(B, L // page).contiguous().to(DEV)
    sl = torch.tensor([640, 333, 1], dtype=torch.int32, device=DEV)
    ks = binding.parallax_strides(kp.stride(0), kp.stride(2), kp.stride(1))
    vs = binding.parallax_strides(vp.stride(0), vp.stride(2), vp.stride(1))
    nbytes = lib.parallax_attn_decode_paged_workspace_size(B, Hq, d)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV)  # NaN-like fill
    outs = []
    for use_ws in (False, True):
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
        args = (q.data_ptr(), r.data_ptr(), kp.data_ptr(), vp.data_ptr(), table.data_ptr(),
                n_pages, page, L // page, sl.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                Hkv, d, ks, vs, 1.0 / d ** 0.5, 0, 0, 16)
        if use_ws:
            st = lib.parallax_attn_decode_paged_ws(*args, ws.data_ptr(), nbytes, None)
        else:
            st = lib.parallax_attn_decode_paged(*args, None)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o1, l1), (o2, l2) = outs
    assert torch.isfinite(o2).all() and torch.isfinite(l2).all()
    if Hq // Hkv < 4:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert bool((ws == 0x7f).all()), "the workspace was touched"
    else:
        err = float((o1 - o2).abs().max())
        say("[parity] key splits vs one workgroup: max|dO|=%.3e" % err)
        assert err <= 2e-2
        assert float((l1 - l2).abs().max()) <= 1e-3
