"""CPU tests of the C-ABI boundary: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

No call here reaches a kernel launch: every call either fails validation or
describes an empty problem, both of which return before any HIP call."""
import ctypes
import os
import re

import pytest

from parallax_local_linear_amd import binding
from parallax_local_linear_amd.binding import parallax_strides as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "parallax.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
A16 = 0x10000          # fake, 16-byte aligned device address (never dereferenced)
CONTIG = S(8 * 128 * 64, 128 * 64, 64)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(parallax_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIBRARY):
        pytest.fail("libparallax.so is not built; run `python -m parallax_local_linear_amd.build`")
    return binding.load_library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(binding.LIBRARY)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for code, name in binding.STATUS_NAMES.items():
        assert binding.parallax_status_string(code) == name
    assert binding.parallax_status_string(99) == "PARALLAX_ERR_UNKNOWN"


def fwd(lib, q=A16, k=A16, v=A16, r=A16, o=A16, lse=A16, B=1, H=2, L=64, d=64,
        sq=CONTIG, sk=CONTIG, sv=CONTIG, sr=CONTIG, so=CONTIG, scale=0.125, window=0,
        n_sink=0, ws=A16, ws_bytes=None, entry="parallax_attn_fwd"):
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return getattr(lib, entry)(q, k, v, r, o, lse, B, H, L, d, sq, sk, sv, sr, so, scale,
                               window, n_sink, ws, ws_bytes, None)


def expected_workspace(B, H, L, d):
    """float16 values of every 32-key stage, B*H*ceil(L/32)*32*d*2 bytes, then
    256 bytes of counters."""
    image = B * H * (-(-L // 32)) * 32 * d * 2
    return image + 256 if image else 0


@pytest.mark.parametrize("B,H,L,d", [(1, 1, 1, 64), (2, 3, 32, 128), (2, 16, 8192, 128),
                                     (4, 16, 2048, 64), (1, 2, 33, 64), (3, 1, 100, 128)])
def test_workspace_size(lib, B, H, L, d):
    assert binding.parallax_attn_fwd_workspace_size(B, H, L, d) == expected_workspace(B, H, L, d)


@pytest.mark.parametrize("B,H,L,d", [(0, 1, 64, 64), (1, 0, 64, 64), (1, 1, 0, 128),
                                     (-1, 1, 64, 64), (1, 1, -2, 64), (1, 1, 64, 96)])
def test_workspace_size_of_empty_or_invalid_is_zero(lib, B, H, L, d):
    assert binding.parallax_attn_fwd_workspace_size(B, H, L, d) == 0


@pytest.mark.parametrize("kw", [dict(ws=None), dict(ws=A16 + 8),
                                dict(ws_bytes=expected_workspace(1, 2, 64, 64) - 1),
                                dict(ws_bytes=0)])
def test_fwd_rejects_bad_workspace(lib, kw):
    assert fwd(lib, **kw) == INVALID
    assert fwd(lib, entry="parallax_attn_fwd_precise", **kw) == INVALID


def dec(lib, q=A16, r=A16, k=A16, v=A16, seqlens=None, o=A16, lse=A16, B=2, H=2, Lmax=64,
        d=128, sk=CONTIG, sv=CONTIG, scale=0.1, splits=16):
    return lib.parallax_attn_decode(q, r, k, v, seqlens, o, lse, B, H, Lmax, d, sk, sv, scale,
                                    splits, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED),
    (dict(d=256), UNSUPPORTED),
    (dict(B=-1), INVALID),
    (dict(H=-2), INVALID),
    (dict(L=-5), INVALID),
    (dict(q=None), INVALID),
    (dict(k=None), INVALID),
    (dict(v=None), INVALID),
    (dict(r=None), INVALID),
    (dict(o=None), INVALID),
    (dict(lse=None), INVALID),
    (dict(q=A16 + 8), INVALID),
    (dict(v=A16 + 2), INVALID),
    (dict(o=A16 + 4), INVALID),
    (dict(lse=A16 + 2), INVALID),
    (dict(window=-1), INVALID),
    (dict(n_sink=-3), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=-0.5), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(sq=S(8 * 128 * 64, 128 * 64, 60)), INVALID),
    (dict(sk=S(8 * 128 * 64, 4, 64)), INVALID),
    (dict(sv=S(-64, 128 * 64, 64)), INVALID),
    (dict(so=S(8 * 128 * 64, 128 * 64, 66)), INVALID),
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert fwd(lib, entry="parallax_attn_fwd_precise", **kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(L=0),
                                dict(B=0, q=None, k=None, v=None, r=None, o=None, lse=None),
                                dict(L=0, ws=None, ws_bytes=0)])
def test_fwd_empty_problem_is_a_no_op(lib, kw):
    assert fwd(lib, **kw) == OK
    assert fwd(lib, entry="parallax_attn_fwd_precise", **kw) == OK


def test_fwd_empty_still_checks_d(lib):
    assert fwd(lib, L=0, d=80) == UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED),
    (dict(splits=3), UNSUPPORTED),
    (dict(splits=32), UNSUPPORTED),
    (dict(splits=0), UNSUPPORTED),
    (dict(B=-1), INVALID),
    (dict(Lmax=-1), INVALID),
    (dict(q=None), INVALID),
    (dict(r=None), INVALID),
    (dict(k=None), INVALID),
    (dict(o=None), INVALID),
    (dict(lse=None), INVALID),
    (dict(q=A16 + 4), INVALID),
    (dict(k=A16 + 8), INVALID),
    (dict(seqlens=A16 + 2), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(sk=S(8, 8, 4)), INVALID),
    (dict(sk=S(1 << 30, 1 << 26, 1 << 24)), UNSUPPORTED),
    (dict(sv=S(1 << 30, 1 << 26, 1 << 24)), UNSUPPORTED),
])
def test_decode_rejects(lib, kw, status):
    assert dec(lib, **kw) == status


def test_decode_empty_batch_is_a_no_op(lib):
    assert dec(lib, B=0, q=None, r=None, k=None, v=None, o=None, lse=None) == OK


def fwd_train(lib, sbar=A16, pv=A16, **kw):
    args = dict(q=A16, k=A16, v=A16, r=A16, o=A16, lse=A16, B=1, H=2, L=64, d=64,
                sq=CONTIG, sk=CONTIG, sv=CONTIG, sr=CONTIG, so=CONTIG, scale=0.125, window=0,
                n_sink=0, ws=A16, ws_bytes=1 << 40)
    args.update(kw)
    a = args
    return lib.parallax_attn_fwd_train(a["q"], a["k"], a["v"], a["r"], a["o"], a["lse"], sbar, pv,
                                       a["B"], a["H"], a["L"], a["d"], a["sq"], a["sk"], a["sv"],
                                       a["sr"], a["so"], a["scale"], a["window"], a["n_sink"],
                                       a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(sbar=None), INVALID), (dict(pv=None), INVALID), (dict(pv=A16 + 4), INVALID),
    (dict(sbar=A16 + 2), INVALID), (dict(d=96), UNSUPPORTED), (dict(q=None), INVALID),
])
def test_fwd_train_rejects(lib, kw, status):
    assert fwd_train(lib, **kw) == status


def test_fwd_train_empty_is_a_no_op(lib):
    assert fwd_train(lib, L=0, sbar=None, pv=None) == OK


def expected_bwd_workspace(B, H, L, d):
    """Per 32-row stage: 512 bytes of row statistics + five bf16 blocks of 32*d."""
    return B * H * (-(-L // 32)) * (512 + 5 * 32 * d * 2)


@pytest.mark.parametrize("B,H,L,d", [(1, 1, 1, 64), (2, 3, 32, 128), (2, 16, 8192, 128),
                                     (1, 2, 33, 64)])
def test_bwd_workspace_size(lib, B, H, L, d):
    assert binding.parallax_attn_bwd_workspace_size(B, H, L, d) == expected_bwd_workspace(B, H, L, d)


@pytest.mark.parametrize("B,H,L,d", [(0, 1, 64, 64), (1, 1, 0, 128), (1, 1, -2, 64),
                                     (1, 1, 64, 96)])
def test_bwd_workspace_size_of_empty_or_invalid_is_zero(lib, B, H, L, d):
    assert binding.parallax_attn_bwd_workspace_size(B, H, L, d) == 0


def bwd(lib, **kw):
    names = ["q", "k", "v", "r", "dout", "o", "lse", "sbar", "pv", "dq", "dk", "dv", "dr"]
    a = {n: A16 for n in names}
    a.update(B=1, H=2, L=64, d=64, sq=CONTIG, sk=CONTIG, sv=CONTIG, sr=CONTIG, sdo=CONTIG,
             scale=0.125, window=0, n_sink=0, ws=A16 * 16, ws_bytes=1 << 40)
    a.update(kw)
    return lib.parallax_attn_bwd(*[a[n] for n in names], a["B"], a["H"], a["L"], a["d"],
                                 a["sq"], a["sk"], a["sv"], a["sr"], a["sdo"], a["scale"],
                                 a["window"], a["n_sink"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(B=-1), INVALID), (dict(L=-1), INVALID),
    (dict(dout=None), INVALID), (dict(o=None), INVALID), (dict(sbar=None), INVALID),
    (dict(pv=None), INVALID), (dict(dq=None), INVALID), (dict(dk=None), INVALID),
    (dict(dv=None), INVALID), (dict(dr=None), INVALID), (dict(dout=A16 + 8), INVALID),
    (dict(dq=A16 + 4), INVALID), (dict(pv=A16 + 4), INVALID), (dict(window=-1), INVALID),
    (dict(n_sink=-1), INVALID), (dict(scale=0.0), INVALID),
    (dict(sdo=S(8 * 128 * 64, 128 * 64, 60)), INVALID),
    (dict(ws=None), INVALID), (dict(ws=A16 * 16 + 16), INVALID),
    (dict(ws_bytes=expected_bwd_workspace(1, 2, 64, 64) - 1), INVALID),
])
def test_bwd_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_bwd_empty_is_a_no_op(lib):
    assert bwd(lib, H=0, q=None, dq=None, ws=None, ws_bytes=0) == OK


def decp(lib, q=A16, r=A16, k=A16, v=A16, bt=A16, num_pages=64, page=16, max_pages=8,
         seqlens=None, o=A16, lse=A16, B=2, Hq=4, Hkv=2, d=128, sk=CONTIG, sv=CONTIG,
         scale=0.1, window=0, n_sink=0, splits=16):
    return lib.parallax_attn_decode_paged(q, r, k, v, bt, num_pages, page, max_pages, seqlens, o,
                                          lse, B, Hq, Hkv, d, sk, sv, scale, window, n_sink,
                                          splits, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(splits=3), UNSUPPORTED), (dict(B=-1), INVALID),
    (dict(Hkv=3), INVALID), (dict(Hkv=0), INVALID), (dict(page=24), INVALID),
    (dict(page=0), INVALID), (dict(num_pages=0), INVALID), (dict(max_pages=0), INVALID),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(o=None), INVALID),
    (dict(q=A16 + 4), INVALID), (dict(bt=A16 + 2), INVALID), (dict(window=-1), INVALID),
    (dict(n_sink=-1), INVALID), (dict(scale=0.0), INVALID), (dict(sk=S(8, 8, 4)), INVALID),
])
def test_decode_paged_rejects(lib, kw, status):
    assert decp(lib, **kw) == status


def test_decode_paged_empty_is_a_no_op(lib):
    assert decp(lib, B=0, q=None, r=None, k=None, v=None, o=None, lse=None) == OK
    # a contiguous cache (no block table) needs no power-of-two page size
    assert decp(lib, Hq=0, bt=None, page=300) == OK


def decp_ws(lib, ws=A16, ws_bytes=None, B=2, Hq=4, d=128, **kw):
    """parallax_attn_decode_paged_ws with decp's defaults and a workspace."""
    if ws_bytes is None:
        ws_bytes = lib.parallax_attn_decode_paged_workspace_size(B, Hq, d)
    args = dict(q=A16, r=A16, k=A16, v=A16, bt=A16, num_pages=64, page=16, max_pages=8,
                seqlens=None, o=A16, lse=A16, Hkv=2, sk=CONTIG, sv=CONTIG, scale=0.1, window=0,
                n_sink=0, splits=16)
    args.update(kw)
    a = args
    return lib.parallax_attn_decode_paged_ws(a["q"], a["r"], a["k"], a["v"], a["bt"],
                                             a["num_pages"], a["page"], a["max_pages"],
                                             a["seqlens"], a["o"], a["lse"], B, Hq, a["Hkv"], d,
                                             a["sk"], a["sv"], a["scale"], a["window"],
                                             a["n_sink"], a["splits"], ws, ws_bytes, None)


def test_decode_paged_workspace_size(lib):
    """[B*Hq][8 splits][m, ell, S, A[d], C[d]] fp32; 0 for an empty or unsupported problem."""
    assert lib.parallax_attn_decode_paged_workspace_size(64, 16, 128) == 64 * 16 * 8 * 259 * 4
    assert lib.parallax_attn_decode_paged_workspace_size(3, 5, 64) == 3 * 5 * 8 * 131 * 4
    assert lib.parallax_attn_decode_paged_workspace_size(0, 16, 128) == 0
    assert lib.parallax_attn_decode_paged_workspace_size(4, 0, 128) == 0
    assert lib.parallax_attn_decode_paged_workspace_size(4, 16, 96) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), INVALID), (dict(ws=A16 + 8), INVALID),
    (dict(ws_bytes=2 * 4 * 8 * 259 * 4 - 1), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(splits=3), UNSUPPORTED), (dict(Hkv=3), INVALID),
    (dict(q=None), INVALID), (dict(page=24), INVALID), (dict(scale=0.0), INVALID),
])
def test_decode_paged_ws_rejects(lib, kw, status):
    assert decp_ws(lib, **kw) == status


def test_decode_paged_ws_empty_is_a_no_op(lib):
    assert decp_ws(lib, B=0, ws=None, ws_bytes=0, q=None, r=None, k=None, v=None, o=None,
                   lse=None) == OK


def proj(lib, x=A16, w=A16, y=A16, M=64, N=64, K=64, ldx=64, ldw=64, ldy=64):
    return lib.parallax_qkvr_project(x, w, y, M, N, K, ldx, ldw, ldy, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID), (dict(K=-32), INVALID), (dict(K=48), UNSUPPORTED),
    (dict(N=60), UNSUPPORTED), (dict(x=None), INVALID), (dict(y=A16 + 8), INVALID),
    (dict(ldx=32), INVALID), (dict(ldy=60), INVALID), (dict(ldw=66), INVALID),
    (dict(K=0, ldx=8, ldw=8), UNSUPPORTED),
])
def test_projection_rejects(lib, kw, status):
    assert proj(lib, **kw) == status


def test_projection_empty_is_a_no_op(lib):
    assert proj(lib, M=0, x=None, y=None) == OK


def had(lib, o=A16, so=S(16 * 8 * 128, 8 * 128, 128), B=2, H=16, L=8, d=128, alpha=None,
        beta=None, y=A16, ldy=2048):
    return lib.parallax_hadamard_out(o, so, B, H, L, d, alpha, beta, y, ldy, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(L=-3), INVALID), (dict(H=-1), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(H=3, ldy=384), UNSUPPORTED),
    (dict(H=1, ldy=128), UNSUPPORTED), (dict(H=64, ldy=8192), UNSUPPORTED),
    (dict(o=None), INVALID), (dict(y=None), INVALID), (dict(o=A16 + 4), INVALID),
    (dict(y=A16 + 2), INVALID), (dict(alpha=A16 + 4), INVALID), (dict(beta=A16 + 8), INVALID),
    (dict(ldy=2044), INVALID), (dict(ldy=2050), INVALID),
    (dict(so=S(16 * 8 * 128, 8 * 128, 130)), INVALID), (dict(so=S(-4, 1024, 128)), INVALID),
])
def test_hadamard_rejects(lib, kw, status):
    assert had(lib, **kw) == status


def test_hadamard_empty_is_a_no_op(lib):
    assert had(lib, B=0, o=None, y=None) == OK
    assert had(lib, L=0, o=None, y=None) == OK


QK16 = S(2 * 300 * 16, 300 * 16, 16)
V128 = S(2 * 300 * 128, 300 * 128, 128)


def based(lib, q=A16, k=A16, v=A16, o=A16, state=None, B=1, H=2, L=300, dk=16, dv=128,
          sq=QK16, sk=QK16, sv=V128, so=V128, scale=0.25, ws=A16, ws_bytes=1 << 40):
    return lib.parallax_based_fwd(q, k, v, o, state, B, H, L, dk, dv, sq, sk, sv, so, scale, ws,
                                  ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(L=-1), INVALID), (dict(dk=32), UNSUPPORTED),
    (dict(dv=96), UNSUPPORTED), (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(ws=None), INVALID), (dict(q=A16 + 8), INVALID), (dict(o=A16 + 4), INVALID),
    (dict(state=A16 + 4), INVALID), (dict(ws=A16 + 8), INVALID), (dict(ws_bytes=0), INVALID),
    (dict(sk=S(2 * 300 * 16, 300 * 16, 12)), INVALID), (dict(so=S(-4, 128, 128)), INVALID),
])
def test_based_rejects(lib, kw, status):
    assert based(lib, **kw) == status


def test_based_empty_is_a_no_op(lib):
    assert based(lib, L=0, q=None, k=None, v=None, o=None, ws=None) == OK


def test_based_sizes(lib):
    nc = 16 * (128 // 16 + 1)
    assert binding.parallax_based_state_floats(16, 128) == 160 * nc
    assert binding.parallax_based_state_floats(16, 64) == 160 * 80
    assert binding.parallax_based_state_floats(8, 128) == 0
    # B * H * ceil(L / 512) * 160 * NC * 6 bytes
    assert binding.parallax_based_workspace_size(2, 16, 8192, 16, 128) == 2 * 16 * 16 * 160 * nc * 6
    assert binding.parallax_based_workspace_size(1, 1, 513, 16, 64) == 2 * 160 * 80 * 6
    assert binding.parallax_based_workspace_size(1, 1, 64, 16, 96) == 0


def test_based_decode_rejects(lib):
    dec_b = lambda **kw: lib.parallax_based_decode(
        kw.get("q", A16), kw.get("k", A16), kw.get("v", A16), kw.get("state", A16),
        kw.get("o", A16), kw.get("B", 2), kw.get("H", 2), kw.get("dk", 16), kw.get("dv", 128),
        kw.get("scale", 0.25), None)
    assert dec_b(dk=8) == UNSUPPORTED
    assert dec_b(dv=32) == UNSUPPORTED
    assert dec_b(B=-1) == INVALID
    assert dec_b(state=None) == INVALID
    assert dec_b(scale=-1.0) == INVALID
    assert dec_b(state=A16 + 2) == INVALID
    assert dec_b(B=0, q=None, state=None) == OK


def test_split_qkvr_views_share_storage():
    import torch
    y = torch.arange(2 * 5 * 4 * 3 * 8, dtype=torch.float32).view(2 * 5, 4 * 3 * 8)
    q, k, v, r = binding.split_qkvr(y, B=2, L=5, H=3, d=8)
    assert q.shape == (2, 3, 5, 8) and q.data_ptr() == y.data_ptr()
    # token (b, l) = row b*L + l; head h of part p = columns p*H*d + h*d .. +d
    assert torch.equal(r[1, 2, 4], y[1 * 5 + 4, 3 * 24 + 2 * 8: 3 * 24 + 3 * 8])
    assert torch.equal(k[0, 1, 3], y[3, 24 + 8: 24 + 16])


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.parallax_attn_fwd(x, x, x, x)
    with pytest.raises(TypeError):
        binding.parallax_attn_fwd(x.float(), x, x, x)


def test_missing_library_fails_loudly(tmp_path):
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError):
            binding.load_library(str(tmp_path / "nope.so"))
    finally:
        binding._lib = saved


def fwd_noalloc(lib, q=A16, k=A16, v=A16, r=A16, o=A16, lse=A16, B=1, H=2, L=64, d=64,
                sq=CONTIG, sk=CONTIG, sv=CONTIG, sr=CONTIG, so=CONTIG, scale=0.125, window=0,
                n_sink=0):
    return lib.parallax_attn_fwd_noalloc(q, k, v, r, o, lse, B, H, L, d, sq, sk, sv, sr, so,
                                         scale, window, n_sink, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(B=-1), INVALID), (dict(q=None), INVALID),
    (dict(o=A16 + 4), INVALID), (dict(window=-1), INVALID), (dict(scale=0.0), INVALID),
    (dict(sk=S(8 * 128 * 64, 4, 64)), INVALID),
    # workspace need above the library's 64 MiB array: 2 x 16 x 8224 tokens at d = 128
    (dict(B=2, H=16, L=8224, d=128), UNSUPPORTED),
    (dict(B=1, H=1, L=(1 << 19) + 32, d=64), UNSUPPORTED),
])
def test_fwd_noalloc_rejects(lib, kw, status):
    """Checked on the host before the library's device array is looked up."""
    assert fwd_noalloc(lib, **kw) == status


def test_fwd_noalloc_empty_problem_is_a_no_op(lib):
    assert fwd_noalloc(lib, B=0, q=None, k=None, v=None, r=None, o=None, lse=None) == OK
    assert fwd_noalloc(lib, L=0) == OK


def test_fwd_noalloc_limit_is_the_headline_size():
    """The 2 x 16 x 8192 x 128 workload's workspace fills the 64 MiB + 256 array."""
    assert expected_workspace(2, 16, 8192, 128) == (64 << 20) + 256


def fwd_f32(lib, q=A16, k=A16, v=A16, r=A16, o=A16, lse=A16, B=1, H=2, L=64, d=64,
            sq=CONTIG, sk=CONTIG, sv=CONTIG, sr=CONTIG, so=CONTIG, scale=0.125, window=0,
            n_sink=0):
    return lib.parallax_attn_fwd_f32(q, k, v, r, o, lse, B, H, L, d, sq, sk, sv, sr, so, scale,
                                     window, n_sink, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(L=-1), INVALID), (dict(r=None), INVALID),
    (dict(lse=None), INVALID), (dict(o=A16 + 2), INVALID), (dict(n_sink=-1), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(sv=S(-64, 64, 64)), INVALID),
])
def test_fwd_f32_rejects(lib, kw, status):
    assert fwd_f32(lib, **kw) == status


def test_fwd_f32_empty_problem_is_a_no_op(lib):
    assert fwd_f32(lib, H=0, q=None, k=None, v=None, r=None, o=None, lse=None) == OK
