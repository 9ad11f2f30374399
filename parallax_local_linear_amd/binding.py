"""Thin ctypes binding over ``libparallax.so`` (the C ABI in include/parallax.h).

Argument marshalling only: tensors are checked for dtype, device and layout,
their data pointers and element strides are passed through, outputs are
allocated with torch when the caller gives none, and every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

torch is imported first on purpose: the library then binds to the HIP
runtime torch already loaded, so torch's streams and device pointers are
valid in it.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import math
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libparallax.so")

PARALLAX_OK = 0
STATUS_NAMES = {0: "PARALLAX_OK", 1: "PARALLAX_ERR_INVALID_ARG",
                2: "PARALLAX_ERR_UNSUPPORTED", 3: "PARALLAX_ERR_LAUNCH"}

# Every symbol include/parallax.h declares.
EXPORTED = ("parallax_attn_fwd_workspace_size", "parallax_attn_fwd", "parallax_attn_fwd_precise",
            "parallax_attn_fwd_noalloc", "parallax_attn_fwd_f32",
            "parallax_attn_fwd_train",
            "parallax_attn_bwd_workspace_size", "parallax_attn_bwd", "parallax_attn_decode",
            "parallax_attn_decode_paged", "parallax_attn_decode_paged_workspace_size",
            "parallax_attn_decode_paged_ws", "parallax_qkvr_project", "parallax_hadamard_out",
            "parallax_based_state_floats", "parallax_based_workspace_size", "parallax_based_fwd",
            "parallax_based_decode", "parallax_status_string")


class parallax_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("l", ctypes.c_int64)]


class ParallaxError(RuntimeError):
    def __init__(self, status: int, name: str):
        super().__init__("%s (status %d)" % (name, status))
        self.status = status
        self.name = name


_lib = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the built library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libparallax.so is not built (%s); run `python -m parallax_local_linear_amd.build`"
            % path)
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    S = parallax_strides
    lib.parallax_attn_fwd_workspace_size.restype = ctypes.c_size_t
    lib.parallax_attn_fwd_workspace_size.argtypes = [i, i, i, i]
    lib.parallax_attn_fwd.restype = ctypes.c_int
    lib.parallax_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, S, S, S, S, S,
                                      f, i, i, vp, ctypes.c_size_t, vp]
    lib.parallax_attn_fwd_precise.restype = ctypes.c_int
    lib.parallax_attn_fwd_precise.argtypes = lib.parallax_attn_fwd.argtypes
    lib.parallax_attn_fwd_f32.restype = ctypes.c_int
    lib.parallax_attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, S, S, S, S, S,
                                          f, i, i, vp]
    lib.parallax_attn_fwd_noalloc.restype = ctypes.c_int
    lib.parallax_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, S, S, S, S, S,
                                              f, i, i, vp]
    lib.parallax_attn_fwd_train.restype = ctypes.c_int
    lib.parallax_attn_fwd_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i,
                                            S, S, S, S, S, f, i, i, vp, ctypes.c_size_t, vp]
    lib.parallax_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.parallax_attn_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.parallax_attn_bwd.restype = ctypes.c_int
    lib.parallax_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      i, i, i, i, S, S, S, S, S, f, i, i, vp,
                                      ctypes.c_size_t, vp]
    lib.parallax_attn_decode.restype = ctypes.c_int
    lib.parallax_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, S, S,
                                         f, i, vp]
    lib.parallax_attn_decode_paged.restype = ctypes.c_int
    lib.parallax_attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, vp, vp,
                                               i, i, i, i, S, S, f, i, i, i, vp]
    lib.parallax_attn_decode_paged_workspace_size.restype = ctypes.c_size_t
    lib.parallax_attn_decode_paged_workspace_size.argtypes = [i, i, i]
    lib.parallax_attn_decode_paged_ws.restype = ctypes.c_int
    lib.parallax_attn_decode_paged_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, vp, vp,
                                                  i, i, i, i, S, S, f, i, i, i, vp,
                                                  ctypes.c_size_t, vp]
    lib.parallax_qkvr_project.restype = ctypes.c_int
    lib.parallax_qkvr_project.argtypes = [vp, vp, vp, i, i, i, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, vp]
    lib.parallax_hadamard_out.restype = ctypes.c_int
    lib.parallax_hadamard_out.argtypes = [vp, S, i, i, i, i, vp, vp, vp, ctypes.c_int64, vp]
    lib.parallax_based_state_floats.restype = ctypes.c_size_t
    lib.parallax_based_state_floats.argtypes = [i, i]
    lib.parallax_based_workspace_size.restype = ctypes.c_size_t
    lib.parallax_based_workspace_size.argtypes = [i, i, i, i, i]
    lib.parallax_based_fwd.restype = ctypes.c_int
    lib.parallax_based_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, S, S, S, S, f, vp,
                                       ctypes.c_size_t, vp]
    lib.parallax_based_decode.restype = ctypes.c_int
    lib.parallax_based_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp]
    lib.parallax_status_string.restype = ctypes.c_char_p
    lib.parallax_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def parallax_status_string(status: int) -> str:
    return load_library().parallax_status_string(int(status)).decode()


def _check(status: int):
    if status != PARALLAX_OK:
        raise ParallaxError(status, parallax_status_string(status))


def _strides(t: torch.Tensor) -> parallax_strides:
    if t.stride(-1) != 1:
        raise ValueError("the feature dimension must be contiguous (stride 1)")
    s = t.stride()
    return parallax_strides(s[0], s[1], s[2])


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _on(device: torch.device, stream):
    """Context for the binding's own allocations (outputs, workspaces, fills):
    the stream the kernels are launched on.  The caching allocator then
    orders the reuse of a buffer freed here (an internal workspace) after
    those kernels; allocated on another stream it could be handed to new
    work there while the kernels still read it."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return torch.cuda.stream(stream)


def _stream_ordered(fn):
    """Runs a binding with its allocations on the launch stream (see _on)."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        dev = args[0].device if args and isinstance(args[0], torch.Tensor) else None
        with _on(dev, stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _need(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))


def parallax_attn_fwd_workspace_size(B: int, H: int, L: int, d: int) -> int:
    """Bytes of device workspace the prefill needs for these sizes."""
    return int(load_library().parallax_attn_fwd_workspace_size(int(B), int(H), int(L), int(d)))


@_stream_ordered
def parallax_attn_fwd(q, k, v, r, *, softmax_scale=None, window=0, n_sink=0,
                      out=None, lse=None, workspace=None, stream=None):
    """Causal Parallax prefill. q, k, v, r: bf16 [B,H,L,d] -> (o fp32 [B,H,L,d], lse fp32 [B,H,L]).

    ``workspace`` (a device tensor of at least
    ``parallax_attn_fwd_workspace_size(B, H, L, d)`` bytes) is allocated with
    torch when not given.
    """
    return _fwd("parallax_attn_fwd", q, k, v, r, softmax_scale, window, n_sink, out, lse,
                workspace, stream)


@_stream_ordered
def parallax_attn_fwd_precise(q, k, v, r, *, softmax_scale=None, window=0, n_sink=0,
                              out=None, lse=None, workspace=None, stream=None):
    """parallax_attn_fwd with two-part float16 weights (accurate for large probe scores)."""
    return _fwd("parallax_attn_fwd_precise", q, k, v, r, softmax_scale, window, n_sink, out, lse,
                workspace, stream)


@_stream_ordered
def parallax_attn_fwd_noalloc(q, k, v, r, *, softmax_scale=None, window=0, n_sink=0, out, lse,
                              stream=None):
    """parallax_attn_fwd with the library's own 64 MiB device workspace per GPU:
    the C call allocates nothing, so ``out`` (fp32 [B,H,L,d]) and ``lse`` (fp32
    [B,H,L], contiguous) must be given.  Calls whose work overlaps on one GPU
    race for that workspace."""
    return _fwd("parallax_attn_fwd_noalloc", q, k, v, r, softmax_scale, window, n_sink, out, lse,
                None, stream)


@_stream_ordered
def parallax_attn_fwd_f32(q, k, v, r, *, softmax_scale=None, window=0, n_sink=0, out=None,
                          lse=None, stream=None):
    """The prefill in fp32 throughout for fp32 inputs (untiled; small problems).
    q, k, v, r: fp32 [B,H,L,d] -> (o fp32 [B,H,L,d], lse fp32 [B,H,L])."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (r, "r")):
        _need(t, n, torch.float32, 4)
        if t.shape != q.shape:
            raise ValueError("q, k, v and r must share one [B,H,L,d] shape")
    B, H, L, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 4)
    _need(lse, "lse", torch.float32, 3)
    if tuple(out.shape) != (B, H, L, d) or tuple(lse.shape) != (B, H, L):
        raise ValueError("out / lse have the wrong shape")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    st = load_library().parallax_attn_fwd_f32(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), r.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, H, L, d, _strides(q), _strides(k), _strides(v), _strides(r), _strides(out),
        float(softmax_scale), int(window), int(n_sink), _stream_handle(q.device, stream))
    _check(st)
    return out, lse


def _fwd(entry, q, k, v, r, softmax_scale, window, n_sink, out, lse, workspace, stream):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (r, "r")):
        _need(t, n, torch.bfloat16, 4)
        if t.shape != q.shape:
            raise ValueError("q, k, v and r must share one [B,H,L,d] shape")
    B, H, L, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 4)
    _need(lse, "lse", torch.float32, 3)
    if tuple(out.shape) != (B, H, L, d) or tuple(lse.shape) != (B, H, L):
        raise ValueError("out / lse have the wrong shape")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    lib = load_library()
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), r.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, H, L, d, _strides(q), _strides(k), _strides(v), _strides(r),
            _strides(out), float(softmax_scale), int(window), int(n_sink)]
    if entry != "parallax_attn_fwd_noalloc":
        ws_bytes = parallax_attn_fwd_workspace_size(B, H, L, d)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
            raise TypeError("workspace must be a device tensor")
        args += [workspace.data_ptr(), workspace.numel() * workspace.element_size()]
    st = getattr(lib, entry)(*args, _stream_handle(q.device, stream))
    _check(st)
    return out, lse


def _workspace(workspace, nbytes: int, device):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
        raise TypeError("workspace must be a device tensor")
    return workspace, workspace.numel() * workspace.element_size()


@_stream_ordered
def parallax_attn_fwd_train(q, k, v, r, *, softmax_scale=None, window=0, n_sink=0,
                            workspace=None, stream=None):
    """Prefill forward that also saves what the backward needs.

    Returns (o [B,H,L,d], lse [B,H,L], sbar [B,H,L], pv [B,H,L,d]), all fp32
    and contiguous.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (r, "r")):
        _need(t, n, torch.bfloat16, 4)
        if t.shape != q.shape:
            raise ValueError("q, k, v and r must share one [B,H,L,d] shape")
    B, H, L, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = torch.empty((B, H, L, d), **f32)
    lse = torch.empty((B, H, L), **f32)
    sbar = torch.empty((B, H, L), **f32)
    pv = torch.empty((B, H, L, d), **f32)
    lib = load_library()
    workspace, have = _workspace(workspace, parallax_attn_fwd_workspace_size(B, H, L, d), q.device)
    st = lib.parallax_attn_fwd_train(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), r.data_ptr(), out.data_ptr(), lse.data_ptr(),
        sbar.data_ptr(), pv.data_ptr(), B, H, L, d, _strides(q), _strides(k), _strides(v),
        _strides(r), _strides(out), float(softmax_scale), int(window), int(n_sink),
        workspace.data_ptr(), have, _stream_handle(q.device, stream))
    _check(st)
    return out, lse, sbar, pv


def parallax_attn_bwd_workspace_size(B: int, H: int, L: int, d: int) -> int:
    """Bytes of device workspace the backward needs for these sizes."""
    return int(load_library().parallax_attn_bwd_workspace_size(int(B), int(H), int(L), int(d)))


@_stream_ordered
def parallax_attn_bwd(q, k, v, r, dout, o, lse, sbar, pv, *, softmax_scale=None, window=0,
                      n_sink=0, grads=None, workspace=None, stream=None):
    """Prefill backward.  q, k, v, r, dout: bf16 [B,H,L,d]; o, lse, sbar, pv from
    parallax_attn_fwd_train.  Returns (dq, dk, dv, dr), fp32 [B,H,L,d] contiguous
    (``grads`` may supply the four output tensors)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (r, "r"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
        if t.shape != q.shape:
            raise ValueError("q, k, v, r and dout must share one [B,H,L,d] shape")
    B, H, L, d = q.shape
    for t, n, shape in ((o, "o", (B, H, L, d)), (lse, "lse", (B, H, L)),
                        (sbar, "sbar", (B, H, L)), (pv, "pv", (B, H, L, d))):
        _need(t, n, torch.float32, len(shape))
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("%s must be a contiguous fp32 tensor of shape %s" % (n, shape))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if grads is None:
        grads = tuple(torch.empty((B, H, L, d), dtype=torch.float32, device=q.device)
                      for _ in range(4))
    for t, n in zip(grads, ("dq", "dk", "dv", "dr")):
        _need(t, n, torch.float32, 4)
        if tuple(t.shape) != (B, H, L, d) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous fp32 [B,H,L,d] tensor" % n)
    dq, dk, dv, dr = grads
    lib = load_library()
    workspace, have = _workspace(workspace, parallax_attn_bwd_workspace_size(B, H, L, d), q.device)
    st = lib.parallax_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), r.data_ptr(), dout.data_ptr(),
        o.data_ptr(), lse.data_ptr(), sbar.data_ptr(), pv.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dr.data_ptr(), B, H, L, d,
        _strides(q), _strides(k), _strides(v), _strides(r), _strides(dout),
        float(softmax_scale), int(window), int(n_sink), workspace.data_ptr(), have,
        _stream_handle(q.device, stream))
    _check(st)
    return dq, dk, dv, dr


@_stream_ordered
def parallax_attn_decode(q, r, k_cache, v_cache, seqlens=None, *, softmax_scale=None,
                         num_splits=16, out=None, lse=None, stream=None):
    """Decode step. q, r: bf16 [B,H,d]; caches bf16 [B,H,Lmax,d]; seqlens int32 [B] or None.

    Returns (o fp32 [B,H,d], lse fp32 [B,H]).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(r, "r", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, H, Lmax, d = k_cache.shape
    if v_cache.shape != k_cache.shape or tuple(q.shape) != (B, H, d) or r.shape != q.shape:
        raise ValueError("decode shapes disagree")
    if not (q.is_contiguous() and r.is_contiguous()):
        raise ValueError("q and r must be contiguous")
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, 1)
        if seqlens.shape[0] != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 [B] tensor")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    if not (out.is_contiguous() and lse.is_contiguous()):
        raise ValueError("out and lse must be contiguous")
    if tuple(out.shape) != (B, H, d) or tuple(lse.shape) != (B, H):
        raise ValueError("out / lse have the wrong shape")
    lib = load_library()
    st = lib.parallax_attn_decode(
        q.data_ptr(), r.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        seqlens.data_ptr() if seqlens is not None else None, out.data_ptr(), lse.data_ptr(),
        B, H, Lmax, d, _strides(k_cache), _strides(v_cache), float(softmax_scale),
        int(num_splits), _stream_handle(q.device, stream))
    _check(st)
    return out, lse


def parallax_attn_decode_paged_workspace_size(B: int, Hq: int, d: int) -> int:
    """Bytes of device workspace parallax_attn_decode_paged_ws needs."""
    return int(load_library().parallax_attn_decode_paged_workspace_size(B, Hq, d))


@_stream_ordered
def parallax_attn_decode_paged(q, r, k_cache, v_cache, block_table=None, seqlens=None, *,
                               softmax_scale=None, window=0, n_sink=0, num_splits=16,
                               out=None, lse=None, workspace=None, stream=None):
    """General decode step.  q, r: bf16 [B,Hq,d].

    Paged (block_table: int32 [B, max_pages]): k_cache, v_cache are page pools
    [num_pages, page_size, Hkv, d] (any strides, d contiguous).  Contiguous
    (block_table None): caches [B, Lmax, Hkv, d]; pass cache.permute(0, 2, 1, 3)
    for a [B, Hkv, Lmax, d] tensor.  seqlens: int32 [B] or None.
    ``workspace``: with four or more query heads per kv head the call goes
    through parallax_attn_decode_paged_ws, which may split each kv head's
    keys over several workgroups; None allocates its workspace here, a
    uint8 device tensor of at least parallax_attn_decode_paged_workspace_size
    bytes is used as given, and False calls parallax_attn_decode_paged.
    Returns (o fp32 [B,Hq,d], lse fp32 [B,Hq]).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(r, "r", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    P, page_size, Hkv, dk = k_cache.shape
    if v_cache.shape != k_cache.shape or r.shape != q.shape or dk != d:
        raise ValueError("decode shapes disagree")
    if not (q.is_contiguous() and r.is_contiguous()):
        raise ValueError("q and r must be contiguous")
    if k_cache.stride(-1) != 1 or v_cache.stride(-1) != 1:
        raise ValueError("the feature dimension must be contiguous (stride 1)")
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, 2)
        if block_table.shape[0] != B or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor")
        max_pages = block_table.shape[1]
    else:
        if P != B:
            raise ValueError("a contiguous cache has one page per sequence")
        max_pages = 1
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, 1)
        if seqlens.shape[0] != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 [B] tensor")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    if not (out.is_contiguous() and lse.is_contiguous()):
        raise ValueError("out and lse must be contiguous")
    if tuple(out.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out / lse have the wrong shape")
    ks = parallax_strides(k_cache.stride(0), k_cache.stride(2), k_cache.stride(1))
    vs = parallax_strides(v_cache.stride(0), v_cache.stride(2), v_cache.stride(1))
    args = (q.data_ptr(), r.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_table.data_ptr() if block_table is not None else None, P, page_size, max_pages,
            seqlens.data_ptr() if seqlens is not None else None, out.data_ptr(), lse.data_ptr(),
            B, Hq, Hkv, d, ks, vs, float(softmax_scale), int(window), int(n_sink),
            int(num_splits))
    lib = load_library()
    grouped = Hkv > 0 and Hq % Hkv == 0 and Hq // Hkv >= 4
    if workspace is False or not grouped:
        st = lib.parallax_attn_decode_paged(*args, _stream_handle(q.device, stream))
    else:
        if workspace is None:
            workspace = torch.empty(max(1, parallax_attn_decode_paged_workspace_size(B, Hq, d)),
                                    dtype=torch.uint8, device=q.device)
        _need(workspace, "workspace", torch.uint8, 1)
        st = lib.parallax_attn_decode_paged_ws(*args, workspace.data_ptr(), workspace.numel(),
                                               _stream_handle(q.device, stream))
    _check(st)
    return out, lse


@_stream_ordered
def parallax_qkvr_project(x, w, *, out=None, stream=None):
    """Fused projections Y = X W^T.  x: bf16 [M, K]; w: bf16 [N, K] (the stacked
    W_Q, W_K, W_V, W_R rows).  Returns bf16 [M, N] (row i = [q_i | k_i | v_i | rho_i])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 2)
    M, K = x.shape
    N, Kw = w.shape
    if Kw != K:
        raise ValueError("x and w disagree on K")
    if x.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("x and w must have contiguous rows")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be a [M, N] bf16 tensor with contiguous rows")
    st = load_library().parallax_qkvr_project(
        x.data_ptr(), w.data_ptr(), out.data_ptr(), M, N, K, x.stride(0), w.stride(0),
        out.stride(0), _stream_handle(x.device, stream))
    _check(st)
    return out


@_stream_ordered
def parallax_hadamard_out(o, alpha=None, beta=None, *, out=None, stream=None):
    """Walsh-Hadamard output projection y = alpha * (O H_n / sqrt(n)) + beta.

    o: fp32 [B, H, L, d] attention output (any strides, d contiguous); the
    heads of each token are concatenated to n = H*d features.  alpha, beta:
    fp32 [n] or None.  Returns bf16 [B, L, n] (or writes ``out``, a bf16
    [B*L, n] or [B, L, n] tensor with contiguous rows)."""
    _need(o, "o", torch.float32, 4)
    B, H, L, d = o.shape
    n = H * d
    for t, name in ((alpha, "alpha"), (beta, "beta")):
        if t is not None:
            _need(t, name, torch.float32, 1)
            if t.shape[0] != n or not t.is_contiguous():
                raise ValueError("%s must be a contiguous fp32 [%d] tensor" % (name, n))
    if out is None:
        out = torch.empty((B, L, n), dtype=torch.bfloat16, device=o.device)
    if out.dtype != torch.bfloat16 or out.device.type != "cuda":
        raise TypeError("out must be a bf16 device tensor")
    rows = out.view(-1, n) if out.dim() == 3 and out.is_contiguous() else out
    if rows.dim() != 2 or tuple(rows.shape) != (B * L, n) or rows.stride(1) != 1:
        raise ValueError("out must be [B*L, n] (or contiguous [B, L, n]) with contiguous rows")
    st = load_library().parallax_hadamard_out(
        o.data_ptr(), _strides(o), B, H, L, d,
        alpha.data_ptr() if alpha is not None else None,
        beta.data_ptr() if beta is not None else None,
        rows.data_ptr(), rows.stride(0), _stream_handle(o.device, stream))
    _check(st)
    return out


BASED_FEATURES = 160


def parallax_based_state_floats(dk: int, dv: int) -> int:
    """fp32 values of one (batch, head) Based state: 160 x 16 (dv / 16 + 1)."""
    return int(load_library().parallax_based_state_floats(int(dk), int(dv)))


def parallax_based_workspace_size(B: int, H: int, L: int, dk: int, dv: int) -> int:
    return int(load_library().parallax_based_workspace_size(int(B), int(H), int(L), int(dk),
                                                             int(dv)))


def based_state_shape(dv: int):
    """Shape of one (batch, head) state: (160 features, 16 (dv/16 + 1) columns)."""
    return (BASED_FEATURES, 16 * (dv // 16 + 1))


@_stream_ordered
def parallax_based_fwd(q, k, v, *, scale=None, return_state=False, out=None, workspace=None,
                       stream=None):
    """Causal Based linear attention (Taylor kernel 1 + x + x^2/2, x = scale q.k).

    q, k: bf16 [B, H, L, 16]; v: bf16 [B, H, L, dv] (dv 64 or 128).  Returns
    o fp32 [B, H, L, dv], and with ``return_state`` also the state after the
    last token (fp32 [B, H, 160, 16 (dv/16 + 1)]) for parallax_based_decode."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, L, dk = q.shape
    dv = v.shape[3]
    if tuple(k.shape) != (B, H, L, dk) or tuple(v.shape[:3]) != (B, H, L):
        raise ValueError("q, k, v shapes disagree")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 4)
    if tuple(out.shape) != (B, H, L, dv):
        raise ValueError("out has the wrong shape")
    state = None
    if return_state:
        state = torch.zeros((B, H) + based_state_shape(dv), dtype=torch.float32, device=q.device)
    nbytes = parallax_based_workspace_size(B, H, L, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = load_library().parallax_based_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        state.data_ptr() if state is not None else None, B, H, L, dk, dv, _strides(q),
        _strides(k), _strides(v), _strides(out), float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device, stream))
    _check(st)
    return (out, state) if return_state else out


@_stream_ordered
def parallax_based_decode(q, k, v, state, *, scale=None, out=None, stream=None):
    """One Based decode step: q, k bf16 [B, H, 16], v bf16 [B, H, dv]; ``state``
    fp32 [B, H, 160, 16 (dv/16 + 1)] is updated in place.  Returns o fp32 [B, H, dv]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(state, "state", torch.float32, 4)
    B, H, dk = q.shape
    dv = v.shape[2]
    if tuple(k.shape) != (B, H, dk) or tuple(v.shape[:2]) != (B, H):
        raise ValueError("q, k, v shapes disagree")
    if tuple(state.shape) != (B, H) + based_state_shape(dv) or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 [B, H, 160, 16 (dv/16 + 1)] tensor")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    if tuple(out.shape) != (B, H, dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [B, H, dv] tensor")
    st = load_library().parallax_based_decode(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), state.data_ptr(), out.data_ptr(), B, H, dk, dv,
        float(scale), _stream_handle(q.device, stream))
    _check(st)
    return out


def split_qkvr(y, B, L, H, d):
    """The four parts of a parallax_qkvr_project output [B*L, 4*H*d] as strided
    [B, H, L, d] views (no copies): (q, k, v, rho)."""
    if y.shape[1] != 4 * H * d or y.shape[0] != B * L:
        raise ValueError("y must be [B*L, 4*H*d]")
    ld = y.stride(0)
    return tuple(torch.as_strided(y, (B, H, L, d), (L * ld, d, ld, 1), y.storage_offset() + p * H * d)
                 for p in range(4))
