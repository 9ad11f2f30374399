"""Loader for the plain fp64 CPU oracle (``parallax_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module; the product path (the HIP library and
its binding) never imports it, and it is no fallback for the GPU.

The oracle computes the Parallax forward from its definition (review page
"Parallax: Parameterized Local Linear Attention for Language Modeling",
sec. 1 and sec. 3): softmax weights over the visible keys, the weighted key
mean, the probe correction rho.(k_j - kbar) and the corrected weighted sum of
values, all in fp64; and its backward (the gradients of a loss through o with
respect to q, k, v and rho) by reverse-mode steps of the same definition;
exact Local Linear Attention (the probe by a conjugate-gradient solve) for
comparison with it; the fused input projections x [W_Q; W_K; W_V; W_R]^T;
the Walsh-Hadamard output projection alpha * (Y H / sqrt(n)) + beta; and
Based linear attention with the second-order Taylor kernel 1 + x + x^2/2.
Everything here converts arrays to contiguous float64
and calls the C code; no arithmetic of the method lives in this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "parallax_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.POINTER(ctypes.c_long)
_I = ctypes.POINTER(ctypes.c_int)


def build(out: str = LIBRARY, source: str = SOURCE) -> str:
    """Compile the oracle with gcc (OpenMP, IEEE fp64; no fast-math).

    ``source`` defaults to ``parallax_oracle.c``; the oracle's self-test
    builds patched copies of it that each plant one deliberate mistake.
    """
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path) or (
                path == LIBRARY and os.path.getmtime(SOURCE) > os.path.getmtime(path)):
            build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.parallax_oracle_rows.restype = ctypes.c_int
        lib.parallax_oracle_rows.argtypes = [
            _D, _D, _L, ctypes.c_long, _D, _D, ctypes.c_long, ctypes.c_int,
            ctypes.c_double, ctypes.c_long, ctypes.c_long, _D, _D, ctypes.c_int]
        lib.parallax_oracle_fwd.restype = ctypes.c_int
        lib.parallax_oracle_fwd.argtypes = [
            _D, _D, _D, _D, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.parallax_oracle_bwd.restype = ctypes.c_int
        lib.parallax_oracle_bwd.argtypes = [
            _D, _D, _D, _D, _D, _D, _D, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.parallax_oracle_project.restype = ctypes.c_int
        lib.parallax_oracle_project.argtypes = [_D, _D, _D, ctypes.c_long, ctypes.c_long,
                                                ctypes.c_long, ctypes.c_int]
        lib.parallax_oracle_hadamard.restype = ctypes.c_int
        lib.parallax_oracle_hadamard.argtypes = [_D, _D, _D, _D, ctypes.c_long, ctypes.c_long,
                                                 ctypes.c_int]
        lib.parallax_oracle_based.restype = ctypes.c_int
        lib.parallax_oracle_based.argtypes = [_D, _D, _D, _D, ctypes.c_long, ctypes.c_long,
                                              ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                              ctypes.c_double, ctypes.c_int]
        lib.parallax_oracle_lla_rows.restype = ctypes.c_int
        lib.parallax_oracle_lla_rows.argtypes = [
            _D, _L, ctypes.c_long, _D, _D, ctypes.c_long, ctypes.c_int, ctypes.c_double,
            ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_double,
            _D, _D, _I, ctypes.c_int]
        lib.parallax_oracle_decode_ext.restype = ctypes.c_int
        lib.parallax_oracle_decode_ext.argtypes = [
            _D, _D, _D, _D, _I, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_long, ctypes.c_long,
            ctypes.c_int]
        lib.parallax_oracle_decode.restype = ctypes.c_int
        lib.parallax_oracle_decode.argtypes = [
            _D, _D, _D, _D, _I, _D, _D, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_int, ctypes.c_double, ctypes.c_int]
        self.lib = lib

    @staticmethod
    def _f64(a) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(a, dtype=np.float64))

    @staticmethod
    def _ptr(a: np.ndarray):
        return a.ctypes.data_as(_D)

    def fwd(self, q, k, v, r, scale=None, window=0, n_sink=0, nthreads=None):
        """Prefill forward on [B,H,L,d] arrays; returns (o [B,H,L,d], lse [B,H,L])."""
        q, k, v, r = (self._f64(x) for x in (q, k, v, r))
        B, H, L, d = q.shape
        for x in (k, v, r):
            if x.shape != q.shape:
                raise ValueError("q, k, v, r must share one [B,H,L,d] shape")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        o = np.zeros_like(q)
        lse = np.zeros((B, H, L), dtype=np.float64)
        rc = self.lib.parallax_oracle_fwd(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(r), self._ptr(o),
            self._ptr(lse), B, H, L, d, float(scale), int(window), int(n_sink),
            int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return o, lse

    def bwd(self, q, k, v, r, dout, scale=None, window=0, n_sink=0, nthreads=None):
        """Prefill backward on [B,H,L,d] arrays: gradients of a loss through o
        (dout = dLoss/do; lse carries none).  Returns (dq, dk, dv, dr)."""
        q, k, v, r, dout = (self._f64(x) for x in (q, k, v, r, dout))
        B, H, L, d = q.shape
        for x in (k, v, r, dout):
            if x.shape != q.shape:
                raise ValueError("q, k, v, r, dout must share one [B,H,L,d] shape")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        dq, dk, dv, dr = (np.zeros_like(q) for _ in range(4))
        rc = self.lib.parallax_oracle_bwd(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(r), self._ptr(dout),
            self._ptr(dq), self._ptr(dk), self._ptr(dv), self._ptr(dr),
            B, H, L, d, float(scale), int(window), int(n_sink),
            int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return dq, dk, dv, dr

    def rows(self, q_rows, r_rows, pos, k, v, scale, window=0, n_sink=0, nthreads=None):
        """Selected rows of one (batch, head) slice.

        q_rows, r_rows: [n, d]; pos: [n] positions; k, v: [n_ctx, d].
        Returns (o [n, d], lse [n]).
        """
        q_rows, r_rows, k, v = (self._f64(x) for x in (q_rows, r_rows, k, v))
        pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
        n, d = q_rows.shape
        n_ctx = k.shape[0]
        o = np.zeros((n, d), dtype=np.float64)
        lse = np.zeros(n, dtype=np.float64)
        rc = self.lib.parallax_oracle_rows(
            self._ptr(q_rows), self._ptr(r_rows), pos.ctypes.data_as(_L), n,
            self._ptr(k), self._ptr(v), n_ctx, d, float(scale), int(window), int(n_sink),
            self._ptr(o), self._ptr(lse), int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return o, lse

    def decode(self, q, r, k_cache, v_cache, seqlens=None, scale=None, nthreads=None):
        """Decode: q, r [B,H,d]; caches [B,H,Lmax,d]; seqlens [B] or None."""
        q, r, k_cache, v_cache = (self._f64(x) for x in (q, r, k_cache, v_cache))
        B, H, Lmax, d = k_cache.shape
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        sl = None
        if seqlens is not None:
            sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
        o = np.zeros((B, H, d), dtype=np.float64)
        lse = np.zeros((B, H), dtype=np.float64)
        rc = self.lib.parallax_oracle_decode(
            self._ptr(q), self._ptr(r), self._ptr(k_cache), self._ptr(v_cache),
            sl.ctypes.data_as(_I) if sl is not None else None, self._ptr(o), self._ptr(lse),
            B, H, Lmax, d, float(scale), int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return o, lse


    def project(self, x, w, nthreads=None):
        """Fused projections y = x w^T: x [M, K], w [N, K] -> y [M, N] (fp64)."""
        x, w = self._f64(x), self._f64(w)
        M, K = x.shape
        N = w.shape[0]
        if w.shape[1] != K:
            raise ValueError("x and w disagree on K")
        y = np.zeros((M, N), dtype=np.float64)
        rc = self.lib.parallax_oracle_project(self._ptr(x), self._ptr(w), self._ptr(y), M, N, K,
                                              int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return y

    def hadamard(self, y, alpha=None, beta=None, nthreads=None):
        """Walsh-Hadamard output projection alpha * (y H_n / sqrt(n)) + beta with H_n
        the Sylvester Hadamard matrix: y [M, n] (n a power of two) -> [M, n] (fp64)."""
        y = self._f64(y)
        M, n = y.shape
        a = None if alpha is None else self._f64(np.broadcast_to(alpha, (n,)))
        b = None if beta is None else self._f64(np.broadcast_to(beta, (n,)))
        out = np.zeros((M, n), dtype=np.float64)
        rc = self.lib.parallax_oracle_hadamard(self._ptr(y), self._ptr(a) if a is not None else None,
                                               self._ptr(b) if b is not None else None,
                                               self._ptr(out), M, n,
                                               int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return out

    def based(self, q, k, v, scale=None, nthreads=None):
        """Based linear attention, causal, weights 1 + x + x^2/2 with x = scale q.k:
        q, k [B, H, L, dk], v [B, H, L, dv] -> o [B, H, L, dv] (fp64).  scale
        defaults to 1/sqrt(dk)."""
        q, k, v = (self._f64(x) for x in (q, k, v))
        B, H, L, dk = q.shape
        dv = v.shape[-1]
        if k.shape != q.shape or v.shape[:3] != (B, H, L):
            raise ValueError("q, k, v shapes disagree")
        if scale is None:
            scale = dk ** -0.5
        o = np.zeros((B, H, L, dv), dtype=np.float64)
        rc = self.lib.parallax_oracle_based(self._ptr(q), self._ptr(k), self._ptr(v),
                                            self._ptr(o), B, H, L, dk, dv, float(scale),
                                            int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return o

    def lla_rows(self, q_rows, pos, k, v, scale, window=0, n_sink=0, max_iters=None, tol=1e-12,
                 ridge=0.0, nthreads=None):
        """Exact Local Linear Attention on selected rows of one (b, h) slice: the
        p-weighted least-squares intercept, with the probe found by conjugate
        gradients.  Returns (o [n, d], rho [n, d], CG iterations [n])."""
        q_rows, k, v = (self._f64(x) for x in (q_rows, k, v))
        pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
        n, d = q_rows.shape
        if max_iters is None:
            max_iters = 4 * d
        o = np.zeros((n, d), dtype=np.float64)
        rho = np.zeros((n, d), dtype=np.float64)
        iters = np.zeros(n, dtype=np.int32)
        rc = self.lib.parallax_oracle_lla_rows(
            self._ptr(q_rows), pos.ctypes.data_as(_L), n, self._ptr(k), self._ptr(v),
            k.shape[0], d, float(scale), int(window), int(n_sink), int(max_iters), float(tol),
            float(ridge), self._ptr(o), self._ptr(rho), iters.ctypes.data_as(_I),
            int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return o, rho, iters

    def decode_ext(self, q, r, k_cache, v_cache, seqlens=None, scale=None, window=0, n_sink=0,
                   nthreads=None):
        """General decode: q, r [B,Hq,d]; caches [B,Hkv,Lmax,d] (Hq a multiple of
        Hkv; query head h reads kv head h // (Hq // Hkv)); window and sinks as
        in the prefill.  Returns (o [B,Hq,d], lse [B,Hq])."""
        q, r, k_cache, v_cache = (self._f64(x) for x in (q, r, k_cache, v_cache))
        B, Hkv, Lmax, d = k_cache.shape
        Hq = q.shape[1]
        if q.shape != (B, Hq, d) or r.shape != q.shape or v_cache.shape != k_cache.shape:
            raise ValueError("decode shapes disagree")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        sl = None
        if seqlens is not None:
            sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
        o = np.zeros((B, Hq, d), dtype=np.float64)
        lse = np.zeros((B, Hq), dtype=np.float64)
        rc = self.lib.parallax_oracle_decode_ext(
            self._ptr(q), self._ptr(r), self._ptr(k_cache), self._ptr(v_cache),
            sl.ctypes.data_as(_I) if sl is not None else None, self._ptr(o), self._ptr(lse),
            B, Hq, Hkv, Lmax, d, float(scale), int(window), int(n_sink),
            int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return o, lse


_default = None


def default_threads() -> int:
    """Host threads for the oracle: all cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def default() -> Oracle:
    """The oracle built from the unmodified source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle(LIBRARY)
    return _default
