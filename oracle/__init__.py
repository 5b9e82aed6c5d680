"""FP64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the two share no
code.

The arithmetic lives in ``oracle.c`` (plain C, double precision), built into
``liboracle.so`` by :func:`build`.  This module only marshals numpy float64
arrays through ctypes.  ``oracle.c`` states the definition each function
follows and the readings taken where the source pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")


def build(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile ``src`` with gcc into the shared library ``out`` (always rebuilds)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """ctypes front end of one build of ``oracle.c``."""

    def __init__(self, path: str = LIBRARY):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.oracle_attention.argtypes = [dp, dp, dp, dp, dp, dp, L, L, L, L, L, L,
                                         ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_softmax_3pass.argtypes = [dp, dp, L, L]
        lib.oracle_softmax_3pass.restype = None
        lib.oracle_softmax_online.argtypes = [dp, dp, L, L, L]
        lib.oracle_softmax_online.restype = None
        lib.oracle_partial_state.argtypes = [dp, dp, L, L, L, dp, dp, dp]
        lib.oracle_partial_state.restype = None
        lib.oracle_merge_states.argtypes = [dp, dp, dp, dp, dp, dp, L, L, dp, dp, dp]
        lib.oracle_merge_states.restype = None
        lib.oracle_split_kv_decode.argtypes = [dp, dp, dp, L, L, L, L, L,
                                               ctypes.c_double, dp, dp]
        lib.oracle_split_kv_decode.restype = ctypes.c_int
        lib.oracle_attention_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, L, L, L, L, L, L,
                                             ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.oracle_attention_bwd.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def attention(self, q, k, v, causal: bool = False, scale: float | None = None,
                  want_p: bool = False, nthreads: int | None = None):
        """Standard attention (materialised scores, three-pass softmax) in FP64.

        q: [..., N, d], k: [..., Nk, d], v: [..., Nk, dv] with identical
        leading dims (flattened to heads).  Query i sits at position Nk-N+i
        under ``causal``.  Returns ``(o, lse)`` or ``(o, lse, p)`` with ``p``
        of shape [..., N, Nk].  A row that sees no key gets o = 0, lse = -inf.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        lead = q.shape[:-2]
        N, d = q.shape[-2:]
        Nk, dv = v.shape[-2:]
        if k.shape[:-2] != lead or v.shape[:-2] != lead or k.shape[-2:] != (Nk, d):
            raise ValueError("shape mismatch between q, k, v")
        heads = int(np.prod(lead)) if lead else 1
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        o = np.empty(lead + (N, dv), dtype=np.float64)
        lse = np.empty(lead + (N,), dtype=np.float64)
        p = np.empty(lead + (N, Nk), dtype=np.float64) if want_p else None
        if nthreads is None:
            nthreads = max(1, len(os.sched_getaffinity(0)))
        rc = self.lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _ptr(p), 1, heads, N, Nk, d, dv,
                                       int(bool(causal)), float(scale), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_attention failed with code {rc}")
        return (o, lse, p) if want_p else (o, lse)

    def attention_bwd(self, q, k, v, dout, causal: bool = False, scale: float | None = None,
                      nthreads: int | None = None):
        """Backward of standard attention in FP64: the gradients (dq, dk, dv) of
        sum(dout * O) with O = attention(q, k, v).  Shapes as :meth:`attention`,
        dout like O."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        lead = q.shape[:-2]
        N, d = q.shape[-2:]
        Nk, dv = v.shape[-2:]
        if (k.shape[:-2] != lead or v.shape[:-2] != lead or k.shape[-2:] != (Nk, d)
                or dout.shape != lead + (N, dv)):
            raise ValueError("shape mismatch between q, k, v, dout")
        heads = int(np.prod(lead)) if lead else 1
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dvv = np.empty_like(v)
        if nthreads is None:
            nthreads = max(1, len(os.sched_getaffinity(0)))
        rc = self.lib.oracle_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                           _ptr(dk), _ptr(dvv), 1, heads, N, Nk, d, dv,
                                           int(bool(causal)), float(scale), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_attention_bwd failed with code {rc}")
        return dq, dk, dvv

    def softmax_3pass(self, x):
        x = _f64(x)
        y = np.empty_like(x)
        n = x.shape[-1]
        self.lib.oracle_softmax_3pass(_ptr(x), _ptr(y), x.size // n, n)
        return y

    def softmax_online(self, x, block: int = 128):
        x = _f64(x)
        y = np.empty_like(x)
        n = x.shape[-1]
        self.lib.oracle_softmax_online(_ptr(x), _ptr(y), x.size // n, n, int(block))
        return y

    def partial_state(self, x, v=None):
        """(m, l, o) of one segment: x [rows, n], v [n, dv] or None."""
        x = _f64(x)
        rows, n = x.shape
        m = np.empty(rows)
        l = np.empty(rows)
        if v is None:
            self.lib.oracle_partial_state(_ptr(x), None, rows, n, 0, _ptr(m), _ptr(l), None)
            return m, l, None
        v = _f64(v)
        dv = v.shape[1]
        o = np.empty((rows, dv))
        self.lib.oracle_partial_state(_ptr(x), _ptr(v), rows, n, dv, _ptr(m), _ptr(l), _ptr(o))
        return m, l, o

    def merge_states(self, a, b):
        """Merge two partial states (m, l, o); o may be None on both sides."""
        ma, la = _f64(a[0]), _f64(a[1])
        mb, lb = _f64(b[0]), _f64(b[1])
        oa = None if a[2] is None else _f64(a[2])
        ob = None if b[2] is None else _f64(b[2])
        rows = ma.shape[0]
        m = np.empty(rows)
        l = np.empty(rows)
        if oa is None or ob is None:
            self.lib.oracle_merge_states(_ptr(ma), _ptr(la), None, _ptr(mb), _ptr(lb), None,
                                         rows, 0, _ptr(m), _ptr(l), None)
            return m, l, None
        dv = oa.shape[1]
        o = np.empty((rows, dv))
        self.lib.oracle_merge_states(_ptr(ma), _ptr(la), _ptr(oa), _ptr(mb), _ptr(lb),
                                     _ptr(ob), rows, dv, _ptr(m), _ptr(l), _ptr(o))
        return m, l, o

    def split_kv_decode(self, q, K, V, n_splits: int, scale: float | None = None):
        """Split-KV decode of q [R,d] against K [S,d], V [S,dv] -> (o, lse, used)."""
        q, K, V = _f64(q), _f64(K), _f64(V)
        R, d = q.shape
        S, dv = V.shape
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        o = np.empty((R, dv))
        lse = np.empty(R)
        used = self.lib.oracle_split_kv_decode(_ptr(q), _ptr(K), _ptr(V), R, S, d, dv,
                                               int(n_splits), float(scale), _ptr(o), _ptr(lse))
        if used < 0:
            raise RuntimeError("oracle_split_kv_decode: bad arguments")
        return o, lse, used


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` in this directory (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def attention(*a, **kw):
    return default().attention(*a, **kw)


def softmax_3pass(x):
    return default().softmax_3pass(x)


def softmax_online(x, block: int = 128):
    return default().softmax_online(x, block)


def partial_state(x, v=None):
    return default().partial_state(x, v)


def merge_states(a, b):
    return default().merge_states(a, b)


def split_kv_decode(q, K, V, n_splits: int, scale: float | None = None):
    return default().split_kv_decode(q, K, V, n_splits, scale)


def attention_bwd(*a, **kw):
    return default().attention_bwd(*a, **kw)
