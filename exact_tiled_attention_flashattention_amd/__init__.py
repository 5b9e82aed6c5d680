"""Exact tiled attention (FlashAttention forward + split-KV flash-decoding)
for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libfa.so``, whose C ABI is declared in
``include/fa.h``.  This module only marshals arguments: it checks tensor
shapes and dtypes, allocates the outputs (and the decode workspace) with
torch on the inputs' device, and passes raw device pointers and the current
torch stream to the library.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "fwd", "decode_splitkv", "decode_splitkv_gqa", "decode_splitkv_noalloc",
    "decode_splitkv_workspace_size", "DECODE_NOALLOC_MAX_WORKSPACE",
    "decode_splitkv_auto_splits", "bwd", "bwd_workspace_size", "status_string",
    "FAError", "library", "LIBRARY_PATH", "FA_OK", "FA_ERR_INVALID_ARG",
    "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_LAUNCH",
]

LIBRARY_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_LAUNCH = range(5)
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
# FA_DECODE_NOALLOC_MAX_WORKSPACE of include/fa.h: the static scratch of
# fa_decode_splitkv_noalloc, in bytes.
DECODE_NOALLOC_MAX_WORKSPACE = 16 << 20

_lib = None


class FAError(RuntimeError):
    """A non-OK status returned by libfa.so."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)}")
        self.status = status


def library() -> ctypes.CDLL:
    """The loaded ``libfa.so`` with its C signatures declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise FileNotFoundError(
            f"{LIBRARY_PATH} is not built; run "
            "`python -m exact_tiled_attention_flashattention_amd.build` first")
    lib = ctypes.CDLL(LIBRARY_PATH)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, c_int,
                           ctypes.c_float, c_int, vp]
    lib.fa_fwd.restype = c_int
    lib.fa_decode_splitkv_workspace_size.argtypes = [i64, i64, i64, i64, c_int]
    lib.fa_decode_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, c_int,
                                      ctypes.c_float, c_int, c_int, vp, ctypes.c_size_t, vp]
    lib.fa_decode_splitkv.restype = c_int
    lib.fa_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                              c_int, ctypes.c_float, c_int, c_int, vp]
    lib.fa_decode_splitkv_noalloc.restype = c_int
    lib.fa_decode_splitkv_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                          c_int, ctypes.c_float, c_int, c_int, vp, ctypes.c_size_t,
                                          vp]
    lib.fa_decode_splitkv_gqa.restype = c_int
    lib.fa_decode_splitkv_auto_splits.argtypes = [i64, i64, i64, i64, i64, i64, i64, c_int]
    lib.fa_decode_splitkv_auto_splits.restype = c_int
    lib.fa_bwd_workspace_size.argtypes = [i64, i64, i64]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                           c_int, ctypes.c_float, c_int, vp, ctypes.c_size_t, vp]
    lib.fa_bwd.restype = c_int
    lib.fa_status_string.argtypes = [c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().fa_status_string(int(status)).decode()


def _check_qkv(q, k, v, grouped=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, rows, dim], got {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must live on a GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODE:
        raise TypeError("q, k, v must share one dtype among float32, float16, bfloat16")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    bad = (k.shape[0] != B or v.shape[:2] != k.shape[:2] or k.shape[3] != d
           or v.shape[2] != k.shape[2])
    bad = bad or (Hkv != H if not grouped else (Hkv < 1 or H % Hkv != 0))
    if bad:
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if grouped:
        return B, H, Hkv, N, k.shape[2], d, v.shape[3]
    return B, H, N, k.shape[2], d, v.shape[3]


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output or operand tensor must match exactly: the C ABI
    sees only a raw pointer, so a short, strided, mistyped or host tensor
    would be written out of bounds instead of failing."""
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        got = (f"{tuple(t.shape)} {t.dtype} on {t.device}"
               f"{'' if t.is_contiguous() else ', non-contiguous'}"
               if isinstance(t, torch.Tensor) else type(t).__name__)
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}, got {got}")
    return t


def _check_workspace(t, nbytes, device):
    """A caller-supplied workspace: a contiguous uint8 tensor on ``device`` of
    at least ``nbytes`` bytes."""
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.device != device
            or not t.is_contiguous() or t.numel() < nbytes):
        got = (f"{t.numel()} {t.dtype} elements on {t.device}" if isinstance(t, torch.Tensor)
               else type(t).__name__)
        raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {nbytes} "
                         f"bytes on {device}, got {got}")
    return t


def _stream_handle(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: float | None = None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Exact attention forward through ``fa_fwd``.

    q [B,H,N,d], k [B,H,Nk,d], v [B,H,Nk,dv] contiguous on one GPU, one dtype.
    Returns ``(o, lse)``: o [B,H,N,dv] in the input dtype, lse [B,H,N] float32.
    ``scale`` defaults to 1/sqrt(d).  The call is asynchronous on ``stream``
    (default: torch's current stream).
    """
    B, H, N, Nk, d, dv = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = (torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device) if out is None
           else _check_buffer("out", out, (B, H, N, dv), q.dtype, q.device))
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _check_buffer("lse", lse, (B, H, N), torch.float32, q.device))
    st = library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, Nk, d, dv, int(bool(causal)), float(scale),
                          _DTYPE_CODE[q.dtype], _stream_handle(q.device, stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return out, lse


def bwd_workspace_size(B: int, H: int, N: int) -> int:
    return int(library().fa_bwd_workspace_size(B, H, N))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, causal: bool = False, scale: float | None = None,
        workspace: torch.Tensor | None = None, dq: torch.Tensor | None = None,
        dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
        stream: torch.cuda.Stream | None = None):
    """Attention backward through ``fa_bwd``.

    ``o`` and ``lse`` are :func:`fwd`'s outputs for the same q, k, v, causal
    and scale; ``dout`` is the gradient of the loss with respect to ``o``.
    Returns ``(dq, dk, dv)`` in the input dtype.
    """
    B, H, N, Nk, d, dvd = _check_qkv(q, k, v)
    for name, t, shape, dtype in (("o", o, (B, H, N, dvd), q.dtype),
                                  ("dout", dout, (B, H, N, dvd), q.dtype),
                                  ("lse", lse, (B, H, N), torch.float32)):
        if (not isinstance(t, torch.Tensor) or tuple(t.shape) != shape or t.dtype != dtype
                or t.device != q.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} "
                             f"on {q.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else _check_buffer("dq", dq, q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _check_buffer("dk", dk, k.shape, q.dtype, q.device)
    dv = torch.empty_like(v) if dv is None else _check_buffer("dv", dv, v.shape, q.dtype, q.device)
    need = bwd_workspace_size(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, need, q.device)
    st = library().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          B, H, N, Nk, d, dvd, int(bool(causal)), float(scale),
                          _DTYPE_CODE[q.dtype], workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(),
                          _stream_handle(q.device, stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def decode_splitkv_workspace_size(B: int, H: int, N: int, dv: int, num_splits: int) -> int:
    return int(library().fa_decode_splitkv_workspace_size(B, H, N, dv, num_splits))


def decode_splitkv_auto_splits(B: int, Hq: int, Hkv: int, N: int, Nk: int, d: int, dv: int,
                               dtype: torch.dtype) -> int:
    """The split count ``num_splits=0`` selects (``fa_decode_splitkv_auto_splits``)."""
    n = int(library().fa_decode_splitkv_auto_splits(B, Hq, Hkv, N, Nk, d, dv, _DTYPE_CODE[dtype]))
    if n < 1:
        raise ValueError(f"no split count for B={B} Hq={Hq} Hkv={Hkv} N={N} Nk={Nk} d={d} dv={dv}")
    return n


def decode_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                   scale: float | None = None, num_splits: int = 64,
                   workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Split-KV flash-decoding through ``fa_decode_splitkv``.

    Same inputs and result as :func:`fwd`; the keys of each head are cut into
    ``num_splits`` segments reduced in parallel, then merged by a second kernel.
    ``workspace`` (a uint8 device tensor of at least
    :func:`decode_splitkv_workspace_size` bytes) is allocated if not given.
    ``num_splits=0`` lets the library choose (:func:`decode_splitkv_auto_splits`).
    """
    B, H, N, Nk, d, dv = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = (torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device) if out is None
           else _check_buffer("out", out, (B, H, N, dv), q.dtype, q.device))
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _check_buffer("lse", lse, (B, H, N), torch.float32, q.device))
    if num_splits < 0:
        raise ValueError(f"num_splits must be >= 0, got {num_splits}")
    splits = num_splits or decode_splitkv_auto_splits(B, H, H, N, Nk, d, dv, q.dtype)
    nbytes = decode_splitkv_workspace_size(B, H, N, dv, splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, nbytes, q.device)
    st = library().fa_decode_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, H, N, Nk, d, dv, int(bool(causal)),
                                     float(scale), _DTYPE_CODE[q.dtype], int(num_splits),
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream_handle(q.device, stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_splitkv")
    return out, lse


def decode_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           causal: bool = False, scale: float | None = None,
                           num_splits: int = 64, out: torch.Tensor | None = None,
                           lse: torch.Tensor | None = None,
                           stream: torch.cuda.Stream | None = None):
    """Split-KV flash-decoding through ``fa_decode_splitkv_noalloc``: the
    result of :func:`decode_splitkv`, with the per-segment partials in the
    library's static per-GPU scratch (``DECODE_NOALLOC_MAX_WORKSPACE`` bytes)
    instead of a workspace; the library allocates nothing.  Calls that
    overlap on one GPU race.  Pass ``out`` and ``lse`` to allocate nothing
    here either."""
    B, H, N, Nk, d, dv = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = (torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device) if out is None
           else _check_buffer("out", out, (B, H, N, dv), q.dtype, q.device))
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _check_buffer("lse", lse, (B, H, N), torch.float32, q.device))
    st = library().fa_decode_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             out.data_ptr(), lse.data_ptr(), B, H, N, Nk, d, dv,
                                             int(bool(causal)), float(scale), _DTYPE_CODE[q.dtype],
                                             int(num_splits), _stream_handle(q.device, stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_splitkv_noalloc")
    return out, lse


def decode_splitkv_gqa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                       scale: float | None = None, num_splits: int = 64,
                       workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Grouped-query split-KV decoding through ``fa_decode_splitkv_gqa``.

    q [B,Hq,N,d]; k [B,Hkv,Nk,d], v [B,Hkv,Nk,dv] with Hq a multiple of Hkv;
    query head h uses key/value head h // (Hq // Hkv).  Returns ``(o, lse)``
    like :func:`decode_splitkv`.
    """
    B, Hq, Hkv, N, Nk, d, dv = _check_qkv(q, k, v, grouped=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = (torch.empty((B, Hq, N, dv), dtype=q.dtype, device=q.device) if out is None
           else _check_buffer("out", out, (B, Hq, N, dv), q.dtype, q.device))
    lse = (torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None
           else _check_buffer("lse", lse, (B, Hq, N), torch.float32, q.device))
    if num_splits < 0:
        raise ValueError(f"num_splits must be >= 0, got {num_splits}")
    splits = num_splits or decode_splitkv_auto_splits(B, Hq, Hkv, N, Nk, d, dv, q.dtype)
    nbytes = decode_splitkv_workspace_size(B, Hq, N, dv, splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, nbytes, q.device)
    st = library().fa_decode_splitkv_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         lse.data_ptr(), B, Hq, Hkv, N, Nk, d, dv,
                                         int(bool(causal)), float(scale), _DTYPE_CODE[q.dtype],
                                         int(num_splits), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         _stream_handle(q.device, stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_splitkv_gqa")
    return out, lse
