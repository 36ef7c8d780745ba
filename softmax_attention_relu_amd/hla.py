"""Thin Python binding of libhla (ctypes).

Argument marshalling only: every step of every operation runs in the HIP
kernels of ``libhla.so``. PyTorch is used for device memory and the current
HIP stream. The functions carry the C entry points' names; tensors are
contiguous device tensors of shape (B, N, H, 64) (bf16, or float32 for the
linear paths), state tensors are float32.

If ``libhla.so`` has not been built, ``lib()`` raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_size_t, c_void_p

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# HLA_LIBRARY selects another build of the library (e.g. the host-sanitizer build)
LIB_PATH = os.environ.get("HLA_LIBRARY") or os.path.join(_PKG, "libhla.so")

HLA_OK, HLA_ERR_INVALID_ARG, HLA_ERR_UNSUPPORTED, HLA_ERR_WORKSPACE, HLA_ERR_HIP = range(5)
HLA_BF16, HLA_F32 = 0, 1

# every function declared in include/hla.h
EXPORTS = (
    "hla_rope_table_host",
    "hla_linear_attn_workspace",
    "hla_linear_attn",
    "hla_linear_attn_noalloc_max_workspace",
    "hla_linear_attn_noalloc",
    "hla_linear_attn_chunked_workspace",
    "hla_linear_attn_chunked",
    "hla_linear_attn_causal_workspace",
    "hla_linear_attn_causal",
    "hla_linear_attn_backward_workspace",
    "hla_linear_attn_backward",
    "hla_linear_attn_backward_saved",
    "hla_linear_attn_chunked_backward_workspace",
    "hla_linear_attn_chunked_backward",
    "hla_softmax_anchor_workspace",
    "hla_softmax_anchor",
    "hla_softmax_anchor_lse",
    "hla_softmax_anchor_block_sparse",
    "hla_softmax_anchor_backward_workspace",
    "hla_softmax_anchor_backward",
    "hla_softmax_anchor_backward_saved",
    "hla_attnres_route",
    "hla_status_string",
)


class HlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {hla_status_string(status)} (status {status})")


class hla_rope3d(ctypes.Structure):
    _fields_ = [
        ("grid_t", c_int), ("grid_h", c_int), ("grid_w", c_int),
        ("d_t", c_int), ("d_h", c_int), ("d_w", c_int),
        ("cs_t", c_void_p), ("cs_h", c_void_p), ("cs_w", c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhla.so (once). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m softmax_attention_relu_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.hla_rope_table_host.argtypes = [c_int, c_int, c_int, c_double, POINTER(c_float)]
        L.hla_rope_table_host.restype = c_int
        L.hla_linear_attn_workspace.argtypes = [c_int, c_int, c_int, c_int]
        L.hla_linear_attn_workspace.restype = c_size_t
        L.hla_linear_attn.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                      POINTER(hla_rope3d), c_float, c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_linear_attn.restype = c_int
        L.hla_linear_attn_noalloc_max_workspace.argtypes = []
        L.hla_linear_attn_noalloc_max_workspace.restype = c_size_t
        L.hla_linear_attn_noalloc.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                              c_void_p, POINTER(hla_rope3d), c_float, c_void_p, c_void_p]
        L.hla_linear_attn_noalloc.restype = c_int
        L.hla_linear_attn_chunked_workspace.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.hla_linear_attn_chunked_workspace.restype = c_size_t
        L.hla_linear_attn_chunked.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                              c_void_p, POINTER(hla_rope3d), c_float, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_linear_attn_chunked.restype = c_int
        L.hla_linear_attn_causal_workspace.argtypes = [c_int, c_int, c_int, c_int]
        L.hla_linear_attn_causal_workspace.restype = c_size_t
        L.hla_linear_attn_causal.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                             c_void_p, POINTER(hla_rope3d), c_float, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_linear_attn_causal.restype = c_int
        L.hla_linear_attn_backward_workspace.argtypes = [c_int, c_int, c_int, c_int]
        L.hla_linear_attn_backward_workspace.restype = c_size_t
        L.hla_linear_attn_backward.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                               c_void_p, POINTER(hla_rope3d), c_float, c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_linear_attn_backward.restype = c_int
        L.hla_linear_attn_backward_saved.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                                     c_void_p, c_void_p, POINTER(hla_rope3d), c_float, c_void_p,
                                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                     c_void_p, c_size_t, c_void_p]
        L.hla_linear_attn_backward_saved.restype = c_int
        L.hla_linear_attn_chunked_backward_workspace.argtypes = [c_int, c_int, c_int, c_int, c_int]
        L.hla_linear_attn_chunked_backward_workspace.restype = c_size_t
        L.hla_linear_attn_chunked_backward.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                                       c_void_p, c_void_p, POINTER(hla_rope3d), c_float, c_void_p,
                                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                                       c_void_p]
        L.hla_linear_attn_chunked_backward.restype = c_int
        L.hla_softmax_anchor_workspace.argtypes = [c_int, c_int, c_int, c_int]
        L.hla_softmax_anchor_workspace.restype = c_size_t
        L.hla_softmax_anchor.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_float, c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_softmax_anchor.restype = c_int
        L.hla_softmax_anchor_lse.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_softmax_anchor_lse.restype = c_int
        L.hla_softmax_anchor_block_sparse.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                                      c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_int,
                                                      c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_softmax_anchor_block_sparse.restype = c_int
        L.hla_softmax_anchor_backward_workspace.argtypes = [c_int, c_int, c_int, c_int]
        L.hla_softmax_anchor_backward_workspace.restype = c_size_t
        L.hla_softmax_anchor_backward.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                                  c_void_p, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                                  c_void_p, c_void_p, c_size_t, c_void_p]
        L.hla_softmax_anchor_backward.restype = c_int
        L.hla_softmax_anchor_backward_saved.argtypes = [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                                        c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p,
                                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                                        c_void_p]
        L.hla_softmax_anchor_backward_saved.restype = c_int
        L.hla_attnres_route.argtypes = [c_int, c_int, c_int, c_int, c_int, POINTER(c_void_p), c_void_p, c_void_p,
                                        c_float, c_void_p, c_void_p, c_void_p]
        L.hla_attnres_route.restype = c_int
        L.hla_status_string.argtypes = [c_int]
        L.hla_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def hla_status_string(status: int) -> str:
    return lib().hla_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != HLA_OK:
        raise HlaError(status, where)


# ----------------------------------------------------------------------------
# torch marshalling helpers

def _torch():
    import torch  # imported lazily so host-only users do not need a GPU

    return torch


def _ptr(t) -> int | None:
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("libhla takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libhla takes contiguous tensors")
    return t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HLA_BF16
    if t.dtype == torch.float32:
        return HLA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream_obj(stream):
    """The torch stream the call runs on (a torch stream, a raw HIP stream handle, or None for current)."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _bnhd(q):
    torch = _torch()
    if not isinstance(q, torch.Tensor):
        raise TypeError("q: expected a torch.Tensor")
    if q.dim() != 4:
        raise ValueError("q: expected a (B, N, H, D) tensor")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"q: unsupported dtype {q.dtype}")
    return tuple(int(x) for x in q.shape)


class _Checks:
    """Shape, dtype and device checks of every tensor argument, before any call into the library.

    The kernels read and write through raw pointers, so a tensor of the wrong
    shape or dtype would be read or written out of bounds; every mismatch is a
    ValueError raised here instead. All shapes and dtypes are checked first,
    then that every tensor is a contiguous device tensor on one device.
    """

    def __init__(self):
        self._items = []

    def add(self, name, t, shape, dtype, optional=True):
        if t is None:
            if not optional:
                raise ValueError(f"{name} is required")
            return self
        self._items.append((name, t, tuple(shape), dtype))
        return self

    def run(self):
        torch = _torch()
        for name, t, shape, dtype in self._items:
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name}: expected a torch.Tensor")
            if tuple(t.shape) != shape:
                raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
            if t.dtype != dtype:
                raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        dev = None
        for name, t, _, _ in self._items:
            if not t.is_cuda:
                raise ValueError(f"{name}: libhla takes device tensors")
            if not t.is_contiguous():
                raise ValueError(f"{name}: libhla takes contiguous tensors")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name}: on {t.device}, the other tensors on {dev}")


def _check_rope(rope, N: int, D: int, device=None):
    """A Rope3D's grid must cover the N tokens and its tables must match its grid and bands (and, when
    ``device`` is given, sit on it)."""
    if rope is None:
        return
    if not isinstance(rope, Rope3D):
        raise TypeError("rope: expected a Rope3D")
    T, Hg, Wg = rope.grid
    if T * Hg * Wg != N:
        raise ValueError(f"rope: grid {rope.grid} covers {T * Hg * Wg} tokens, the call has {N}")
    if sum(rope.bands) != D:
        raise ValueError(f"rope: bands {rope.bands} do not sum to D = {D}")
    torch = _torch()
    for nm, tab, n, d in zip("thw", rope.tables, rope.grid, rope.bands):
        if d == 0:
            continue
        if tuple(tab.shape) != (n, d // 2, 2) or tab.dtype != torch.float32:
            raise ValueError(f"rope: the {nm} table is {tuple(tab.shape)} {tab.dtype}, expected ({n}, {d // 2}, 2) "
                             "float32")
        if device is not None and (not tab.is_cuda or tab.device != device or not tab.is_contiguous()):
            raise ValueError(f"rope: the {nm} table must be a contiguous tensor on {device}")


def _workspace(nbytes: int, device, ws):
    torch = _torch()
    if ws is None:
        ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    else:
        if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous() or ws.device != device:
            raise ValueError(f"ws: expected a contiguous device tensor on {device}")
    return ws, ws.numel() * ws.element_size()


# ----------------------------------------------------------------------------
# RoPE tables

def hla_rope_table_host(length: int, pos0: int, d_band: int, base: float = 10000.0) -> np.ndarray:
    """(cos, sin) table of one band: float32 array of shape (length, d_band/2, 2)."""
    out = np.zeros((max(int(length), 0), max(int(d_band), 0) // 2, 2), dtype=np.float32)
    ptr = out.ctypes.data_as(POINTER(c_float)) if out.size else POINTER(c_float)()
    _check(lib().hla_rope_table_host(int(length), int(pos0), int(d_band), float(base), ptr), "hla_rope_table_host")
    return out


class Rope3D:
    """Device RoPE tables for a (T, Hg, Wg) grid; the t table starts at frame ``t_offset``."""

    def __init__(self, grid, bands=(16, 24, 24), base: float = 10000.0, t_offset: int = 0, device="cuda",
                 tables=None):
        torch = _torch()
        self.grid = tuple(int(x) for x in grid)
        self.bands = tuple(int(x) for x in bands)
        if tables is None:
            pos0 = (int(t_offset), 0, 0)
            tables = [hla_rope_table_host(n, p, d, base) if d > 0 else np.zeros((1, 1, 2), np.float32)
                      for n, p, d in zip(self.grid, pos0, self.bands)]
        self.tables = [torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device) for t in tables]
        s = hla_rope3d()
        s.grid_t, s.grid_h, s.grid_w = self.grid
        s.d_t, s.d_h, s.d_w = self.bands
        s.cs_t, s.cs_h, s.cs_w = (t.data_ptr() for t in self.tables)
        self._struct = s

    def struct(self) -> hla_rope3d:
        return self._struct


def _rope_ptr(rope):
    return None if rope is None else ctypes.byref(rope.struct())


# ----------------------------------------------------------------------------
# entry points
#
# Every function checks each tensor argument's shape, dtype and device against
# q (or the router's first source) before calling into the library, and
# allocates what it returns and any workspace on the stream the call runs on.

def _like(chk: _Checks, ref, **named):
    """Register tensors that must have q's shape and dtype."""
    for name, t in named.items():
        chk.add(name, t, ref.shape, ref.dtype)
    return chk


def _state(chk: _Checks, B, H, D, **named):
    """Register fp32 state tensors: the kv ones are (B, H, D, D), the key sums (B, H, D)."""
    torch = _torch()
    for name, t in named.items():
        chk.add(name, t, (B, H, D, D) if "kv" in name else (B, H, D), torch.float32)
    return chk


def hla_linear_attn_workspace(B: int, N: int, H: int, D: int = 64) -> int:
    return int(lib().hla_linear_attn_workspace(B, N, H, D))


def hla_linear_attn(q, k, v, g=None, rope: Rope3D | None = None, eps: float = 1e-6, o=None, ws=None, stream=None):
    """Bidirectional ReLU+RoPE linear attention; returns o."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if o is None:
            o = torch.empty_like(q)
        ws, nbytes = _workspace(hla_linear_attn_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_linear_attn(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _rope_ptr(rope),
                              float(eps), _ptr(o), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_linear_attn")
    return o


def hla_linear_attn_noalloc_max_workspace() -> int:
    return int(lib().hla_linear_attn_noalloc_max_workspace())


def hla_linear_attn_noalloc(q, k, v, g=None, rope: Rope3D | None = None, eps: float = 1e-6, o=None, stream=None):
    """hla_linear_attn with the library's static workspace (the C call allocates nothing); returns o.

    Calls that overlap on one GPU share that workspace and race. ``o`` is allocated here when not given.
    """
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    if o is None:
        with torch.cuda.stream(st):
            o = torch.empty_like(q)
    r = lib().hla_linear_attn_noalloc(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                      _rope_ptr(rope), float(eps), _ptr(o), st.cuda_stream)
    _check(r, "hla_linear_attn_noalloc")
    return o


def hla_linear_attn_chunked_workspace(B: int, N: int, H: int, D: int, chunk_tokens: int) -> int:
    return int(lib().hla_linear_attn_chunked_workspace(B, N, H, D, chunk_tokens))


def hla_linear_attn_chunked(q, k, v, chunk_tokens: int, g=None, rope: Rope3D | None = None, eps: float = 1e-6,
                            kv_in=None, ksum_in=None, kv_out=None, ksum_out=None, o=None, ws=None, stream=None):
    """Block-causal linear attention with carried state; returns o (state goes to kv_out/ksum_out)."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o)
    _state(chk, B, H, D, kv_in=kv_in, ksum_in=ksum_in, kv_out=kv_out, ksum_out=ksum_out)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if o is None:
            o = torch.empty_like(q)
        ws, nbytes = _workspace(hla_linear_attn_chunked_workspace(B, N, H, D, chunk_tokens), q.device, ws)
    r = lib().hla_linear_attn_chunked(_dtype_code(q), B, N, H, D, int(chunk_tokens), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(g), _rope_ptr(rope), float(eps), _ptr(kv_in), _ptr(ksum_in),
                                      _ptr(kv_out), _ptr(ksum_out), _ptr(o), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_linear_attn_chunked")
    return o


def hla_linear_attn_causal_workspace(B: int, N: int, H: int, D: int) -> int:
    return int(lib().hla_linear_attn_causal_workspace(B, N, H, D))


def hla_linear_attn_causal(q, k, v, g=None, rope: Rope3D | None = None, eps: float = 1e-6, kv_in=None, ksum_in=None,
                           kv_out=None, ksum_out=None, o=None, ws=None, stream=None):
    """Token-causal linear attention (bf16) with optional carried state; returns o."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o)
    _state(chk, B, H, D, kv_in=kv_in, ksum_in=ksum_in, kv_out=kv_out, ksum_out=ksum_out)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if o is None:
            o = torch.empty_like(q)
        ws, nbytes = _workspace(hla_linear_attn_causal_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_linear_attn_causal(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                     _rope_ptr(rope), float(eps), _ptr(kv_in), _ptr(ksum_in), _ptr(kv_out),
                                     _ptr(ksum_out), _ptr(o), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_linear_attn_causal")
    return o


def hla_linear_attn_backward_workspace(B: int, N: int, H: int, D: int = 64) -> int:
    return int(lib().hla_linear_attn_backward_workspace(B, N, H, D))


def _grad_outputs(q, k, v, g, dq, dk, dv, dg):
    torch = _torch()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if g is not None and dg is None:
        dg = torch.empty_like(g)
    return dq, dk, dv, dg


def hla_linear_attn_backward_saved(q, k, v, kv, ksum, do, g=None, rope: Rope3D | None = None, eps: float = 1e-6,
                                   dq=None, dk=None, dv=None, dg=None, ws=None, stream=None):
    """Gradients of the bidirectional linear attention (bf16) given the forward's state kv (B, H, D, D) and
    ksum (B, H, D), as hla_linear_attn_chunked returns for chunk_tokens = N; returns (dq, dk, dv, dg)."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, do=do, dq=dq, dk=dk, dv=dv, dg=dg)
    chk.add("kv", kv, (B, H, D, D), torch.float32, optional=False)
    chk.add("ksum", ksum, (B, H, D), torch.float32, optional=False)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        dq, dk, dv, dg = _grad_outputs(q, k, v, g, dq, dk, dv, dg)
        ws, nbytes = _workspace(hla_linear_attn_backward_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_linear_attn_backward_saved(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                             _rope_ptr(rope), float(eps), _ptr(kv), _ptr(ksum), _ptr(do), _ptr(dq),
                                             _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_linear_attn_backward_saved")
    return dq, dk, dv, dg


def hla_linear_attn_backward(q, k, v, do, g=None, rope: Rope3D | None = None, eps: float = 1e-6, dq=None, dk=None,
                             dv=None, dg=None, ws=None, stream=None):
    """Gradients of the bidirectional linear attention (bf16); returns (dq, dk, dv, dg), dg None without g."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, do=do, dq=dq, dk=dk, dv=dv, dg=dg)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        dq, dk, dv, dg = _grad_outputs(q, k, v, g, dq, dk, dv, dg)
        ws, nbytes = _workspace(hla_linear_attn_backward_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_linear_attn_backward(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _rope_ptr(rope), float(eps), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                       _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_linear_attn_backward")
    return dq, dk, dv, dg


def hla_linear_attn_chunked_backward_workspace(B: int, N: int, H: int, D: int, chunk_tokens: int) -> int:
    return int(lib().hla_linear_attn_chunked_backward_workspace(B, N, H, D, chunk_tokens))


def hla_linear_attn_chunked_backward(q, k, v, do, chunk_tokens: int, g=None, rope: Rope3D | None = None,
                                     eps: float = 1e-6, kv_in=None, ksum_in=None, dkv_out=None, dksum_out=None,
                                     dq=None, dk=None, dv=None, dg=None, dkv_in=None, dksum_in=None, ws=None,
                                     stream=None):
    """Gradients of the block-causal linear attention (bf16), cache terms included.

    Returns (dq, dk, dv, dg); the carried state's gradient goes to dkv_in/dksum_in when given.
    """
    torch = _torch()
    B, N, H, D = _bnhd(q)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, do=do, dq=dq, dk=dk, dv=dv, dg=dg)
    _state(chk, B, H, D, kv_in=kv_in, ksum_in=ksum_in, dkv_out=dkv_out, dksum_out=dksum_out, dkv_in=dkv_in,
           dksum_in=dksum_in)
    _check_rope(rope, N, D)
    chk.run()
    _check_rope(rope, N, D, q.device)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        dq, dk, dv, dg = _grad_outputs(q, k, v, g, dq, dk, dv, dg)
        ws, nbytes = _workspace(hla_linear_attn_chunked_backward_workspace(B, N, H, D, chunk_tokens), q.device, ws)
    r = lib().hla_linear_attn_chunked_backward(
        _dtype_code(q), B, N, H, D, int(chunk_tokens), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _rope_ptr(rope),
        float(eps), _ptr(kv_in), _ptr(ksum_in), _ptr(do), _ptr(dkv_out), _ptr(dksum_out), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dg), _ptr(dkv_in), _ptr(dksum_in), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_linear_attn_chunked_backward")
    return dq, dk, dv, dg


def hla_softmax_anchor_workspace(B: int, N: int, H: int, D: int = 64) -> int:
    return int(lib().hla_softmax_anchor_workspace(B, N, H, D))


def _default_scale(scale, D):
    return 1.0 / float(D) ** 0.5 if scale is None else scale


def hla_softmax_anchor(q, k, v, g=None, scale: float | None = None, o=None, ws=None, stream=None):
    """Gated non-causal softmax attention (bf16); returns o."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    scale = _default_scale(scale, D)
    _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o).run()
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if o is None:
            o = torch.empty_like(q)
        ws, nbytes = _workspace(hla_softmax_anchor_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_softmax_anchor(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g), float(scale),
                                 _ptr(o), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_softmax_anchor")
    return o


def hla_softmax_anchor_lse(q, k, v, g=None, scale: float | None = None, o=None, lse=None, ws=None, stream=None):
    """Gated softmax anchor (bf16) that also writes each row's natural-log normaliser; returns (o, lse),
    lse float [B, H, N]."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    scale = _default_scale(scale, D)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o)
    chk.add("lse", lse, (B, H, N), torch.float32).run()
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        ws, nbytes = _workspace(hla_softmax_anchor_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_softmax_anchor_lse(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g), float(scale),
                                     _ptr(o), _ptr(lse), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_softmax_anchor_lse")
    return o, lse


def hla_softmax_anchor_backward_workspace(B: int, N: int, H: int, D: int = 64) -> int:
    return int(lib().hla_softmax_anchor_backward_workspace(B, N, H, D))


def hla_softmax_anchor_backward(q, k, v, do, g=None, scale: float | None = None, dq=None, dk=None, dv=None, dg=None,
                                ws=None, stream=None):
    """Gradients of the gated softmax anchor (bf16); returns (dq, dk, dv, dg), dg None without g."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    scale = _default_scale(scale, D)
    _like(_Checks(), q, q=q, k=k, v=v, g=g, do=do, dq=dq, dk=dk, dv=dv, dg=dg).run()
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        dq, dk, dv, dg = _grad_outputs(q, k, v, g, dq, dk, dv, dg)
        ws, nbytes = _workspace(hla_softmax_anchor_backward_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_softmax_anchor_backward(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          float(scale), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                          _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_softmax_anchor_backward")
    return dq, dk, dv, dg


def hla_softmax_anchor_backward_saved(q, k, v, o, lse, do, g=None, scale: float | None = None, dq=None, dk=None,
                                      dv=None, dg=None, ws=None, stream=None):
    """Gradients of the gated softmax anchor from its saved output o and normalisers lse (as written by
    hla_softmax_anchor_lse); returns (dq, dk, dv, dg), dg None without g."""
    torch = _torch()
    B, N, H, D = _bnhd(q)
    scale = _default_scale(scale, D)
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, do=do, dq=dq, dk=dk, dv=dv, dg=dg)
    chk.add("o", o, q.shape, q.dtype, optional=False)
    chk.add("lse", lse, (B, H, N), torch.float32, optional=False).run()
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        dq, dk, dv, dg = _grad_outputs(q, k, v, g, dq, dk, dv, dg)
        ws, nbytes = _workspace(hla_softmax_anchor_backward_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_softmax_anchor_backward_saved(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                                float(scale), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                                _ptr(dv), _ptr(dg), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_softmax_anchor_backward_saved")
    return dq, dk, dv, dg


SPARSE_Q_BLOCK = 128  # query rows per block of the block-sparse anchor
SPARSE_K_BLOCK = 64   # keys per named block


def hla_softmax_anchor_block_sparse(q, k, v, blocks, counts, g=None, scale: float | None = None, o=None, ws=None,
                                    stream=None):
    """Block-sparse gated softmax anchor (bf16); returns o.

    blocks: int32 device tensor (B, H, ceil(N/128), max_blocks) of key-block indices (64 keys each);
    counts: int32 device tensor (B, H, ceil(N/128)) of entries used per query block.
    """
    torch = _torch()
    B, N, H, D = _bnhd(q)
    scale = _default_scale(scale, D)
    nqb = -(-N // SPARSE_Q_BLOCK)
    if not isinstance(blocks, torch.Tensor) or blocks.dim() != 4:
        raise ValueError("blocks must be a (B, H, ceil(N/128), max_blocks) tensor")
    chk = _like(_Checks(), q, q=q, k=k, v=v, g=g, o=o)
    chk.add("blocks", blocks, (B, H, nqb, int(blocks.shape[3])), torch.int32, optional=False)
    chk.add("counts", counts, (B, H, nqb), torch.int32, optional=False).run()
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if o is None:
            o = torch.empty_like(q)
        ws, nbytes = _workspace(hla_softmax_anchor_workspace(B, N, H, D), q.device, ws)
    r = lib().hla_softmax_anchor_block_sparse(_dtype_code(q), B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                              float(scale), _ptr(blocks), _ptr(counts), int(blocks.shape[3]),
                                              _ptr(o), _ptr(ws), nbytes, st.cuda_stream)
    _check(r, "hla_softmax_anchor_block_sparse")
    return o


def hla_attnres_route(sources, w, phi_t=None, eps: float = 1e-6, h=None, alpha=None, stream=None):
    """AttnRes router over S sources of shape (B, T, C); returns (h, alpha).

    ``alpha`` may be a float32 (B, T, S) tensor to fill, True to allocate one,
    or None to skip the routing-weight output.
    """
    torch = _torch()
    srcs = list(sources)
    if not srcs:
        raise ValueError("need at least one source")
    s0 = srcs[0]
    if not isinstance(s0, torch.Tensor) or s0.dim() != 3:
        raise ValueError("sources: expected (B, T, C) tensors")
    if s0.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"sources: unsupported dtype {s0.dtype}")
    B, T, C = (int(x) for x in s0.shape)
    S = len(srcs)
    chk = _Checks()
    for i, src in enumerate(srcs):
        chk.add(f"sources[{i}]", src, (B, T, C), s0.dtype, optional=False)
    chk.add("w", w, (C,), torch.float32, optional=False)
    chk.add("phi_t", phi_t, (B, C), torch.float32)
    chk.add("h", h, (B, T, C), s0.dtype)
    if alpha is not True:
        chk.add("alpha", alpha, (B, T, S), torch.float32)
    chk.run()
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if h is None:
            h = torch.empty_like(s0)
        if alpha is True:
            alpha = torch.empty((B, T, S), dtype=torch.float32, device=s0.device)
    arr = (c_void_p * S)(*[_ptr(x) for x in srcs])
    r = lib().hla_attnres_route(_dtype_code(s0), B, T, C, S, arr, _ptr(w), _ptr(phi_t), float(eps), _ptr(h),
                                _ptr(alpha), st.cuda_stream)
    _check(r, "hla_attnres_route")
    return h, alpha
