"""Python binding of the HIP library ``libtw.so`` (C ABI in ``include/tw.h``).

Argument marshalling only: every step of the forward runs in the library's
gfx950 kernels.  PyTorch provides device memory and the current HIP stream.
Importing this module fails loudly when the library has not been built
(``python -m activation_sparse_feed_gate_amd.build``); there is no fallback.

Low-level functions carry the C names and take preallocated tensors:
``tw_pack_gate`` (and ``tw_pack_gate_noalloc``, which takes no workspace),
``tw_sparse_ffn_fwd``, ``tw_ffn_fwd``, ``tw_workspace_bytes``,
``tw_ffn_workspace_bytes``, ``tw_gate_dense``, ``tw_pack_dense`` and the
hybrid training storage ``tw_hybrid_pack``, ``tw_hybrid_up``,
``tw_hybrid_down`` with its backward ``tw_hybrid_bwd_dh``, ``tw_hybrid_bwd_dx``,
``tw_hybrid_bwd_dw``.  ``pack_gate``, ``pack_unfused``, ``sparse_ffn``, ``ffn``,
``hybrid_forward`` and ``hybrid_backward`` allocate their outputs and return
them.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library links against

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libtw.so")

if not os.path.exists(LIBRARY):
    raise ImportError(
        f"{LIBRARY} is missing: build it with `python -m activation_sparse_feed_gate_amd.build`")

_lib = ctypes.CDLL(LIBRARY)

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_lib.tw_status_str.restype = ctypes.c_char_p
_lib.tw_status_str.argtypes = [_i]
_lib.tw_last_error.restype = ctypes.c_char_p
_lib.tw_last_error.argtypes = []
_lib.tw_workspace_bytes.restype = _sz
_lib.tw_workspace_bytes.argtypes = [_i] * 6
_lib.tw_ffn_workspace_bytes.restype = _sz
_lib.tw_ffn_workspace_bytes.argtypes = [_i] * 3
_lib.tw_pack_gate.restype = _i
_lib.tw_pack_gate.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                              _vp, _sz, _vp, _vp]
_lib.tw_pack_gate_noalloc.restype = _i
_lib.tw_pack_gate_noalloc.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i,
                                      _vp, _vp, _vp]
_lib.tw_sparse_ffn_fwd.restype = _i
_lib.tw_sparse_ffn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                   _vp, _i, _vp, _vp, _sz, _vp, _vp]
_lib.tw_ffn_fwd.restype = _i
_lib.tw_ffn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp, _vp]
_lib.tw_gate_dense.restype = _i
_lib.tw_gate_dense.argtypes = [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]
_lib.tw_pack_dense_workspace_bytes.restype = _sz
_lib.tw_pack_dense_workspace_bytes.argtypes = [_i, _i]
_lib.tw_pack_dense.restype = _i
_lib.tw_pack_dense.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp,
                               _vp]
_lib.tw_hybrid_pack.restype = _i
_lib.tw_hybrid_pack.argtypes = [_i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                _i, _vp, _vp]
_lib.tw_hybrid_up.restype = _i
_lib.tw_hybrid_up.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.tw_hybrid_down_workspace_bytes.restype = _sz
_lib.tw_hybrid_down_workspace_bytes.argtypes = [_i]
_lib.tw_hybrid_down.restype = _i
_lib.tw_hybrid_down.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp,
                                _vp, _sz, _vp, _vp]
_lib.tw_hybrid_bwd_dh.restype = _i
_lib.tw_hybrid_bwd_dh.argtypes = [_vp, _vp, _i, _i, _i, _i, ctypes.c_float, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.tw_hybrid_bwd_dx_workspace_bytes.restype = _sz
_lib.tw_hybrid_bwd_dx_workspace_bytes.argtypes = [_i]
_lib.tw_hybrid_bwd_dx.restype = _i
_lib.tw_hybrid_bwd_dx.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _i, _vp, _vp, _vp, _vp, _sz, _vp, _vp]
_lib.tw_hybrid_bwd_dw_workspace_bytes.restype = _sz
_lib.tw_hybrid_bwd_dw_workspace_bytes.argtypes = [_i] * 5
_lib.tw_hybrid_bwd_dw.restype = _i
_lib.tw_hybrid_bwd_dw.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]

TW_OK, TW_EINVAL, TW_EUNSUPPORTED, TW_EHIP = 0, 1, 2, 3


class TwError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.tw_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_lib.tw_status_str(status).decode()}: {msg}")


def _check(status: int, where: str) -> None:
    if status != TW_OK:
        raise TwError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return t.data_ptr()


_F32, _I32, _BF16, _U8T = torch.float32, torch.int32, torch.bfloat16, torch.uint8


class _Args:
    """Checks every tensor of one call against the shape, dtype and device
    the kernels assume.  The C ABI receives bare pointers and cannot see a
    buffer's size, so a tensor of the wrong shape (say a packing made for
    another T or C) would be read or written out of bounds on the device:
    such calls raise here, before the library is called."""

    def __init__(self, where, ref):
        self.where = where
        self.device = ref.device

    def _common(self, t, name, dtype):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.where}: {name} must be a tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{self.where}: {name} must be {dtype}, got {t.dtype}")
        if t.device != self.device:
            raise ValueError(f"{self.where}: {name} is on {t.device}, the inputs on {self.device}")

    def shape(self, t, name, dtype, shape):
        """t must have exactly this shape (None: t may be None)."""
        if t is None:
            raise ValueError(f"{self.where}: {name} is required")
        self._common(t, name, dtype)
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.where}: {name} has shape {tuple(t.shape)}, "
                             f"expected {tuple(shape)}")

    def opt(self, t, name, dtype, shape):
        if t is not None:
            self.shape(t, name, dtype, shape)

    def overflow_list(self, ovf_rows, ovf_count, R_max):
        """The overflow list of tw_pack_gate: both tensors, or both None (no
        list is built)."""
        if ovf_rows is None and ovf_count is None:
            return
        self.room(ovf_rows, "ovf_rows", _I32, max(R_max, 1))
        self.room(ovf_count, "ovf_count", _I32, 1)

    def room(self, t, name, dtype, n):
        """t must be one-dimensional with at least n elements."""
        if t is None:
            raise ValueError(f"{self.where}: {name} is required")
        self._common(t, name, dtype)
        if t.dim() != 1 or t.numel() < n:
            raise ValueError(f"{self.where}: {name} has shape {tuple(t.shape)}, expected "
                             f"one dimension of at least {n} elements")

    def bytes(self, t, name):
        """A workspace: any dtype, on the inputs' device (its size is checked
        by the library against the bytes it needs)."""
        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.where}: {name} must be a tensor")
        if t.device != self.device:
            raise ValueError(f"{self.where}: {name} is on {t.device}, the inputs on {self.device}")


def _dims2(t, name, where):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{where}: {name} must be a two-dimensional tensor")
    return t.shape


def _tiles(N, T, where):
    if T <= 0 or N % T:
        raise ValueError(f"{where}: N={N} is not a multiple of the tile width T={T}")
    return N // T


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _events(events):
    if events is None:
        return None
    arr = (ctypes.c_void_p * len(events))(*[int(e) for e in events])
    return ctypes.cast(arr, ctypes.c_void_p), arr


# ----------------------------------------------------------------- C names --
def tw_workspace_bytes(M, K, N, T, C, R_max) -> int:
    return int(_lib.tw_workspace_bytes(M, K, N, T, C, R_max))


def tw_ffn_workspace_bytes(M, K, N) -> int:
    return int(_lib.tw_ffn_workspace_bytes(M, K, N))


def tw_pack_gate(x, wg_t, T, C, tw_val, tw_idx, tw_cnt, ovf_rows, ovf_count, R_max, ws,
                 z_debug=None, stream=None, events=None) -> None:
    M, K = _dims2(x, "x", "tw_pack_gate")
    N = _dims2(wg_t, "wg_t", "tw_pack_gate")[0]
    NT = _tiles(N, T, "tw_pack_gate")
    a = _Args("tw_pack_gate", x)
    a.shape(x, "x", _BF16, (M, K))
    a.shape(wg_t, "wg_t", _BF16, (N, K))
    a.shape(tw_val, "tw_val", _F32, (M, NT, C))
    a.shape(tw_idx, "tw_idx", _I32, (M, NT, C))
    a.shape(tw_cnt, "tw_cnt", _I32, (M, NT))
    a.overflow_list(ovf_rows, ovf_count, R_max)
    a.opt(z_debug, "z_debug", _F32, (M, N))
    a.bytes(ws, "ws")
    ev = _events(events)
    st = _lib.tw_pack_gate(_ptr(x), _ptr(wg_t), M, K, N, T, C, _ptr(tw_val), _ptr(tw_idx),
                           _ptr(tw_cnt), _ptr(ovf_rows), _ptr(ovf_count), R_max, _ptr(z_debug),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
                           ev[0] if ev else None)
    _check(st, "tw_pack_gate")


def tw_pack_gate_noalloc(x, wg_t, T, C, tw_val, tw_idx, tw_cnt, ovf_rows, ovf_count, R_max,
                         z_debug=None, stream=None, events=None) -> None:
    """tw_pack_gate on the library's static per-GPU scratch (no workspace)."""
    M, K = _dims2(x, "x", "tw_pack_gate_noalloc")
    N = _dims2(wg_t, "wg_t", "tw_pack_gate_noalloc")[0]
    NT = _tiles(N, T, "tw_pack_gate_noalloc")
    a = _Args("tw_pack_gate_noalloc", x)
    a.shape(x, "x", _BF16, (M, K))
    a.shape(wg_t, "wg_t", _BF16, (N, K))
    a.shape(tw_val, "tw_val", _F32, (M, NT, C))
    a.shape(tw_idx, "tw_idx", _I32, (M, NT, C))
    a.shape(tw_cnt, "tw_cnt", _I32, (M, NT))
    a.overflow_list(ovf_rows, ovf_count, R_max)
    a.opt(z_debug, "z_debug", _F32, (M, N))
    ev = _events(events)
    st = _lib.tw_pack_gate_noalloc(_ptr(x), _ptr(wg_t), M, K, N, T, C, _ptr(tw_val),
                                   _ptr(tw_idx), _ptr(tw_cnt), _ptr(ovf_rows), _ptr(ovf_count),
                                   R_max, _ptr(z_debug), _stream(stream), ev[0] if ev else None)
    _check(st, "tw_pack_gate_noalloc")


def tw_sparse_ffn_fwd(x, wg_t, wu_t, wd, T, C, tw_val, tw_idx, tw_cnt, ovf_rows, ovf_count,
                      R_max, y, ws, stream=None, events=None) -> None:
    M, K = _dims2(x, "x", "tw_sparse_ffn_fwd")
    N = _dims2(wg_t, "wg_t", "tw_sparse_ffn_fwd")[0]
    NT = _tiles(N, T, "tw_sparse_ffn_fwd")
    a = _Args("tw_sparse_ffn_fwd", x)
    a.shape(x, "x", _BF16, (M, K))
    for t, n in ((wg_t, "wg_t"), (wu_t, "wu_t"), (wd, "wd")):
        a.shape(t, n, _BF16, (N, K))
    a.shape(tw_val, "tw_val", _F32, (M, NT, C))
    a.shape(tw_idx, "tw_idx", _I32, (M, NT, C))
    a.shape(tw_cnt, "tw_cnt", _I32, (M, NT))
    a.room(ovf_rows, "ovf_rows", _I32, max(R_max, 1))
    a.room(ovf_count, "ovf_count", _I32, 1)
    a.shape(y, "y", _F32, (M, K))
    a.bytes(ws, "ws")
    ev = _events(events)
    st = _lib.tw_sparse_ffn_fwd(_ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), M, K, N, T, C,
                                _ptr(tw_val), _ptr(tw_idx), _ptr(tw_cnt), _ptr(ovf_rows),
                                _ptr(ovf_count), R_max, _ptr(y), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream),
                                ev[0] if ev else None)
    _check(st, "tw_sparse_ffn_fwd")


def tw_ffn_fwd(x, wg_t, wu_t, wd, y, ws, stream=None, events=None) -> None:
    M, K = _dims2(x, "x", "tw_ffn_fwd")
    N = _dims2(wg_t, "wg_t", "tw_ffn_fwd")[0]
    a = _Args("tw_ffn_fwd", x)
    a.shape(x, "x", _BF16, (M, K))
    for t, n in ((wg_t, "wg_t"), (wu_t, "wu_t"), (wd, "wd")):
        a.shape(t, n, _BF16, (N, K))
    a.shape(y, "y", _F32, (M, K))
    a.bytes(ws, "ws")
    ev = _events(events)
    st = _lib.tw_ffn_fwd(_ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), M, K, N, _ptr(y), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream(stream), ev[0] if ev else None)
    _check(st, "tw_ffn_fwd")


def tw_gate_dense(x, wg_t, z, stream=None, events=None) -> None:
    M, K = _dims2(x, "x", "tw_gate_dense")
    N = _dims2(wg_t, "wg_t", "tw_gate_dense")[0]
    a = _Args("tw_gate_dense", x)
    a.shape(x, "x", _BF16, (M, K))
    a.shape(wg_t, "wg_t", _BF16, (N, K))
    a.shape(z, "z", _F32, (M, N))
    ev = _events(events)
    st = _lib.tw_gate_dense(_ptr(x), _ptr(wg_t), M, K, N, _ptr(z), _stream(stream),
                            ev[0] if ev else None)
    _check(st, "tw_gate_dense")


def tw_pack_dense_workspace_bytes(M, N) -> int:
    return int(_lib.tw_pack_dense_workspace_bytes(M, N))


def tw_pack_dense(z, T, C, tw_val, tw_idx, tw_cnt, ovf_rows, ovf_count, R_max, ws, stream=None,
                  events=None) -> None:
    M, N = _dims2(z, "z", "tw_pack_dense")
    NT = _tiles(N, T, "tw_pack_dense")
    a = _Args("tw_pack_dense", z)
    a.shape(z, "z", _F32, (M, N))
    a.shape(tw_val, "tw_val", _F32, (M, NT, C))
    a.shape(tw_idx, "tw_idx", _I32, (M, NT, C))
    a.shape(tw_cnt, "tw_cnt", _I32, (M, NT))
    a.room(ovf_rows, "ovf_rows", _I32, max(R_max, 1))
    a.room(ovf_count, "ovf_count", _I32, 1)
    a.bytes(ws, "ws")
    ev = _events(events)
    st = _lib.tw_pack_dense(_ptr(z), M, N, T, C, _ptr(tw_val), _ptr(tw_idx), _ptr(tw_cnt),
                            _ptr(ovf_rows), _ptr(ovf_count), R_max, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream),
                            ev[0] if ev else None)
    _check(st, "tw_pack_dense")


def tw_hybrid_pack(T, C, tw_val, tw_idx, tw_cnt, P, hy_val, hy_idx, hy_cnt, route, bk_rows,
                   bk_count, R_max, stream=None, events=None) -> None:
    M, NT = _dims2(tw_cnt, "tw_cnt", "tw_hybrid_pack")
    a = _Args("tw_hybrid_pack", tw_cnt)
    a.shape(tw_cnt, "tw_cnt", _I32, (M, NT))
    a.shape(tw_val, "tw_val", _F32, (M, NT, C))
    a.shape(tw_idx, "tw_idx", _I32, (M, NT, C))
    a.shape(hy_val, "hy_val", _F32, (M, P))
    a.shape(hy_idx, "hy_idx", _I32, (M, P))
    a.shape(hy_cnt, "hy_cnt", _I32, (M,))
    a.shape(route, "route", _U8T, (M,))
    a.room(bk_rows, "bk_rows", _I32, max(R_max, 1))
    a.room(bk_count, "bk_count", _I32, 1)
    ev = _events(events)
    st = _lib.tw_hybrid_pack(M, NT * T, T, C, _ptr(tw_val), _ptr(tw_idx), _ptr(tw_cnt), P,
                             _ptr(hy_val), _ptr(hy_idx), _ptr(hy_cnt), _ptr(route), _ptr(bk_rows),
                             _ptr(bk_count), R_max, _stream(stream), ev[0] if ev else None)
    _check(st, "tw_hybrid_pack")


def tw_hybrid_up(x, wg_t, wu_t, P, hy_g, hy_idx, hy_cnt, route, bk_rows, bk_count, R_max,
                 hy_u, hy_h, bk_g, bk_u, bk_h, stream=None, events=None) -> None:
    M, K = _dims2(x, "x", "tw_hybrid_up")
    N = _dims2(wg_t, "wg_t", "tw_hybrid_up")[0]
    R1 = max(R_max, 1)
    a = _Args("tw_hybrid_up", x)
    a.shape(x, "x", _BF16, (M, K))
    a.shape(wg_t, "wg_t", _BF16, (N, K))
    a.shape(wu_t, "wu_t", _BF16, (N, K))
    a.shape(hy_g, "hy_g", _F32, (M, P))
    a.shape(hy_idx, "hy_idx", _I32, (M, P))
    a.shape(hy_cnt, "hy_cnt", _I32, (M,))
    a.shape(route, "route", _U8T, (M,))
    a.room(bk_rows, "bk_rows", _I32, R1)
    a.room(bk_count, "bk_count", _I32, 1)
    a.opt(hy_u, "hy_u", _F32, (M, P))
    a.shape(hy_h, "hy_h", _F32, (M, P))
    a.opt(bk_g, "bk_g", _BF16, (R1, N))
    a.opt(bk_u, "bk_u", _BF16, (R1, N))
    a.shape(bk_h, "bk_h", _BF16, (R1, N))
    ev = _events(events)
    st = _lib.tw_hybrid_up(_ptr(x), _ptr(wg_t), _ptr(wu_t), M, K, N, P, _ptr(hy_g), _ptr(hy_idx),
                           _ptr(hy_cnt), _ptr(route), _ptr(bk_rows), _ptr(bk_count), R_max,
                           _ptr(hy_u), _ptr(hy_h), _ptr(bk_g), _ptr(bk_u), _ptr(bk_h),
                           _stream(stream), ev[0] if ev else None)
    _check(st, "tw_hybrid_up")


def tw_hybrid_down_workspace_bytes(R_max) -> int:
    return int(_lib.tw_hybrid_down_workspace_bytes(R_max))


def tw_hybrid_down(wd, M, P, hy_h, hy_idx, hy_cnt, route, bk_rows, bk_count, R_max, bk_h, y,
                   ws, stream=None, events=None) -> None:
    N, K = _dims2(wd, "wd", "tw_hybrid_down")
    R1 = max(R_max, 1)
    a = _Args("tw_hybrid_down", wd)
    a.shape(wd, "wd", _BF16, (N, K))
    a.shape(hy_h, "hy_h", _F32, (M, P))
    a.shape(hy_idx, "hy_idx", _I32, (M, P))
    a.shape(hy_cnt, "hy_cnt", _I32, (M,))
    a.shape(route, "route", _U8T, (M,))
    a.room(bk_rows, "bk_rows", _I32, R1)
    a.room(bk_count, "bk_count", _I32, 1)
    a.shape(bk_h, "bk_h", _BF16, (R1, N))
    a.shape(y, "y", _F32, (M, K))
    a.bytes(ws, "ws")
    ev = _events(events)
    nws = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib.tw_hybrid_down(_ptr(wd), M, K, N, P, _ptr(hy_h), _ptr(hy_idx), _ptr(hy_cnt),
                             _ptr(route), _ptr(bk_rows), _ptr(bk_count), R_max, _ptr(bk_h),
                             _ptr(y), _ptr(ws), nws, _stream(stream), ev[0] if ev else None)
    _check(st, "tw_hybrid_down")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def tw_hybrid_bwd_dh(dy, wd, P, l1, hy_g, hy_u, hy_idx, hy_cnt, route, bk_rows, bk_count, R_max,
                     bk_g, bk_u, hy_du, hy_dz, bk_du, bk_dz, stream=None, events=None) -> None:
    M, K = _dims2(dy, "dy", "tw_hybrid_bwd_dh")
    N = _dims2(wd, "wd", "tw_hybrid_bwd_dh")[0]
    R1 = max(R_max, 1)
    a = _Args("tw_hybrid_bwd_dh", dy)
    a.shape(dy, "dy", _BF16, (M, K))
    a.shape(wd, "wd", _BF16, (N, K))
    for t, n in ((hy_g, "hy_g"), (hy_u, "hy_u"), (hy_du, "hy_du"), (hy_dz, "hy_dz")):
        a.shape(t, n, _F32, (M, P))
    a.shape(hy_idx, "hy_idx", _I32, (M, P))
    a.shape(hy_cnt, "hy_cnt", _I32, (M,))
    a.shape(route, "route", _U8T, (M,))
    a.room(bk_rows, "bk_rows", _I32, R1)
    a.room(bk_count, "bk_count", _I32, 1)
    for t, n in ((bk_g, "bk_g"), (bk_u, "bk_u"), (bk_du, "bk_du"), (bk_dz, "bk_dz")):
        a.shape(t, n, _BF16, (R1, N))
    ev = _events(events)
    st = _lib.tw_hybrid_bwd_dh(_ptr(dy), _ptr(wd), M, K, N, P, float(l1), _ptr(hy_g), _ptr(hy_u),
                               _ptr(hy_idx), _ptr(hy_cnt), _ptr(route), _ptr(bk_rows),
                               _ptr(bk_count), R_max, _ptr(bk_g), _ptr(bk_u), _ptr(hy_du),
                               _ptr(hy_dz), _ptr(bk_du), _ptr(bk_dz), _stream(stream),
                               ev[0] if ev else None)
    _check(st, "tw_hybrid_bwd_dh")


def tw_hybrid_bwd_dx_workspace_bytes(R_max) -> int:
    return int(_lib.tw_hybrid_bwd_dx_workspace_bytes(R_max))


def tw_hybrid_bwd_dx(wg_t, wu_t, M, P, hy_du, hy_dz, hy_idx, hy_cnt, route, bk_rows, bk_count,
                     R_max, bk_du, bk_dz, dx, ws, stream=None, events=None) -> None:
    N, K = _dims2(wg_t, "wg_t", "tw_hybrid_bwd_dx")
    R1 = max(R_max, 1)
    a = _Args("tw_hybrid_bwd_dx", wg_t)
    a.shape(wg_t, "wg_t", _BF16, (N, K))
    a.shape(wu_t, "wu_t", _BF16, (N, K))
    a.shape(hy_du, "hy_du", _F32, (M, P))
    a.shape(hy_dz, "hy_dz", _F32, (M, P))
    a.shape(hy_idx, "hy_idx", _I32, (M, P))
    a.shape(hy_cnt, "hy_cnt", _I32, (M,))
    a.shape(route, "route", _U8T, (M,))
    a.room(bk_rows, "bk_rows", _I32, R1)
    a.room(bk_count, "bk_count", _I32, 1)
    a.shape(bk_du, "bk_du", _BF16, (R1, N))
    a.shape(bk_dz, "bk_dz", _BF16, (R1, N))
    a.shape(dx, "dx", _F32, (M, K))
    a.bytes(ws, "ws")
    ev = _events(events)
    st = _lib.tw_hybrid_bwd_dx(_ptr(wg_t), _ptr(wu_t), M, K, N, P, _ptr(hy_du), _ptr(hy_dz),
                               _ptr(hy_idx), _ptr(hy_cnt), _ptr(route), _ptr(bk_rows),
                               _ptr(bk_count), R_max, _ptr(bk_du), _ptr(bk_dz), _ptr(dx), _ptr(ws),
                               _nbytes(ws), _stream(stream), ev[0] if ev else None)
    _check(st, "tw_hybrid_bwd_dx")


def tw_hybrid_bwd_dw_workspace_bytes(M, K, N, P, R_max) -> int:
    return int(_lib.tw_hybrid_bwd_dw_workspace_bytes(M, K, N, P, R_max))


def tw_hybrid_bwd_dw(x, dy, P, hy_h, hy_du, hy_dz, hy_idx, hy_cnt, route, bk_rows, bk_count,
                     R_max, bk_h, bk_du, bk_dz, dwg_t, dwu_t, dwd, ws, stream=None,
                     events=None) -> None:
    M, K = _dims2(x, "x", "tw_hybrid_bwd_dw")
    N = _dims2(dwd, "dwd", "tw_hybrid_bwd_dw")[0]
    R1 = max(R_max, 1)
    a = _Args("tw_hybrid_bwd_dw", x)
    a.shape(x, "x", _BF16, (M, K))
    a.shape(dy, "dy", _BF16, (M, K))
    for t, n in ((hy_h, "hy_h"), (hy_du, "hy_du"), (hy_dz, "hy_dz")):
        a.shape(t, n, _F32, (M, P))
    a.shape(hy_idx, "hy_idx", _I32, (M, P))
    a.shape(hy_cnt, "hy_cnt", _I32, (M,))
    a.shape(route, "route", _U8T, (M,))
    a.room(bk_rows, "bk_rows", _I32, R1)
    a.room(bk_count, "bk_count", _I32, 1)
    for t, n in ((bk_h, "bk_h"), (bk_du, "bk_du"), (bk_dz, "bk_dz")):
        a.shape(t, n, _BF16, (R1, N))
    for t, n in ((dwg_t, "dwg_t"), (dwu_t, "dwu_t"), (dwd, "dwd")):
        a.shape(t, n, _F32, (N, K))
    a.bytes(ws, "ws")
    ev = _events(events)
    st = _lib.tw_hybrid_bwd_dw(_ptr(x), _ptr(dy), M, K, N, P, _ptr(hy_h), _ptr(hy_du),
                               _ptr(hy_dz), _ptr(hy_idx), _ptr(hy_cnt), _ptr(route),
                               _ptr(bk_rows), _ptr(bk_count), R_max, _ptr(bk_h),
                               _ptr(bk_du), _ptr(bk_dz), _ptr(dwg_t), _ptr(dwu_t), _ptr(dwd),
                               _ptr(ws), _nbytes(ws), _stream(stream), ev[0] if ev else None)
    _check(st, "tw_hybrid_bwd_dw")


# ------------------------------------------------------------- allocating --
def alloc_pack(M, N, T, C, R_max, device="cuda"):
    """Output buffers of tw_pack_gate."""
    NT = N // T
    return {
        "tw_val": torch.empty((M, NT, C), dtype=torch.float32, device=device),
        "tw_idx": torch.empty((M, NT, C), dtype=torch.int32, device=device),
        "tw_cnt": torch.empty((M, NT), dtype=torch.int32, device=device),
        "ovf_rows": torch.empty((max(R_max, 1),), dtype=torch.int32, device=device),
        "ovf_count": torch.empty((1,), dtype=torch.int32, device=device),
    }


def workspace(M, K, N, T, C, R_max, device="cuda"):
    n = tw_workspace_bytes(M, K, N, T, C, R_max)
    if n == 0:
        raise ValueError("unsupported shape for the TwELL path")
    return torch.empty((n,), dtype=torch.uint8, device=device)


def pack_gate(x, wg_t, T, C, R_max=None, z_debug=False, ws=None):
    """Gate GEMM + ReLU + TwELL packing; returns the packing as a dict."""
    M, K = x.shape
    N = wg_t.shape[0]
    R_max = M if R_max is None else R_max
    out = alloc_pack(M, N, T, C, R_max, x.device)
    ws = workspace(M, K, N, T, C, R_max, x.device) if ws is None else ws
    z = torch.empty((M, N), dtype=torch.float32, device=x.device) if z_debug else None
    tw_pack_gate(x, wg_t, T, C, out["tw_val"], out["tw_idx"], out["tw_cnt"], out["ovf_rows"],
                 out["ovf_count"], R_max, ws, z_debug=z)
    if z_debug:
        out["z"] = z
    out.update(T=T, C=C, R_max=R_max)
    return out


def pack_unfused(x, wg_t, T, C, R_max=None):
    """The unfused equivalent of pack_gate: dense gate in memory, then packed."""
    M, K = x.shape
    N = wg_t.shape[0]
    R_max = M if R_max is None else R_max
    out = alloc_pack(M, N, T, C, R_max, x.device)
    z = torch.empty((M, N), dtype=torch.float32, device=x.device)
    ws = torch.empty((tw_pack_dense_workspace_bytes(M, N),), dtype=torch.uint8, device=x.device)
    tw_gate_dense(x, wg_t, z)
    tw_pack_dense(z, T, C, out["tw_val"], out["tw_idx"], out["tw_cnt"], out["ovf_rows"],
                  out["ovf_count"], R_max, ws)
    out.update(T=T, C=C, R_max=R_max, z=z)
    return out


def sparse_ffn(x, wg_t, wu_t, wd, packed, ws=None):
    """Sparse up+down (and dense fallback) from a packing; returns y fp32."""
    M, K = x.shape
    N = wg_t.shape[0]
    T, C, R_max = packed["T"], packed["C"], packed["R_max"]
    y = torch.empty((M, K), dtype=torch.float32, device=x.device)
    ws = workspace(M, K, N, T, C, R_max, x.device) if ws is None else ws
    tw_sparse_ffn_fwd(x, wg_t, wu_t, wd, T, C, packed["tw_val"], packed["tw_idx"],
                      packed["tw_cnt"], packed["ovf_rows"], packed["ovf_count"], R_max, y, ws)
    return y


def ffn(x, wg_t, wu_t, wd, ws=None):
    """Dense gated FFN over all rows; returns y fp32."""
    M, K = x.shape
    N = wg_t.shape[0]
    y = torch.empty((M, K), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty((tw_ffn_workspace_bytes(M, K, N),), dtype=torch.uint8, device=x.device)
    tw_ffn_fwd(x, wg_t, wu_t, wd, y, ws)
    return y


def alloc_hybrid(M, N, P, R_max, keep=True, device="cuda"):
    """Buffers of the hybrid storage (sparse rows, routing, backup rows).
    ``keep`` also allocates the up values and the backup gate and up rows
    (what the backward reads); without it only the product h is stored."""
    R1 = max(R_max, 1)
    f32, i32, b16 = torch.float32, torch.int32, torch.bfloat16
    out = {
        "hy_cnt": torch.empty((M,), dtype=i32, device=device),
        "hy_idx": torch.empty((M, P), dtype=i32, device=device),
        "hy_g": torch.empty((M, P), dtype=f32, device=device),
        "hy_h": torch.empty((M, P), dtype=f32, device=device),
        "route": torch.empty((M,), dtype=torch.uint8, device=device),
        "bk_rows": torch.empty((R1,), dtype=i32, device=device),
        "bk_count": torch.empty((1,), dtype=i32, device=device),
        "bk_h": torch.empty((R1, N), dtype=b16, device=device),
        "hy_u": None, "bk_g": None, "bk_u": None,
    }
    if keep:
        out["hy_u"] = torch.empty((M, P), dtype=f32, device=device)
        out["bk_g"] = torch.empty((R1, N), dtype=b16, device=device)
        out["bk_u"] = torch.empty((R1, N), dtype=b16, device=device)
    out.update(P=P, R_max=R_max)
    return out


def hybrid_forward(x, wg_t, wu_t, wd, packed, P=128, R_max=None, keep=True, hy=None, ws=None):
    """Training forward over hybrid storage, from a TwELL packing of the gate
    (``pack_gate``'s output): TwELL -> hybrid, up at the stored entries, down
    to dense.  Returns (y fp32 [M][K], the hybrid storage dict)."""
    M, K = x.shape
    N = wg_t.shape[0]
    R_max = max(M // 8, 1) if R_max is None else R_max
    R_max = min(R_max, M)
    hy = alloc_hybrid(M, N, P, R_max, keep, x.device) if hy is None else hy
    tw_hybrid_pack(packed["T"], packed["C"], packed["tw_val"], packed["tw_idx"],
                   packed["tw_cnt"], P, hy["hy_g"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                   hy["bk_rows"], hy["bk_count"], R_max)
    tw_hybrid_up(x, wg_t, wu_t, P, hy["hy_g"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                 hy["bk_rows"], hy["bk_count"], R_max, hy["hy_u"], hy["hy_h"], hy["bk_g"],
                 hy["bk_u"], hy["bk_h"])
    y = torch.empty((M, K), dtype=torch.float32, device=x.device)
    nws = tw_hybrid_down_workspace_bytes(R_max)
    if ws is None and nws:
        ws = torch.empty((nws,), dtype=torch.uint8, device=x.device)
    tw_hybrid_down(wd, M, P, hy["hy_h"], hy["hy_idx"], hy["hy_cnt"], hy["route"], hy["bk_rows"],
                   hy["bk_count"], R_max, hy["bk_h"], y, ws)
    return y, hy


def hybrid_backward(x, wg_t, wu_t, wd, dy, hy, l1=0.0):
    """Backward over the hybrid storage ``hy`` of ``hybrid_forward`` (with
    ``keep=True``): returns a dict with dx [M][K], dwg_t, dwu_t, dwd [N][K]
    (fp32) and the activations' gradients (hy_du, hy_dz, bk_du, bk_dz)."""
    M, K = x.shape
    N = wg_t.shape[0]
    P, R_max = hy["P"], hy["R_max"]
    if hy["hy_u"] is None:
        raise ValueError("the forward did not keep u and g (keep=False)")
    dev = x.device
    R1 = max(R_max, 1)
    out = {
        "hy_du": torch.empty((M, P), dtype=torch.float32, device=dev),
        "hy_dz": torch.empty((M, P), dtype=torch.float32, device=dev),
        "bk_du": torch.empty((R1, N), dtype=torch.bfloat16, device=dev),
        "bk_dz": torch.empty((R1, N), dtype=torch.bfloat16, device=dev),
        "dx": torch.empty((M, K), dtype=torch.float32, device=dev),
        "dwg_t": torch.empty((N, K), dtype=torch.float32, device=dev),
        "dwu_t": torch.empty((N, K), dtype=torch.float32, device=dev),
        "dwd": torch.empty((N, K), dtype=torch.float32, device=dev),
    }
    tw_hybrid_bwd_dh(dy, wd, P, l1, hy["hy_g"], hy["hy_u"], hy["hy_idx"], hy["hy_cnt"],
                     hy["route"], hy["bk_rows"], hy["bk_count"], R_max, hy["bk_g"], hy["bk_u"],
                     out["hy_du"], out["hy_dz"], out["bk_du"], out["bk_dz"])
    nx = tw_hybrid_bwd_dx_workspace_bytes(R_max)
    wsx = torch.empty((nx,), dtype=torch.uint8, device=dev) if nx else None
    tw_hybrid_bwd_dx(wg_t, wu_t, M, P, out["hy_du"], out["hy_dz"], hy["hy_idx"], hy["hy_cnt"],
                     hy["route"], hy["bk_rows"], hy["bk_count"], R_max, out["bk_du"],
                     out["bk_dz"], out["dx"], wsx)
    wsw = torch.empty((tw_hybrid_bwd_dw_workspace_bytes(M, K, N, P, R_max),), dtype=torch.uint8,
                      device=dev)
    tw_hybrid_bwd_dw(x, dy, P, hy["hy_h"], out["hy_du"], out["hy_dz"], hy["hy_idx"],
                     hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"], R_max,
                     hy["bk_h"], out["bk_du"], out["bk_dz"], out["dwg_t"], out["dwu_t"],
                     out["dwd"], wsw)
    return out


def library_path() -> str:
    return LIBRARY
