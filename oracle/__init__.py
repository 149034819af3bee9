"""Plain FP64 CPU oracle for RMSNorm training -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The library under
``rmsnorm_train_fwd_amd`` never imports it and shares no code with it.

This module only marshals numpy arrays to the C oracle in ``rmsn_oracle.c``;
all arithmetic of the method lives there (see that file's header for the
definitions and the passages of the pages they follow).

Inputs are BF16 bit patterns (numpy uint16) in the layouts the library takes:
element (t, h, j) at ``buf[t*st + h*sh + j]``; rows are numbered r = t*heads + h.
The weight is passed as float64, converted exactly from its BF16 or FP32
storage (``w_to_f64``).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

_lib = None


class _View(C.Structure):
    _fields_ = [
        ("p", C.c_void_p),
        ("T", C.c_int64),
        ("heads", C.c_int64),
        ("width", C.c_int64),
        ("st", C.c_int64),
        ("sh", C.c_int64),
    ]


def lib():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        L = C.CDLL(path)
        dp = C.POINTER(C.c_double)
        vp = C.POINTER(_View)
        i64p = C.POINTER(C.c_int64)
        u16p = C.POINTER(C.c_uint16)
        L.orc_bf16_to_f64.restype = C.c_double
        L.orc_bf16_to_f64.argtypes = [C.c_uint16]
        L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_f64_to_bf16.argtypes = [C.c_double]
        L.orc_bf16_to_f64_array.argtypes = [u16p, C.c_int64, dp]
        L.orc_f64_to_bf16_array.argtypes = [dp, C.c_int64, u16p]
        L.orc_zero_centred_weight.argtypes = [C.c_int64, dp, dp]
        L.orc_rmsnorm_fwd_f64.argtypes = [C.c_int64, C.c_int64, dp, dp, C.c_double, dp, dp]
        L.orc_rmsnorm_bwd_f64.argtypes = [C.c_int64, C.c_int64, dp, dp, dp, C.c_double, dp, dp]
        L.orc_gate_fwd_f64.argtypes = [C.c_int64, C.c_int64, dp, dp, dp, C.c_double, dp, dp]
        L.orc_gate_bwd_f64.argtypes = [C.c_int64, C.c_int64, dp, dp, dp, dp, C.c_double, dp, dp, dp]
        for name, args in [
            ("orc_fwd_bf16", [vp, dp, C.c_double, i64p, C.c_int64, dp, dp]),
            ("orc_res_fwd_bf16", [vp, vp, dp, C.c_double, i64p, C.c_int64, u16p, dp, dp]),
            ("orc_bwd_bf16", [vp, vp, vp, dp, C.c_double, i64p, C.c_int64, dp, dp]),
            ("orc_gate_fwd_bf16", [vp, vp, dp, C.c_double, i64p, C.c_int64, dp, dp]),
            ("orc_gate_bwd_bf16", [vp, vp, vp, dp, C.c_double, i64p, C.c_int64, dp, dp, dp]),
        ]:
            f = getattr(L, name)
            f.restype = C.c_int
            f.argtypes = args
        _lib = L
    return _lib


def _dp(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ---- number formats ---------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_to_f64_array(b.ctypes.data_as(C.POINTER(C.c_uint16)), b.size, _dp(out))
    return out


def f64_to_bf16(a) -> np.ndarray:
    a = _f64(a)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f64_to_bf16_array(_dp(a), a.size, out.ctypes.data_as(C.POINTER(C.c_uint16)))
    return out


def zero_centred_weight(w) -> np.ndarray:
    """Effective weight 1 + w of the zero-centred form (float64)."""
    w = _f64(w)
    out = np.empty_like(w)
    lib().orc_zero_centred_weight(w.size, _dp(w), _dp(out))
    return out


def w_to_f64(w: np.ndarray) -> np.ndarray:
    """Exact conversion of a weight stored as BF16 bits (uint16) or float32."""
    if w.dtype == np.uint16:
        return bf16_to_f64(w)
    if w.dtype == np.float32:
        return w.astype(np.float64)
    raise TypeError(f"weight dtype {w.dtype}")


# ---- dense FP64 rows -------------------------------------------------------

def rmsnorm_fwd_f64(x, w, eps):
    x, w = _f64(x), _f64(w)
    rows, n = x.shape
    y = np.empty_like(x)
    r = np.empty(rows, np.float64)
    lib().orc_rmsnorm_fwd_f64(rows, n, _dp(x), _dp(w), eps, _dp(y), _dp(r))
    return y, r


def rmsnorm_bwd_f64(dy, x, w, eps):
    dy, x, w = _f64(dy), _f64(x), _f64(w)
    rows, n = x.shape
    dx = np.empty_like(x)
    dw = np.empty(n, np.float64)
    lib().orc_rmsnorm_bwd_f64(rows, n, _dp(dy), _dp(x), _dp(w), eps, _dp(dx), _dp(dw))
    return dx, dw


def gate_fwd_f64(x, z, w, eps):
    x, z, w = _f64(x), _f64(z), _f64(w)
    rows, n = x.shape
    y = np.empty_like(x)
    r = np.empty(rows, np.float64)
    lib().orc_gate_fwd_f64(rows, n, _dp(x), _dp(z), _dp(w), eps, _dp(y), _dp(r))
    return y, r


def gate_bwd_f64(dy, x, z, w, eps):
    dy, x, z, w = _f64(dy), _f64(x), _f64(z), _f64(w)
    rows, n = x.shape
    dx = np.empty_like(x)
    dz = np.empty_like(x)
    dw = np.empty(n, np.float64)
    lib().orc_gate_bwd_f64(rows, n, _dp(dy), _dp(x), _dp(z), _dp(w), eps, _dp(dx), _dp(dz), _dp(dw))
    return dx, dz, dw


# ---- BF16 views --------------------------------------------------------------

@dataclass
class View:
    """BF16 bits ``buf`` (any shape, C-contiguous uint16) seen as [T, heads, width]."""

    buf: np.ndarray
    T: int
    heads: int
    width: int
    st: int
    sh: int

    @staticmethod
    def dense(a: np.ndarray, heads: int = 1) -> "View":
        a = np.ascontiguousarray(a, dtype=np.uint16)
        width = a.shape[-1]
        T = a.size // (width * heads)
        return View(a, T, heads, width, heads * width, width)

    @property
    def rows(self) -> int:
        return self.T * self.heads

    def c(self) -> _View:
        assert self.buf.dtype == np.uint16 and self.buf.flags["C_CONTIGUOUS"]
        if self.rows > 0:
            last = (self.T - 1) * self.st + (self.heads - 1) * self.sh + self.width
            assert last <= self.buf.size, "view runs past its buffer"
        return _View(self.buf.ctypes.data, self.T, self.heads, self.width, self.st, self.sh)


def _sel(sel, rows):
    if sel is None:
        return None, rows
    s = np.ascontiguousarray(sel, dtype=np.int64)
    return s, s.size


def _selp(s):
    return None if s is None else s.ctypes.data_as(C.POINTER(C.c_int64))


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name}: bad arguments")


def fwd(x: View, w, eps, sel=None):
    """Returns y [nsel, width] and rstd [nsel], float64."""
    w = _f64(w)
    s, n = _sel(sel, x.rows)
    y = np.empty((n, x.width), np.float64)
    r = np.empty(n, np.float64)
    xv = x.c()
    _check(lib().orc_fwd_bf16(C.byref(xv), _dp(w), eps, _selp(s), n, _dp(y), _dp(r)), "fwd")
    return y, r


def res_fwd(x: View, res: View, w, eps, sel=None):
    """Returns h [rows, width] BF16 bits, y [nsel, width], rstd [nsel]."""
    w = _f64(w)
    s, n = _sel(sel, x.rows)
    h = np.empty((x.rows, x.width), np.uint16)
    y = np.empty((n, x.width), np.float64)
    r = np.empty(n, np.float64)
    xv, rv = x.c(), res.c()
    _check(lib().orc_res_fwd_bf16(C.byref(xv), C.byref(rv), _dp(w), eps, _selp(s), n,
                                  h.ctypes.data_as(C.POINTER(C.c_uint16)), _dp(y), _dp(r)),
           "res_fwd")
    return h, y, r


def bwd(dy: View, x: View, w, eps, dh: Optional[View] = None, sel=None, want_rows=True,
        want_dw=True):
    """Returns (dx or grad_h) [nsel, width] and dw [width] (sum over all rows)."""
    w = _f64(w)
    s, n = _sel(sel, x.rows)
    out = np.empty((n, x.width), np.float64) if want_rows else None
    dw = np.empty(x.width, np.float64) if want_dw else None
    dyv, xv = dy.c(), x.c()
    dhv = dh.c() if dh is not None else None
    _check(lib().orc_bwd_bf16(C.byref(dyv), C.byref(xv), C.byref(dhv) if dhv else None,
                              _dp(w), eps, _selp(s), n, _dp(out), _dp(dw)), "bwd")
    return out, dw


def gate_fwd(x: View, z: View, w, eps, sel=None):
    w = _f64(w)
    s, n = _sel(sel, x.rows)
    y = np.empty((n, x.width), np.float64)
    r = np.empty(n, np.float64)
    xv, zv = x.c(), z.c()
    _check(lib().orc_gate_fwd_bf16(C.byref(xv), C.byref(zv), _dp(w), eps, _selp(s), n,
                                   _dp(y), _dp(r)), "gate_fwd")
    return y, r


def gate_bwd(dy: View, x: View, z: View, w, eps, sel=None, want_rows=True, want_dw=True):
    """Returns dx, dz [nsel, width] and dw [width]."""
    w = _f64(w)
    s, n = _sel(sel, x.rows)
    dx = np.empty((n, x.width), np.float64) if want_rows else None
    dz = np.empty((n, x.width), np.float64) if want_rows else None
    dw = np.empty(x.width, np.float64) if want_dw else None
    dyv, xv, zv = dy.c(), x.c(), z.c()
    _check(lib().orc_gate_bwd_bf16(C.byref(dyv), C.byref(xv), C.byref(zv), _dp(w), eps,
                                   _selp(s), n, _dp(dx), _dp(dz), _dp(dw)), "gate_bwd")
    return dx, dz, dw
