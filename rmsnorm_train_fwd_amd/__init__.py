"""RMSNorm for training on MI355X (gfx950): Python binding of librmsnorm_train.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/rmsnorm_train.h. PyTorch supplies
device memory and the current HIP stream. There is no fallback: if the library
is not built, or a tensor is not on a ROCm device, the call raises.

Names follow the C ABI:
  rmsnorm_train_fwd(x, w, eps, residual=None)        -> y, rstd[, h]
  rmsnorm_train_bwd(dy, x, rstd, w, deterministic, dh=None) -> dx | grad_h, dw
  rmsnorm_train_bwd_query(shape..., deterministic)   -> plan (host only)
  rmsnorm_silu_gate_train_fwd(x, z, w, eps)          -> y, rstd
  rmsnorm_silu_gate_train_bwd(dy, x, z, rstd, w, deterministic) -> dx, dz, dw
  rmsnorm_train_bwd_noalloc(dy, x, rstd, w, deterministic, dh=None) -> dx | grad_h, dw
    (the library's workspace-free backward; this binding still allocates the outputs)
Row tensors are BF16 [T, H] (one row per token) or [T, heads, width] views
whose last dimension is contiguous; w is [width] BF16 or FP32.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm_train.so")

RMSN_BF16, RMSN_F32, RMSN_BF16_ZERO_CENTRED, RMSN_F32_ZERO_CENTRED = 0, 1, 2, 3
PATH_AUTO, PATH_SMALL, PATH_LARGE = 0, 1, 2
STATUS = {
    0: "RMSN_OK", 1: "RMSN_E_NULL", 2: "RMSN_E_DTYPE", 3: "RMSN_E_SHAPE", 4: "RMSN_E_STRIDE",
    5: "RMSN_E_ALIGN", 6: "RMSN_E_ALIAS", 7: "RMSN_E_WORKSPACE", 8: "RMSN_E_LAUNCH",
    9: "RMSN_E_ARG", 10: "RMSN_E_HIP",
}
EXPORTS = (
    "rmsnorm_train_fwd", "rmsnorm_train_bwd", "rmsnorm_train_bwd_query",
    "rmsnorm_silu_gate_train_fwd", "rmsnorm_silu_gate_train_bwd", "rmsnorm_train_bwd_noalloc",
    "rmsn_status_str",
)


class Layout(C.Structure):
    _fields_ = [(n, C.c_int64) for n in
                ("T", "heads", "width", "x_stride_t", "x_stride_h", "g_stride_t", "g_stride_h")]


class Launch(C.Structure):
    _fields_ = [("grid", C.c_int32), ("fold_grid", C.c_int32), ("path", C.c_int32)]


class BwdPlan(C.Structure):
    _fields_ = [
        ("path", C.c_int32), ("rows", C.c_int64),
        ("chunks", C.c_int64), ("subchains", C.c_int32), ("fold_group", C.c_int32),
        ("grid", C.c_int32), ("fold_grid", C.c_int32), ("workspace_bytes", C.c_size_t),
    ]


class RmsnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.status = STATUS.get(code, str(code))
        super().__init__(f"{where}: {self.status} ({lib().rmsn_status_str(code).decode()})")


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m rmsnorm_train_fwd_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, lp, lap, fp = C.c_void_p, C.POINTER(Layout), C.POINTER(Launch), C.c_float
        L.rmsnorm_train_fwd.argtypes = [vp, vp, vp, C.c_int, fp, lp, vp, vp, vp, vp]
        L.rmsnorm_train_bwd.argtypes = [vp, vp, vp, vp, C.c_int, vp, C.c_int, lp, vp, vp, C.c_int,
                                        vp, C.c_size_t, lap, vp]
        L.rmsnorm_train_bwd_query.argtypes = [lp, C.c_int, lap, C.POINTER(BwdPlan)]
        L.rmsnorm_silu_gate_train_fwd.argtypes = [vp, vp, vp, C.c_int, fp, lp, vp, vp, vp]
        L.rmsnorm_silu_gate_train_bwd.argtypes = [vp, vp, vp, vp, C.c_int, vp, C.c_int, lp, vp,
                                                  vp, vp, C.c_int, vp, C.c_size_t, lap, vp]
        L.rmsnorm_train_bwd_noalloc.argtypes = [vp, vp, vp, vp, C.c_int, vp, C.c_int, lp, vp, vp,
                                                C.c_int, lap, vp]
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = C.c_int
        L.rmsn_status_str.argtypes = [C.c_int]
        L.rmsn_status_str.restype = C.c_char_p
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != 0:
        raise RmsnError(code, where)


# --------------------------------------------------------------- marshalling --

def _geometry(t: torch.Tensor, name: str):
    """(T, heads, width, stride_t, stride_h) of a [T, H] or [T, heads, width] tensor."""
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() == 2:
        T, W = t.shape
        return (T, 1, W, t.stride(0) if T > 1 else W, W)
    if t.dim() == 3:
        T, H, W = t.shape
        return (T, H, W, t.stride(0) if T > 1 else H * W, t.stride(1) if H > 1 else W)
    raise ValueError(f"{name} must be 2-D [T, H] or 3-D [T, heads, width]")


def _inner_contiguous(t: torch.Tensor, name: str):
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")


def _device(t: torch.Tensor, name: str):
    if t.device.type != "cuda":
        raise RuntimeError(f"{name} must be on a ROCm GPU device (no CPU path exists)")


def _on_device(x: torch.Tensor, **tensors):
    """Every given tensor (None allowed) must sit on x's GPU: the kernels
    dereference all of them on that device."""
    _device(x, "x")
    for name, t in tensors.items():
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}: all tensors of a call "
                             "must be on the same GPU")


def _layout(x: torch.Tensor, g: Optional[torch.Tensor]) -> Layout:
    gx = _geometry(x, "x")
    gg = _geometry(g, "dy") if g is not None else gx
    if gx[:3] != gg[:3]:
        raise ValueError(f"shape mismatch: {tuple(x.shape)} vs {tuple(g.shape)}")
    return Layout(gx[0], gx[1], gx[2], gx[3], gx[4], gg[3], gg[4])


def _same_geometry(a: torch.Tensor, b: torch.Tensor, an: str, bn: str):
    """b must be laid out like a: same shape, same token and head strides, and a
    contiguous last dimension (the kernels read each row as 16-byte vectors)."""
    _inner_contiguous(b, bn)
    if _geometry(a, an) != _geometry(b, bn):
        raise ValueError(f"{bn} must have the shape and strides of {an}")


def _w(w: torch.Tensor, width: int, zero_centred: bool = False):
    """ABI weight code: storage dtype, plain or zero-centred (used as 1 + w)."""
    if w.dim() != 1 or w.shape[0] != width or not w.is_contiguous():
        raise ValueError(f"w must be a contiguous [{width}] vector")
    if w.dtype == torch.bfloat16:
        return RMSN_BF16_ZERO_CENTRED if zero_centred else RMSN_BF16
    if w.dtype == torch.float32:
        return RMSN_F32_ZERO_CENTRED if zero_centred else RMSN_F32
    raise TypeError(f"w must be bfloat16 or float32, got {w.dtype}")


def _rstd(rstd: torch.Tensor, L: Layout):
    if rstd.dtype != torch.float32 or rstd.numel() != L.T * L.heads or not rstd.is_contiguous():
        raise ValueError("rstd must be a contiguous float32 tensor with one value per row")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr() or None


def _launch(grid=0, fold_grid=0, path=PATH_AUTO) -> Launch:
    return Launch(grid, fold_grid, path)


def _rows_shape(x: torch.Tensor):
    return tuple(x.shape), tuple(x.shape[:-1])


# -------------------------------------------------------------------- calls --

def rmsnorm_train_fwd(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                      residual: Optional[torch.Tensor] = None, zero_centred: bool = False):
    """y = RMSNorm(x) * w (BF16) and rstd (FP32). With a residual: h = x + residual
    (BF16) is normalised and returned as well: (y, rstd, h). zero_centred: the
    stored w is centred on zero and used as 1 + w."""
    _inner_contiguous(x, "x")
    L = _layout(x, None)
    wd = _w(w, L.width, zero_centred)
    if residual is not None:
        _same_geometry(x, residual, "x", "residual")
    _on_device(x, w=w, residual=residual)
    full, rows = _rows_shape(x)
    y = torch.empty(full, dtype=torch.bfloat16, device=x.device)
    rstd = torch.empty(rows, dtype=torch.float32, device=x.device)
    h = torch.empty(full, dtype=torch.bfloat16, device=x.device) if residual is not None else None
    with torch.cuda.device(x.device):
        _check(lib().rmsnorm_train_fwd(_ptr(x), _ptr(residual), _ptr(w), wd, float(eps),
                                       C.byref(L), _ptr(y), _ptr(h), _ptr(rstd), _stream(x)),
               "rmsnorm_train_fwd")
    return (y, rstd) if h is None else (y, rstd, h)


def rmsnorm_train_bwd_query(x: torch.Tensor, deterministic: bool = True,
                            launch: Optional[Launch] = None, dy: Optional[torch.Tensor] = None):
    L = _layout(x, dy)
    plan = BwdPlan()
    _check(lib().rmsnorm_train_bwd_query(C.byref(L), int(bool(deterministic)),
                                         C.byref(launch) if launch else None, C.byref(plan)),
           "rmsnorm_train_bwd_query")
    return plan


def _workspace(plan: BwdPlan, x: torch.Tensor, workspace: Optional[torch.Tensor]):
    if plan.workspace_bytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=x.device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace, workspace.numel() * workspace.element_size()


def _dw(width: int, dtype: torch.dtype, device):
    """The dw output tensor and its ABI dtype code."""
    if dtype == torch.float32:
        return torch.empty(width, dtype=torch.float32, device=device), RMSN_F32
    if dtype == torch.bfloat16:
        return torch.empty(width, dtype=torch.bfloat16, device=device), RMSN_BF16
    raise ValueError("dw_dtype must be torch.float32 or torch.bfloat16")


def rmsnorm_train_bwd(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor, w: torch.Tensor,
                      deterministic: bool = True, dh: Optional[torch.Tensor] = None,
                      launch: Optional[Launch] = None, workspace: Optional[torch.Tensor] = None,
                      dw_dtype: torch.dtype = torch.float32, zero_centred: bool = False):
    """dx (BF16) and dw (FP32, or BF16 with dw_dtype=torch.bfloat16). With dh
    (residual form; x is then the forward's BF16 h): grad_h = dh + dx replaces dx.
    zero_centred: w is used as 1 + w (dw is the gradient of the stored w)."""
    _inner_contiguous(x, "x")
    _inner_contiguous(dy, "dy")
    L = _layout(x, dy)
    wd = _w(w, L.width, zero_centred)
    if dh is not None:
        _same_geometry(dy, dh, "dy", "dh")
    _rstd(rstd, L)
    _on_device(x, dy=dy, rstd=rstd, w=w, dh=dh, workspace=workspace)
    plan = rmsnorm_train_bwd_query(x, deterministic, launch, dy)
    ws, ws_bytes = _workspace(plan, x, workspace)
    full, _ = _rows_shape(x)
    dx = torch.empty(full, dtype=torch.bfloat16, device=x.device)
    dw, dwd = _dw(L.width, dw_dtype, x.device)
    with torch.cuda.device(x.device):
        _check(lib().rmsnorm_train_bwd(_ptr(dy), _ptr(x), _ptr(dh), _ptr(w), wd, _ptr(rstd),
                                       int(bool(deterministic)), C.byref(L), _ptr(dx), _ptr(dw),
                                       dwd, _ptr(ws), ws_bytes,
                                       C.byref(launch) if launch else None, _stream(x)),
               "rmsnorm_train_bwd")
    return dx, dw


def rmsnorm_silu_gate_train_fwd(x: torch.Tensor, z: torch.Tensor, w: torch.Tensor,
                                eps: float = 1e-6, zero_centred: bool = False):
    """y = RMSNorm(x) * w * silu(z) (BF16) and rstd (FP32); zero_centred: w used as 1 + w."""
    _inner_contiguous(x, "x")
    _same_geometry(x, z, "x", "z")
    L = _layout(x, None)
    wd = _w(w, L.width, zero_centred)
    _on_device(x, z=z, w=w)
    full, rows = _rows_shape(x)
    y = torch.empty(full, dtype=torch.bfloat16, device=x.device)
    rstd = torch.empty(rows, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().rmsnorm_silu_gate_train_fwd(_ptr(x), _ptr(z), _ptr(w), wd, float(eps),
                                                 C.byref(L), _ptr(y), _ptr(rstd), _stream(x)),
               "rmsnorm_silu_gate_train_fwd")
    return y, rstd


def rmsnorm_silu_gate_train_bwd(dy: torch.Tensor, x: torch.Tensor, z: torch.Tensor,
                                rstd: torch.Tensor, w: torch.Tensor, deterministic: bool = True,
                                launch: Optional[Launch] = None,
                                workspace: Optional[torch.Tensor] = None,
                                dw_dtype: torch.dtype = torch.float32,
                                zero_centred: bool = False):
    """dx, dz (BF16) and dw (FP32, or BF16 with dw_dtype=torch.bfloat16) of the
    SiLU-gated form; zero_centred: w used as 1 + w."""
    _inner_contiguous(x, "x")
    _inner_contiguous(dy, "dy")
    _same_geometry(x, z, "x", "z")
    L = _layout(x, dy)
    wd = _w(w, L.width, zero_centred)
    _rstd(rstd, L)
    _on_device(x, dy=dy, z=z, rstd=rstd, w=w, workspace=workspace)
    plan = rmsnorm_train_bwd_query(x, deterministic, launch, dy)
    ws, ws_bytes = _workspace(plan, x, workspace)
    full, _ = _rows_shape(x)
    dx = torch.empty(full, dtype=torch.bfloat16, device=x.device)
    dz = torch.empty(full, dtype=torch.bfloat16, device=x.device)
    dw, dwd = _dw(L.width, dw_dtype, x.device)
    with torch.cuda.device(x.device):
        _check(lib().rmsnorm_silu_gate_train_bwd(_ptr(dy), _ptr(x), _ptr(z), _ptr(w), wd,
                                                 _ptr(rstd), int(bool(deterministic)), C.byref(L),
                                                 _ptr(dx), _ptr(dz), _ptr(dw), dwd, _ptr(ws),
                                                 ws_bytes, C.byref(launch) if launch else None,
                                                 _stream(x)),
               "rmsnorm_silu_gate_train_bwd")
    return dx, dz, dw


def rmsnorm_train_bwd_noalloc(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor,
                              w: torch.Tensor, deterministic: bool = True,
                              dh: Optional[torch.Tensor] = None, launch: Optional[Launch] = None,
                              dw_dtype: torch.dtype = torch.float32, zero_centred: bool = False):
    """rmsnorm_train_bwd through the library's workspace-free entry point (its
    workspace is a device array inside the library, shared by every call on a
    GPU: calls that can overlap in time on one GPU race). Same results, bit for
    bit. Only the outputs are allocated here."""
    _inner_contiguous(x, "x")
    _inner_contiguous(dy, "dy")
    L = _layout(x, dy)
    wd = _w(w, L.width, zero_centred)
    if dh is not None:
        _same_geometry(dy, dh, "dy", "dh")
    _rstd(rstd, L)
    _on_device(x, dy=dy, rstd=rstd, w=w, dh=dh)
    full, _ = _rows_shape(x)
    dx = torch.empty(full, dtype=torch.bfloat16, device=x.device)
    dw, dwd = _dw(L.width, dw_dtype, x.device)
    with torch.cuda.device(x.device):
        _check(lib().rmsnorm_train_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(dh), _ptr(w), wd,
                                               _ptr(rstd), int(bool(deterministic)), C.byref(L),
                                               _ptr(dx), _ptr(dw), dwd,
                                               C.byref(launch) if launch else None, _stream(x)),
               "rmsnorm_train_bwd_noalloc")
    return dx, dw
