"""Shared test utilities: move seeded problems to the GPU, call the library,
compare with the oracle under the pages' tolerances.

Tolerances (PR #8626 merge text, "Baselines and measurement"; PR #8848 page,
"Measurement"): dx atol = rtol = 1e-2; dw per element atol 1e-4 + rtol 1e-4
against FP64. Readings of this project: y atol = rtol = 1e-2 and at most 1
BF16 ulp from the oracle's rounded value; rstd rtol 1e-5; h bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import rmsnorm_train_fwd_amd as R
import synth

TOL_DX = (1e-2, 1e-2)
TOL_DW = (1e-4, 1e-4)
TOL_Y = (1e-2, 1e-2)
RTOL_RSTD = 1e-5


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor (any device) -> numpy uint16 bit patterns (contiguous copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def oview(p: synth.Problem, buf: torch.Tensor) -> oracle.View:
    return oracle.View(bits(buf), p.T, p.heads, p.width, p.row_stride, p.head_stride)


def gview(p: synth.Problem, buf_gpu: torch.Tensor) -> torch.Tensor:
    """The GPU tensor view the library receives: [T, H] for heads == 1, else [T, heads, W]."""
    if p.heads == 1:
        return buf_gpu.as_strided((p.T, p.width), (p.row_stride, 1))
    return buf_gpu.as_strided((p.T, p.heads, p.width), (p.row_stride, p.head_stride, 1))


def ratio(got, ref, atol, rtol) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    tol = atol + rtol * np.abs(ref)
    bad = ~np.isfinite(got)
    if bad.any():
        return float("inf")
    return float(np.max(err / tol))


def assert_within(got, ref, tol, what):
    r = ratio(got, ref, *tol)
    assert r <= 1.0, f"{what}: worst error is {r:.3g}x the tolerance {tol}"
    return r


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def key(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))


def sample_rows(rows: int, n: int = 48, seed: int = 0, extra=()) -> np.ndarray:
    """All rows if few; otherwise both ends, given extras and a random sample."""
    if rows <= 4 * n:
        return np.arange(rows, dtype=np.int64)
    rng = np.random.default_rng(seed)
    s = set(range(4)) | set(range(rows - 4, rows)) | {r for r in extra if 0 <= r < rows}
    s |= set(rng.choice(rows, n, replace=False).tolist())
    return np.array(sorted(s), dtype=np.int64)


def w_f64(w: torch.Tensor) -> np.ndarray:
    if w.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(bits(w))
    return w.double().numpy()


class OnGpu:
    """A synth.Problem with its buffers copied to the GPU."""

    def __init__(self, p: synth.Problem, device="cuda"):
        self.p = p
        self.w = p.w.to(device)
        self.xb = p.x.to(device)
        self.dyb = p.dy.to(device)
        self.eb = p.extra.to(device) if p.extra is not None else None
        self.dhb = p.dh.to(device) if p.dh is not None else None

    @property
    def x(self):
        return gview(self.p, self.xb)

    @property
    def dy(self):
        return gview(self.p, self.dyb)

    @property
    def e(self):
        return gview(self.p, self.eb)

    @property
    def dh(self):
        return gview(self.p, self.dhb)


def dense_rows(t: torch.Tensor, width: int) -> torch.Tensor:
    return t.reshape(-1, width)
