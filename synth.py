"""Seeded synthetic inputs for RMSNorm training (no arithmetic of the method).

The pages measure on synthetic tensors only (no dataset): x, dy, dh, residual
and z are standard-normal values stored as BF16, w = 1 + 0.1 N(0, 1) stored as
FP32 or BF16, eps = 1e-6 (PR #8626 merge text, "Baselines and measurement" and
"Key"; PR #8848 page, "Measurement"). The accuracy campaign there names "three
input families" without defining them; the three families here are this
project's own:

  F1  "normal":   every tensor ~ N(0, 1).
  F2  "cancel":   rows come in pairs (x, dy) and (x, -dy) placed half the
                  tensor apart, plus a small tail of ordinary rows, so that dw
                  is small while running column sums are large (the
                  cancellation pattern a review on the PR #8848 page raises).
  F3  "spread":   each row of x is scaled by 2^k, k uniform in [-8, 8], so the
                  per-row scale spans 2^16.

Every tensor is produced on the CPU by torch's seeded generator and cast to
BF16 by torch (round to nearest even); the same host tensors feed the oracle
and, after a copy, the GPU.

Both the tests and ``bench.py`` draw from this module; the oracle and the HIP
library never import each other.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

EPS = 1e-6
FAMILIES = ("normal", "cancel", "spread")


def _gen(seed: int, salt: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed) * 1000003 + salt)


def normal_bf16(shape, seed: int, salt: int, scale: float = 1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(seed, salt), dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch.bfloat16)


def weight(width: int, seed: int, w_dtype: str = "f32", centre: float = 1.0) -> torch.Tensor:
    """w = centre + 0.1 N(0,1), FP32, or cast once to BF16 (centre 1 for the
    plain weight, 0 for a zero-centred one)."""
    w = torch.randn(width, generator=_gen(seed, 7), dtype=torch.float32).mul_(0.1).add_(centre)
    if w_dtype == "bf16":
        return w.to(torch.bfloat16)
    if w_dtype == "f32":
        return w
    raise ValueError(w_dtype)


def row_buffer(T: int, heads: int, width: int, seed: int, salt: int, family: str = "normal",
               row_stride: Optional[int] = None, head_stride: Optional[int] = None,
               role: str = "x") -> torch.Tensor:
    """A BF16 buffer whose view (T, heads, width) with strides (row_stride,
    head_stride, 1) holds the rows; padding elements are also random.

    Returns the flat buffer; the view is buffer.as_strided((T, heads, width),
    (row_stride, head_stride, 1)).
    """
    hs = width if head_stride is None else head_stride
    rs = heads * hs if row_stride is None else row_stride
    n = max(T * rs, 1)
    buf = normal_bf16((n,), seed, salt)
    if T == 0:
        return buf
    view = buf.as_strided((T, heads, width), (rs, hs, 1))
    if family == "spread" and role == "x":
        k = torch.randint(-8, 9, (T, heads, 1), generator=_gen(seed, salt + 101))
        view.copy_((view.float() * torch.pow(2.0, k.float())).to(torch.bfloat16))
    elif family == "cancel":
        rows = T * heads
        tail = min(rows, max(1, rows // 64))
        pairs = (rows - tail) // 2
        if pairs > 0:
            src = torch.arange(pairs)
            dst = src + pairs
            rows_src = view[src // heads, src % heads]
            if role == "dy":
                rows_src = rows_src * 16          # power of two: exact in BF16
                view[src // heads, src % heads] = rows_src
                view[dst // heads, dst % heads] = -rows_src
            else:
                view[dst // heads, dst % heads] = rows_src
    return buf


def view_of(buf: torch.Tensor, T: int, heads: int, width: int,
            row_stride: Optional[int] = None, head_stride: Optional[int] = None) -> torch.Tensor:
    hs = width if head_stride is None else head_stride
    rs = heads * hs if row_stride is None else row_stride
    return buf.as_strided((T, heads, width), (rs, hs, 1))


@dataclass
class Problem:
    """One workload: BF16 row tensors as flat buffers + the view geometry."""

    T: int
    heads: int
    width: int
    row_stride: int
    head_stride: int
    w: torch.Tensor
    x: torch.Tensor
    dy: torch.Tensor
    extra: Optional[torch.Tensor] = None   # residual (fwd) or z (gate)
    dh: Optional[torch.Tensor] = None      # gradient of h (residual bwd)
    eps: float = EPS

    def view(self, buf: torch.Tensor) -> torch.Tensor:
        return view_of(buf, self.T, self.heads, self.width, self.row_stride, self.head_stride)

    @property
    def rows(self) -> int:
        return self.T * self.heads


def make(T: int, width: int, seed: int = 0, heads: int = 1, w_dtype: str = "f32",
         family: str = "normal", form: str = "plain", row_stride: Optional[int] = None,
         head_stride: Optional[int] = None, w_centre: float = 1.0) -> Problem:
    """form: 'plain', 'residual' (extra = residual, dh given) or 'gate' (extra = z).
    w_centre: the weight's centre (1, or 0 for the zero-centred-weight form)."""
    hs = width if head_stride is None else head_stride
    rs = heads * hs if row_stride is None else row_stride
    x = row_buffer(T, heads, width, seed, 1, family, rs, hs, role="x")
    dy = row_buffer(T, heads, width, seed, 2, family, rs, hs, role="dy")
    extra = dh = None
    if form == "residual":
        extra = row_buffer(T, heads, width, seed, 3, "normal", rs, hs, role="res")
        dh = row_buffer(T, heads, width, seed, 4, "normal", rs, hs, role="dh")
    elif form == "gate":
        extra = row_buffer(T, heads, width, seed, 5, "normal", rs, hs, role="z")
    elif form != "plain":
        raise ValueError(form)
    return Problem(T, heads, width, rs, hs, weight(width, seed, w_dtype, w_centre), x, dy, extra,
                   dh)
