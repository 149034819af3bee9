"""Tensors of more than 2**32 elements: 64-bit addressing in every kernel.

The inputs repeat a seeded block of P rows (P = 97, a prime, so a 32-bit wrap
of an element offset would land inside some other row rather than on a copy of
the same one). Row t of every output then equals the oracle's output for block
row t % P, and with rows = q*P + rem the weight gradient over the whole call is
q * dw(block) + dw(first rem rows of the block), exactly in real arithmetic; the
oracle evaluates both terms in FP64. Row outputs are compared on a sample of
rows that straddles the 2**31- and 2**32-element boundaries; dw on every
column.

The dw bound. The kernels take each row's factors in FP32: the forward's rstd
(FP32 sum of squares over at most 8 terms per lane and a 10-level lane tree,
then a division, a sqrt and a reciprocal: relative error below 11 * 2**-24),
the SiLU value of the gated form (exp2, reciprocal and two products: below
5 * 2**-24), and, in the non-deterministic mode, FP32 sums of 8-row blocks
(below 8 * 2**-24 of the block's absolute sum). On independent rows these
errors are random and the pages' budget (atol 1e-4 + rtol 1e-4) covers them;
here every block row appears q times, so its rounding errors repeat q times and
add up coherently. The check is therefore the pages' budget plus
2**-19 * sum over rows |dy * xhat * s| (s = |silu(z)| for the gate, else 1),
which bounds those repeated errors; a wrong address would miss by the size of
dw itself (1e3 to 1e5 here).
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_train_fwd_amd as R
import synth

from helpers import TOL_DW, TOL_DX, TOL_Y, RTOL_RSTD, assert_within, bits, w_f64

pytestmark = pytest.mark.gpu

P = 97


def tile_rows(block: torch.Tensor, T: int) -> torch.Tensor:
    """A contiguous [T, ...] tensor on the GPU whose row t is block row t % P."""
    dev = torch.device("cuda")
    block = block.to(dev).contiguous()
    out = torch.empty((T,) + tuple(block.shape[1:]), dtype=block.dtype, device=dev)
    q, rem = divmod(T, block.shape[0])
    out[: q * block.shape[0]].view(q, *block.shape).copy_(block.unsqueeze(0).expand(q, *block.shape))
    out[q * block.shape[0]:].copy_(block[:rem])
    return out


def sample(T: int, heads: int, width: int) -> np.ndarray:
    """Row indices (t*heads + h) around the 2**31 and 2**32 element offsets, both ends, and a
    seeded spread."""
    rows = T * heads
    s = {0, 1, rows - 2, rows - 1}
    for b in (1 << 31, 1 << 32):
        r = b // width
        s |= {r - 1, r, r + 1}
    s |= set(np.random.default_rng(0).choice(rows, 24, replace=False).tolist())
    return np.array(sorted(r for r in s if 0 <= r < rows), dtype=np.int64)


def views(p: synth.Problem, buf: torch.Tensor, rem: int):
    full = oracle.View(bits(buf), p.T, p.heads, p.width, p.row_stride, p.head_stride)
    part = oracle.View(full.buf, rem, p.heads, p.width, p.row_stride, p.head_stride)
    return full, part


def abs_terms(dy: np.ndarray, x: np.ndarray, eps: float, z=None) -> np.ndarray:
    """Per column: sum over rows of |dy * xhat| (times |z| >= |silu(z)| for the gate), FP64,
    for the error bound only."""
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    t = np.abs(dy) * np.abs(x) * r[:, None]
    if z is not None:
        t *= np.abs(z)
    return t.sum(axis=0)


def block_f64(buf: np.ndarray, rows: int, width: int) -> np.ndarray:
    return oracle.bf16_to_f64(np.asarray(buf).reshape(-1, width)[:rows])


def dw_bound(p, q, rem, dy_bits, x_bits, z_bits=None):
    """2**-19 * sum over all q*P + rem rows of |dy * xhat * s|."""
    W, n = p.width, P * p.heads
    def s(rows):
        z = block_f64(z_bits, rows, W) if z_bits is not None else None
        return abs_terms(block_f64(dy_bits, rows, W), block_f64(x_bits, rows, W), p.eps, z)
    return 2.0 ** -19 * (q * s(n) + s(rem * p.heads))


def assert_dw(got: torch.Tensor, block, rem_part, q, bound, what):
    ref = q * block + rem_part
    got = got.double().cpu().numpy()
    tol = TOL_DW[0] + TOL_DW[1] * np.abs(ref) + bound
    r = float(np.max(np.abs(got - ref) / tol))
    assert np.isfinite(got).all() and r <= 1.0, f"{what}: worst error is {r:.3g}x the bound"


def gather(t: torch.Tensor, rows: np.ndarray, width: int) -> np.ndarray:
    idx = torch.from_numpy(rows).to(t.device)
    return oracle.bf16_to_f64(bits(t.reshape(-1, width).index_select(0, idx)))


@pytest.mark.parametrize("heads,W,T,seed", [(1, 6144, 720899, 3), (24, 256, 720899, 0)],
                         ids=["6144", "24x256"])
def test_plain_past_2_pow_32_elements(heads, W, T, seed):
    p = synth.make(P, W, seed=seed, heads=heads, w_dtype="f32")
    assert T * heads * W > 1 << 32
    x = tile_rows(p.view(p.x), T)
    dy = tile_rows(p.view(p.dy), T)
    if heads == 1:
        x, dy = x.view(T, W), dy.view(T, W)
    w = p.w.cuda()
    y, rstd = R.rmsnorm_train_fwd(x, w, p.eps)
    sel = sample(T, heads, W)
    q, rem = divmod(T, P)
    xo, xr = views(p, p.x, rem)
    dyo, dyr = views(p, p.dy, rem)
    w64 = w_f64(p.w)
    yo, ro = oracle.fwd(xo, w64, p.eps, sel % (P * heads))
    assert_within(gather(y, sel, W), yo, TOL_Y, "y")
    rg = rstd.reshape(-1).index_select(0, torch.from_numpy(sel).cuda()).double().cpu().numpy()
    assert_within(rg, ro, (0.0, RTOL_RSTD), "rstd")
    del y
    dxo, dwb = oracle.bwd(dyo, xo, w64, p.eps, sel=sel % (P * heads))
    _, dwr = oracle.bwd(dyr, xr, w64, p.eps, want_rows=False)
    bound = dw_bound(p, q, rem, bits(p.dy), bits(p.x))
    for det in (True, False):
        dx, dw = R.rmsnorm_train_bwd(dy, x, rstd, w, det)
        torch.cuda.synchronize()
        assert_within(gather(dx, sel, W), dxo, TOL_DX, f"dx det={det}")
        assert_dw(dw, dwb, dwr, q, bound, f"dw det={det}")
        del dx, dw


def test_residual_past_2_pow_32_elements():
    W, T = 6144, 720899
    p = synth.make(P, W, seed=1, w_dtype="bf16", form="residual")
    x = tile_rows(p.view(p.x), T).view(T, W)
    res = tile_rows(p.view(p.extra), T).view(T, W)
    w = p.w.cuda()
    y, rstd, h = R.rmsnorm_train_fwd(x, w, p.eps, residual=res)
    del x, res
    sel = sample(T, 1, W)
    q, rem = divmod(T, P)
    xo, _ = views(p, p.x, rem)
    reso, _ = views(p, p.extra, rem)
    w64 = w_f64(p.w)
    hb, yo, ro = oracle.res_fwd(xo, reso, w64, p.eps, sel % P)
    idx = torch.from_numpy(sel).cuda()
    assert np.array_equal(bits(h.index_select(0, idx)), hb[sel % P]), "h must be bit-exact"
    assert_within(gather(y, sel, W), yo, TOL_Y, "y")
    del y
    dy = tile_rows(p.view(p.dy), T).view(T, W)
    dh = tile_rows(p.view(p.dh), T).view(T, W)
    hv = oracle.View(hb, P, 1, W, W, W)
    hr = oracle.View(hb, rem, 1, W, W, W)
    dyo, dyr = views(p, p.dy, rem)
    dho, dhr = views(p, p.dh, rem)
    gho, dwb = oracle.bwd(dyo, hv, w64, p.eps, dh=dho, sel=sel % P)
    _, dwr = oracle.bwd(dyr, hr, w64, p.eps, dh=dhr, want_rows=False)
    bound = dw_bound(p, q, rem, bits(p.dy), hb)
    gh, dw = R.rmsnorm_train_bwd(dy, h, rstd, w, False, dh=dh)
    torch.cuda.synchronize()
    assert_within(gather(gh, sel, W), gho, TOL_DX, "grad_h")
    assert_dw(dw, dwb, dwr, q, bound, "dw")


def test_gate_past_2_pow_32_elements():
    W, T = 4096, 1081349  # 4.43e9 elements
    p = synth.make(P, W, seed=2, w_dtype="f32", form="gate")
    assert T * W > 1 << 32
    x = tile_rows(p.view(p.x), T).view(T, W)
    z = tile_rows(p.view(p.extra), T).view(T, W)
    w = p.w.cuda()
    y, rstd = R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)
    sel = sample(T, 1, W)
    q, rem = divmod(T, P)
    xo, xr = views(p, p.x, rem)
    zo, zr = views(p, p.extra, rem)
    dyo, dyr = views(p, p.dy, rem)
    w64 = w_f64(p.w)
    yo, ro = oracle.gate_fwd(xo, zo, w64, p.eps, sel % P)
    assert_within(gather(y, sel, W), yo, TOL_Y, "y")
    del y
    dy = tile_rows(p.view(p.dy), T).view(T, W)
    dxo, dzo, dwb = oracle.gate_bwd(dyo, xo, zo, w64, p.eps, sel % P)
    _, _, dwr = oracle.gate_bwd(dyr, xr, zr, w64, p.eps, want_rows=False)
    bound = dw_bound(p, q, rem, bits(p.dy), bits(p.x), bits(p.extra))
    dx, dz, dw = R.rmsnorm_silu_gate_train_bwd(dy, x, z, rstd, w, True)
    torch.cuda.synchronize()
    assert_within(gather(dx, sel, W), dxo, TOL_DX, "dx")
    assert_within(gather(dz, sel, W), dzo, TOL_DX, "dz")
    assert_dw(dw, dwb, dwr, q, bound, "dw")
