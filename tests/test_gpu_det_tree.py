"""Deterministic dw, bit for bit, against an emulation of the documented tree.

include/rmsnorm_train.h defines the deterministic dw as a fixed summation
tree (PR #8512 page, description: exact products, TwoSum-compensated
summation, fixed-order FP64 fold, one rounding): rows form tiles of R rows,
the tiles are dealt in turn to K chunks, row q of each of a chunk's tiles
forms sub-chain q, summed in ascending tile order by Dot2 in FP32 (TwoProduct
of dy*x and rstd, TwoSum into s, errors into c); d_q = (double)s + (double)c;
the chunk partial is 0.0 + d_0 + ... + d_{R-1}; partials fold in FP64 in
groups of 32 consecutive chunks, then over the groups, each from 0.0; one
rounding to FP32. This file implements that text in numpy (every FP32
operation rounded to FP32; the FMA error term taken from the exact FP64
product) with R and K from the library's plan, and requires the GPU's dw to
have exactly those bits. rstd is computed on the host by the oracle, so no
input or expected value comes from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_train_fwd_amd as R
import synth

from helpers import OnGpu, oview, w_f64

pytestmark = pytest.mark.gpu

f32 = np.float32


def _two_sum(a, b):
    s = (a + b).astype(f32)
    bb = (s - a).astype(f32)
    e = ((a - (s - bb).astype(f32)).astype(f32) + (b - bb).astype(f32)).astype(f32)
    return s, e


def emulate_det_dw(x: np.ndarray, dy: np.ndarray, rstd32: np.ndarray, R_: int, K: int) -> np.ndarray:
    """x, dy: [rows, W] float32 (BF16 values); rstd32: [rows] float32."""
    rows, W = x.shape
    tiles = -(-rows // R_)
    part = np.zeros((K, W), np.float64)
    for k in range(K):
        d = []
        for q in range(R_):
            s = np.zeros(W, f32)
            c = np.zeros(W, f32)
            for t in range(k, tiles, K):            # the chunk's tiles, ascending
                r = t * R_ + q
                if r >= rows:
                    continue
                a = (dy[r] * x[r]).astype(f32)      # exact: 8 + 8 significant bits
                b = rstd32[r]
                p = (a * b).astype(f32)
                exact = a.astype(np.float64) * np.float64(b)
                pe = (exact - p.astype(np.float64)).astype(f32)  # fma(a, b, -p)
                s, t_err = _two_sum(s, p)
                c = (c + (t_err + pe).astype(f32)).astype(f32)
            d.append(s.astype(np.float64) + c.astype(np.float64))
        acc = np.zeros(W, np.float64)
        for dq in d:
            acc = acc + dq
        part[k] = acc
    total = np.zeros(W, np.float64)
    for g0 in range(0, K, 32):
        sg = np.zeros(W, np.float64)
        for k in range(g0, min(g0 + 32, K)):
            sg = sg + part[k]
        total = total + sg
    return total.astype(f32)


# On ordinary inputs Dot2 with an FP64 fold is accurate enough that most trees
# round to the same bits; these cases check every form and layout, and the
# cancellation cases below check the grouping itself.
@pytest.mark.parametrize("path", [R.PATH_LARGE, R.PATH_SMALL], ids=["large", "small"])
@pytest.mark.parametrize("T,H,heads,form", [
    (203, 512, 1, "plain"), (1, 6144, 1, "plain"), (257, 1536, 1, "plain"), (4099, 4096, 1, "plain"),
    (2053, 5120, 1, "plain"), (1500, 6144, 1, "plain"), (997, 2048, 1, "plain"), (150, 256, 24, "plain"),
    (777, 6144, 1, "residual"), (300, 512, 1, "residual")])
def test_det_dw_bits_follow_the_documented_tree(T, H, heads, form, path):
    p = synth.make(T, H, seed=31, heads=heads, w_dtype="f32", form=form)
    g = OnGpu(p)
    if form == "residual":
        # the backward reads the BF16 h; the oracle's h is bit-exact with the GPU's
        hbits, _, r64 = oracle.res_fwd(oview(p, p.x), oview(p, p.extra), w_f64(p.w), p.eps)
        xin_host = torch.from_numpy(hbits.view(np.int16)).view(torch.bfloat16).reshape(-1, H)
        xin = xin_host.cuda().reshape(g.x.shape)
    else:
        _, r64 = oracle.fwd(oview(p, p.x), w_f64(p.w), p.eps)
        xin_host = p.view(p.x).reshape(-1, H)
        xin = g.x
    r32 = np.asarray(r64, np.float64).astype(f32)
    rstd = torch.from_numpy(np.ascontiguousarray(r32)).cuda()
    plan = R.rmsnorm_train_bwd_query(xin, True)
    launch = R.Launch(0, 0, path)
    if form == "residual":
        _, dw = R.rmsnorm_train_bwd(g.dy, xin, rstd, g.w, True, dh=g.dh, launch=launch)
    else:
        _, dw = R.rmsnorm_train_bwd(g.dy, xin, rstd, g.w, True, launch=launch)
    x = xin_host.float().numpy().astype(f32)
    dy = p.view(p.dy).reshape(-1, H).float().numpy().astype(f32)
    want = emulate_det_dw(x, dy, r32, plan.subchains, plan.chunks)
    got = dw.cpu().numpy()
    diff = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert diff.size == 0, f"{diff.size} of {H} columns differ from the documented tree, e.g. column {diff[:5]}"


def cancellation_rows(rows: int, W: int, seed: int):
    """Inputs on which the tree shows in the result: pairs of rows with products
    near 2^28 that cancel exactly (the second row of a pair is x, -dy with the
    same rstd), laid out half the rows apart so that a pair lands in different
    chunks, plus a tail of ordinary rows. Within a sub-chain, Dot2's FP32
    compensation then carries rounding errors near ulp(2^28), far above the
    ulp of the small final sum, so trees that group the rows differently give
    different bits. rstd is an input of the backward and is drawn here."""
    g = torch.Generator().manual_seed(seed)
    tail = max(1, rows // 8)
    m = (rows - tail) // 2
    tail = rows - 2 * m

    def big(shape):
        mag = (torch.rand(shape, generator=g) + 1) * 2.0**14
        return (mag * (torch.randint(0, 2, shape, generator=g) * 2 - 1)).bfloat16()

    x, dy = big((m, W)), big((m, W))
    X = torch.cat([x, torch.randn(tail, W, generator=g).bfloat16(), x])
    DY = torch.cat([dy, torch.randn(tail, W, generator=g).bfloat16(), -dy])
    rs = (torch.rand(rows, generator=g) + 1).float()
    rs[m + tail:] = rs[:m]
    return X, DY, rs


@pytest.mark.parametrize("path", [R.PATH_LARGE, R.PATH_SMALL], ids=["large", "small"])
@pytest.mark.parametrize("rows", [203, 997, 4099])
@pytest.mark.parametrize("H", [256, 512, 1536, 2048, 4096, 5120, 6144])
def test_det_dw_bits_follow_the_documented_tree_under_cancellation(H, rows, path):
    X, DY, rs = cancellation_rows(rows, H, seed=H + rows)
    x, dy, r32 = X.float().numpy(), DY.float().numpy(), rs.numpy()
    xg, dyg = X.cuda(), DY.cuda()
    w = torch.ones(H, device="cuda")
    plan = R.rmsnorm_train_bwd_query(xg, True)
    want = emulate_det_dw(x, dy, r32, plan.subchains, plan.chunks)
    # the input separates trees: halving the chunk count changes most columns
    other = emulate_det_dw(x, dy, r32, plan.subchains, max(1, plan.chunks // 2))
    assert (other != want).mean() > 0.5
    _, dw = R.rmsnorm_train_bwd(dyg, xg, rs.cuda(), w, True, launch=R.Launch(0, 0, path))
    got = dw.cpu().numpy()
    diff = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert diff.size == 0, f"{diff.size} of {H} columns differ from the documented tree"


# Row counts where the tree switches from at most 8 tiles per chunk (and the
# single-launch path) to up to 256 chunks (main kernel + fold): S(width).
SMALL_ROWS = {256: 1280, 512: 960, 1536: 640, 2048: 640, 4096: 512, 5120: 512, 6144: 384}


@pytest.mark.parametrize("path", [R.PATH_LARGE, R.PATH_SMALL], ids=["large", "small"])
@pytest.mark.parametrize("above", [0, 1], ids=["S", "S+1"])
@pytest.mark.parametrize("H", [256, 512, 1536, 2048, 4096, 5120, 6144])
def test_det_dw_bits_at_the_small_row_limit(H, above, path):
    rows = SMALL_ROWS[H] + above
    X, DY, rs = cancellation_rows(rows, H, seed=7 * H + rows)
    x, dy, r32 = X.float().numpy(), DY.float().numpy(), rs.numpy()
    xg, dyg = X.cuda(), DY.cuda()
    plan = R.rmsnorm_train_bwd_query(xg, True)
    tiles = -(-rows // plan.subchains)
    assert plan.chunks == (min(tiles, 256) if above else -(-tiles // 8))
    assert plan.path == (R.PATH_LARGE if above else R.PATH_SMALL)
    want = emulate_det_dw(x, dy, r32, plan.subchains, plan.chunks)
    _, dw = R.rmsnorm_train_bwd(dyg, xg, rs.cuda(), torch.ones(H, device="cuda"), True,
                                launch=R.Launch(0, 0, path))
    got = dw.cpu().numpy()
    diff = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert diff.size == 0, f"{diff.size} of {H} columns differ from the documented tree"
