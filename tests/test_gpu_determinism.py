"""Bitwise reproducibility on the GPU.

Deterministic mode (PR #8512 page, description): dw does not depend on the
grid size or the number of compute units. Checked here as bit equality of dw
over repeats, over workgroup counts of the main and fold launches, and across
the two paths (one launch for small row counts; main kernel + fold), since all
of them follow one canonical summation tree. dx, y and rstd are bit-equal
across paths and modes, as the row arithmetic is shared.
"""
import numpy as np
import pytest
import torch

import rmsnorm_train_fwd_amd as R
import synth

from helpers import OnGpu, bits

pytestmark = pytest.mark.gpu

LAUNCHES = [
    None,
    R.Launch(0, 0, R.PATH_LARGE),
    R.Launch(1, 1, R.PATH_LARGE),
    R.Launch(3, 5, R.PATH_LARGE),
    R.Launch(64, 2, R.PATH_LARGE),
    R.Launch(4096, 0, R.PATH_LARGE),
    R.Launch(0, 0, R.PATH_SMALL),
    R.Launch(1, 1, R.PATH_SMALL),
    R.Launch(2, 3, R.PATH_SMALL),
    R.Launch(97, 0, R.PATH_SMALL),
]

CASES = [
    # (T, width, heads, form)
    (1, 512, 1, "plain"), (7, 4096, 1, "plain"), (16, 6144, 1, "plain"),
    (203, 1536, 1, "plain"), (257, 2048, 1, "plain"), (1000, 5120, 1, "plain"),
    (4099, 4096, 1, "plain"), (33, 256, 24, "plain"), (300, 512, 1, "residual"),
    (129, 4096, 1, "gate"), (17, 6144, 1, "residual"), (600, 256, 4, "gate"),
    (777, 5120, 1, "residual"), (300, 5120, 1, "gate"), (2000, 1536, 1, "gate"),
]


def _bwd(g, form, rstd, h, det, launch):
    if form == "residual":
        dx, dw = R.rmsnorm_train_bwd(g.dy, h, rstd, g.w, det, dh=g.dh, launch=launch)
        return bits(dx), dw.cpu().numpy().view(np.uint32)
    if form == "gate":
        dx, dz, dw = R.rmsnorm_silu_gate_train_bwd(g.dy, g.x, g.e, rstd, g.w, det, launch=launch)
        return np.concatenate([bits(dx).ravel(), bits(dz).ravel()]), dw.cpu().numpy().view(np.uint32)
    dx, dw = R.rmsnorm_train_bwd(g.dy, g.x, rstd, g.w, det, launch=launch)
    return bits(dx), dw.cpu().numpy().view(np.uint32)


def _fwd(g, form):
    h = None
    if form == "residual":
        y, rstd, h = R.rmsnorm_train_fwd(g.x, g.w, residual=g.e)
    elif form == "gate":
        y, rstd = R.rmsnorm_silu_gate_train_fwd(g.x, g.e, g.w)
    else:
        y, rstd = R.rmsnorm_train_fwd(g.x, g.w)
    return y, rstd, h


@pytest.mark.parametrize("T,W,heads,form", CASES)
def test_det_dw_bitwise_across_grids_and_paths(T, W, heads, form):
    p = synth.make(T, W, seed=11, heads=heads, w_dtype="f32", form=form)
    g = OnGpu(p)
    y, rstd, h = _fwd(g, form)
    y2, rstd2, h2 = _fwd(g, form)
    assert np.array_equal(bits(y), bits(y2))
    assert torch.equal(rstd, rstd2)
    ref_dx, ref_dw = _bwd(g, form, rstd, h, True, None)
    for launch in LAUNCHES:
        dx, dw = _bwd(g, form, rstd, h, True, launch)
        tag = None if launch is None else (launch.grid, launch.fold_grid, launch.path)
        assert np.array_equal(dw, ref_dw), f"det dw bits changed with launch {tag}"
        assert np.array_equal(dx, ref_dx), f"dx bits changed with launch {tag}"
    # the non-deterministic mode shares the row arithmetic: dx is bit-equal
    dx_nd, _ = _bwd(g, form, rstd, h, False, R.Launch(0, 0, R.PATH_LARGE))
    assert np.array_equal(dx_nd, ref_dx)


def test_det_dw_bitwise_over_repeats_large():
    p = synth.make(65537, 4096, seed=12, w_dtype="bf16")
    g = OnGpu(p)
    _, rstd = R.rmsnorm_train_fwd(g.x, g.w)
    first = None
    for grid in (0, 256, 1000, 7):
        for _ in range(2):
            _, dw = R.rmsnorm_train_bwd(g.dy, g.x, rstd, g.w, True, launch=R.Launch(grid, 0, 0))
            b = dw.cpu().numpy().view(np.uint32)
            if first is None:
                first = b
            assert np.array_equal(b, first)


def test_plan_is_grid_independent():
    # the chunking (the summation tree) depends on the row count and width only
    x = torch.empty((131072, 4096), dtype=torch.bfloat16)
    a = R.rmsnorm_train_bwd_query(x, True)
    b = R.rmsnorm_train_bwd_query(x, True, R.Launch(7, 3, R.PATH_LARGE))
    assert (a.chunks, a.subchains) == (b.chunks, b.subchains)


@pytest.mark.parametrize("T,W,form", [(203, 512, "plain"), (4099, 4096, "plain"), (300, 4096, "gate")])
def test_det_bf16_dw_bitwise_across_grids_and_paths(T, W, form):
    p = synth.make(T, W, seed=13, w_dtype="bf16", form=form)
    g = OnGpu(p)
    if form == "gate":
        _, rstd = R.rmsnorm_silu_gate_train_fwd(g.x, g.e, g.w)
    else:
        _, rstd = R.rmsnorm_train_fwd(g.x, g.w)
    first = None
    for launch in LAUNCHES:
        if form == "gate":
            dw = R.rmsnorm_silu_gate_train_bwd(g.dy, g.x, g.e, rstd, g.w, True, launch=launch,
                                               dw_dtype=torch.bfloat16)[2]
        else:
            dw = R.rmsnorm_train_bwd(g.dy, g.x, rstd, g.w, True, launch=launch,
                                     dw_dtype=torch.bfloat16)[1]
        b = bits(dw)
        if first is None:
            first = b
        assert np.array_equal(b, first), f"BF16 det dw bits changed with launch {launch}"
