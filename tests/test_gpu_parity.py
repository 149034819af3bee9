"""GPU parity: the HIP library against the FP64 oracle on the same seeded
inputs, element by element (row outputs on all rows, or on a sample of rows
at the full sizes; dw always on every column, summed over every row).

Workloads are the five configurations of the build (seeded synthetic inputs,
synth.py): [8,512] fwd+bwd; the small-row deterministic sweep incl. per-head
[T,24,256] views; large-T non-deterministic and deterministic backward;
fused residual at width 6144; the SiLU gate at width 4096.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_train_fwd_amd as R
import synth

from helpers import (TOL_DW, TOL_DX, TOL_Y, RTOL_RSTD, OnGpu, assert_within, bf16_ulp_distance,
                     bits, oview, ratio, sample_rows, w_f64)

pytestmark = pytest.mark.gpu

WIDTHS = (512, 1536, 2048, 4096, 5120, 6144)
SMALL_T = (1, 2, 4, 8, 16, 32, 64, 128, 203)


def run_case(p: synth.Problem, det=True, form="plain", launch=None, nsample=None, seed=0,
             zero_centred=False):
    """fwd + bwd on the GPU, checked against the oracle. `det` is one mode or a
    tuple of modes: the forward and the oracle run once and every mode's
    backward is checked against them. zero_centred: the stored w is used as
    1 + w (the oracle gets that effective weight). Returns error ratios (of the
    last mode)."""
    modes = tuple(det) if isinstance(det, (tuple, list)) else (det,)
    zc = dict(zero_centred=zero_centred)
    g = OnGpu(p)
    bwd_out = {}
    if form == "residual":
        y, rstd, h = R.rmsnorm_train_fwd(g.x, g.w, p.eps, residual=g.e, **zc)
        for m in modes:
            bwd_out[m] = R.rmsnorm_train_bwd(g.dy, h, rstd, g.w, m, dh=g.dh, launch=launch,
                                             **zc) + (None,)
    elif form == "gate":
        y, rstd = R.rmsnorm_silu_gate_train_fwd(g.x, g.e, g.w, p.eps, **zc)
        for m in modes:
            dx, dz, dw = R.rmsnorm_silu_gate_train_bwd(g.dy, g.x, g.e, rstd, g.w, m, launch=launch,
                                                       **zc)
            bwd_out[m] = (dx, dw, dz)
    else:
        y, rstd = R.rmsnorm_train_fwd(g.x, g.w, p.eps, **zc)
        for m in modes:
            bwd_out[m] = R.rmsnorm_train_bwd(g.dy, g.x, rstd, g.w, m, launch=launch, **zc) + (None,)
    torch.cuda.synchronize()

    rows, W = p.rows, p.width
    sel = sample_rows(rows, nsample, seed) if nsample else np.arange(rows, dtype=np.int64)
    w64 = oracle.zero_centred_weight(w_f64(p.w)) if zero_centred else w_f64(p.w)
    xo, dyo = oview(p, p.x), oview(p, p.dy)
    out = {}
    if form == "residual":
        ho, yo, ro = oracle.res_fwd(xo, oview(p, p.extra), w64, p.eps, sel)
        hg = bits(h).reshape(rows, W)
        assert np.array_equal(hg, ho), "h = bf16(x + residual) must be bit-exact"
        xb = oracle.View(ho, p.T, p.heads, W, p.heads * W, W)
        rows_out, dwo = oracle.bwd(dyo, xb, w64, p.eps, dh=oview(p, p.dh), sel=sel)
    elif form == "gate":
        zo = oview(p, p.extra)
        yo, ro = oracle.gate_fwd(xo, zo, w64, p.eps, sel)
        rows_out, dzo, dwo = oracle.gate_bwd(dyo, xo, zo, w64, p.eps, sel)
    else:
        yo, ro = oracle.fwd(xo, w64, p.eps, sel)
        rows_out, dwo = oracle.bwd(dyo, xo, w64, p.eps, sel=sel)

    yb = bits(y).reshape(rows, W)[sel]
    out["y"] = assert_within(oracle.bf16_to_f64(yb), yo, TOL_Y, "y")
    ulp = bf16_ulp_distance(yb, oracle.f64_to_bf16(yo))
    assert ulp.max(initial=0) <= 1, f"y differs from the rounded oracle by {ulp.max()} BF16 ulp"
    rg = rstd.reshape(-1).cpu().double().numpy()[sel]
    out["rstd"] = assert_within(rg, ro, (0.0, RTOL_RSTD), "rstd")
    for m in modes:
        dx, dw, dz = bwd_out[m]
        tag = "det" if m else "nondet"
        if form == "gate":
            dzg = oracle.bf16_to_f64(bits(dz).reshape(rows, W)[sel])
            out["dz"] = assert_within(dzg, dzo, TOL_DX, f"dz ({tag})")
        dxg = oracle.bf16_to_f64(bits(dx).reshape(rows, W)[sel])
        out["dx"] = assert_within(dxg, rows_out, TOL_DX,
                                  f"{'dx' if form != 'residual' else 'grad_h'} ({tag})")
        out["dw"] = assert_within(dw.cpu().double().numpy(), dwo, TOL_DW, f"dw ({tag})")
    return out


# ------------------------------------------------------------- config 1 ---

@pytest.mark.parametrize("seed", range(5))
def test_config1_8x512_det_fwd_bwd(seed):
    p = synth.make(8, 512, seed=seed, w_dtype="bf16")
    run_case(p, det=True)


# ------------------------------------------------------------- config 2 ---

@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H", WIDTHS)
def test_config2_small_row_det_sweep(H, w_dtype):
    for T in SMALL_T:
        for seed in range(5):
            run_case(synth.make(T, H, seed=seed, w_dtype=w_dtype), det=True)


@pytest.mark.parametrize("strides", [(12288, 512), (6144, 256)], ids=["pages_12288_512", "dense_6144_256"])
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_config2_per_head_views(strides, w_dtype):
    for T in SMALL_T:
        for seed in range(2):
            p = synth.make(T, 256, seed=seed, heads=24, w_dtype=w_dtype,
                           row_stride=strides[0], head_stride=strides[1])
            run_case(p, det=True)
    p = synth.make(64, 256, seed=3, heads=4, w_dtype=w_dtype)  # [T,4,256] contiguous
    run_case(p, det=True)
    run_case(p, det=False)


# ------------------------------------------------------------- config 3 ---

@pytest.mark.parametrize("det", [False, True], ids=["nondet", "det"])
@pytest.mark.parametrize("H", WIDTHS)
def test_config3_large_path_elementwise_ragged(H, det):
    # every chunk holds several tiles, the last tile is ragged; every row checked
    run_case(synth.make(4099, H, seed=1, w_dtype="f32"), det=det)


@pytest.mark.parametrize("det", [False, True], ids=["nondet", "det"])
def test_config3_headline_131072x4096(det):
    run_case(synth.make(131072, 4096, seed=0, w_dtype="f32"), det=det, nsample=64)


@pytest.mark.parametrize("T,H", [(65537, 6144), (98304, 1536), (131072, 5120), (65537, 2048)])
def test_config3_full_size_nondet(T, H):
    run_case(synth.make(T, H, seed=2, w_dtype="f32"), det=False, nsample=32)


@pytest.mark.parametrize("T", [65537, 98304, 131072])
@pytest.mark.parametrize("H", (1536, 2048, 4096, 5120, 6144))
def test_config3_full_sweep(H, T):
    # every config-3 shape in both modes (PR #8848 page, "Measurement": every
    # row of the table runs both); sampled rows, dw on every column
    print(f"[config3] [{T}, {H}] non-det + det", flush=True)
    run_case(synth.make(T, H, seed=3, w_dtype="f32"), det=(False, True), nsample=24)


# ------------------------------------------------------------- config 4 ---

@pytest.mark.parametrize("det", [False, True], ids=["nondet", "det"])
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_config4_residual_6144(w_dtype, det):
    for seed in range(3):
        run_case(synth.make(32, 6144, seed=seed, w_dtype=w_dtype, form="residual"), det=det,
                 form="residual")
    run_case(synth.make(65537, 6144, seed=0, w_dtype=w_dtype, form="residual"), det=det,
             form="residual", nsample=32)


@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_config4_residual_131072(w_dtype):
    print(f"[config4] residual [131072, 6144] w {w_dtype}, non-det + det", flush=True)
    run_case(synth.make(131072, 6144, seed=1, w_dtype=w_dtype, form="residual"),
             det=(False, True), form="residual", nsample=24)


# ------------------------------------------------------------- config 5 ---

@pytest.mark.parametrize("det", [False, True], ids=["nondet", "det"])
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_config5_gate_3534x4096(w_dtype, det):
    run_case(synth.make(3534, 4096, seed=0, w_dtype=w_dtype, form="gate"), det=det, form="gate")


@pytest.mark.parametrize("T", [8192, 16384])
def test_config5_gate_larger(T):
    run_case(synth.make(T, 4096, seed=1, w_dtype="f32", form="gate"), det=False, form="gate",
             nsample=48)


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("H", (256, 512, 1536, 2048, 5120, 6144))
def test_gate_other_widths(H, det):
    # 300 rows: main kernel + fold; 4099 rows: several tiles per chunk
    run_case(synth.make(300, H, seed=4, w_dtype="f32", form="gate"), det=det, form="gate")
    run_case(synth.make(4099, H, seed=5, w_dtype="f32", form="gate"), det=det, form="gate",
             nsample=48)


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("H", (256, 512, 1536, 4096, 5120))
def test_residual_other_widths(H, det):
    run_case(synth.make(300, H, seed=4, w_dtype="bf16", form="residual"), det=det,
             form="residual")
    run_case(synth.make(4099, H, seed=5, w_dtype="f32", form="residual"), det=det,
             form="residual", nsample=48)


# ------------------------------------------------------------ input families --

@pytest.mark.parametrize("family", ["cancel", "spread"])
@pytest.mark.parametrize("H", (512, 4096))
def test_det_adversarial_families(H, family):
    # deterministic dw keeps the budget on cancellation and scale-spread inputs
    run_case(synth.make(8192, H, seed=5, family=family, w_dtype="f32"), det=True, nsample=64)


def test_nondet_spread_family():
    run_case(synth.make(8192, 2048, seed=6, family="spread", w_dtype="f32"), det=False, nsample=64)


# ---------------------------------------------------------------- edge cases --

def test_zero_tokens():
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, dtype=torch.float32, device="cuda")
    y, rstd = R.rmsnorm_train_fwd(x, w)
    assert y.shape == (0, 512) and rstd.shape == (0,)
    for det in (True, False):
        dx, dw = R.rmsnorm_train_bwd(x, x, rstd, w, det)
        torch.cuda.synchronize()
        assert dx.shape == (0, 512)
        assert torch.all(dw == 0)


def test_zero_and_constant_rows():
    # zero row: rstd = 1/sqrt(eps) = 1000, y = 0, dx = rstd * dy * w
    T, H = 5, 1536
    p = synth.make(T, H, seed=0, w_dtype="f32")
    view = p.view(p.x)
    view[0].zero_()
    view[2].fill_(3.0)
    out = run_case(p, det=True)
    g = OnGpu(p)
    _, rstd = R.rmsnorm_train_fwd(g.x, g.w)
    assert abs(rstd[0].item() - 1000.0) <= 1000.0 * 1e-6
    assert abs(rstd[2].item() - 1.0 / np.sqrt(9.0 + 1e-6)) <= 1e-6
    assert out["dw"] <= 1.0


# ------------------------------------------------------- dw in BF16 --

@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("T,H,form", [(8, 512, "plain"), (4099, 4096, "plain"), (65537, 2048, "plain"),
                                      (777, 6144, "residual"), (3534, 4096, "gate")])
def test_bf16_dw_within_one_ulp_of_the_oracle(T, H, form, det):
    """dw_dtype BF16: the FP64 value rounded once to BF16; within one BF16 ulp
    of the FP64 oracle rounded to BF16 (one ulp covers the FP32 blocks of the
    non-deterministic mode and values at a rounding boundary)."""
    p = synth.make(T, H, seed=6, w_dtype="bf16", form=form)
    g = OnGpu(p)
    w = w_f64(p.w)
    if form == "residual":
        _, rstd, h = R.rmsnorm_train_fwd(g.x, g.w, p.eps, residual=g.e)
        _, dw = R.rmsnorm_train_bwd(g.dy, h, rstd, g.w, det, dh=g.dh, dw_dtype=torch.bfloat16)
        ho, _, _ = oracle.res_fwd(oview(p, p.x), oview(p, p.extra), w, p.eps)
        hb = oracle.View(ho, p.T, p.heads, H, p.heads * H, H)   # the oracle's own h
        _, ref = oracle.bwd(oview(p, p.dy), hb, w, p.eps, dh=oview(p, p.dh), want_rows=False)
    elif form == "gate":
        _, rstd = R.rmsnorm_silu_gate_train_fwd(g.x, g.e, g.w, p.eps)
        _, _, dw = R.rmsnorm_silu_gate_train_bwd(g.dy, g.x, g.e, rstd, g.w, det,
                                                 dw_dtype=torch.bfloat16)
        _, _, ref = oracle.gate_bwd(oview(p, p.dy), oview(p, p.x), oview(p, p.extra), w, p.eps,
                                    want_rows=False)
    else:
        _, rstd = R.rmsnorm_train_fwd(g.x, g.w, p.eps)
        _, dw = R.rmsnorm_train_bwd(g.dy, g.x, rstd, g.w, det, dw_dtype=torch.bfloat16)
        _, ref = oracle.bwd(oview(p, p.dy), oview(p, p.x), w, p.eps, want_rows=False)
    assert dw.dtype == torch.bfloat16
    ulp = bf16_ulp_distance(bits(dw), oracle.f64_to_bf16(ref))
    assert ulp.max() <= 1, f"BF16 dw differs from the rounded oracle by {ulp.max()} ulp"


# ------------------------------------------------- grouped per-head gate --
# The PR #8656 page (Tables 1 and 2) times the gated form on tokens x heads
# shapes: each head's slice is normalised on its own and gated by its own z, one
# w shared by all heads. The head dimension is not stated there; these cases use
# 256 (the per-head width of the other pages) and 512.

@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("T,heads,W", [(37, 48, 256), (300, 48, 256), (40, 8, 512), (257, 8, 512)])
def test_grouped_per_head_gate(T, heads, W, det):
    run_case(synth.make(T, W, seed=8, heads=heads, w_dtype="f32", form="gate"), det=det,
             form="gate")


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("T,heads", [(3534, 48), (8192, 32)])
def test_grouped_per_head_gate_table_shapes(T, heads, det):
    run_case(synth.make(T, 256, seed=9, heads=heads, w_dtype="f32", form="gate"), det=det,
             form="gate", nsample=64)
