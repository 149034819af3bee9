"""Deterministic dw against the exact sum of its own terms.

The deterministic backward forms each dw term dy*x*rstd with exact products,
sums the terms with TwoSum compensation and an FP64 fold, and rounds once to
FP32 (PR #8512 page, description: exact products, compensated summation,
fixed-order FP64 fold, one rounding). With dy, x BF16 and rstd FP32 each term
has at most 8 + 8 + 24 significant bits, so it is exact in FP64, and
math.fsum over a column is the exact column sum rounded once to FP64. Hence,
on inputs without heavy cancellation, dw must be within one FP32 ulp of that
exact sum, and equal to the exact term rounded once where a column has a
single term (one row).

rstd is an input of the backward. These tests pass one computed on the host
by the FP64 oracle and rounded to FP32, so every expected value here comes
from the inputs and exact arithmetic, none from the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rmsnorm_train_fwd_amd as R
import synth

from helpers import OnGpu, oview, w_f64

pytestmark = pytest.mark.gpu


def _host_rstd(p: synth.Problem) -> np.ndarray:
    _, r = oracle.fwd(oview(p, p.x), w_f64(p.w), p.eps)
    return np.asarray(r, dtype=np.float64).astype(np.float32)


def _terms(p: synth.Problem, rstd32: np.ndarray) -> np.ndarray:
    """[rows, W] FP64 terms dy*x*rstd, each exact."""
    x = p.view(p.x).reshape(-1, p.width).double().numpy()    # BF16 -> FP64, exact
    dy = p.view(p.dy).reshape(-1, p.width).double().numpy()
    return (dy * x) * rstd32.astype(np.float64).reshape(-1, 1)


def _gpu_det_dw(p: synth.Problem, rstd32: np.ndarray, path: int) -> np.ndarray:
    g = OnGpu(p)
    r = torch.from_numpy(np.ascontiguousarray(rstd32)).cuda()  # one value per row
    _, dw = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, True, launch=R.Launch(0, 0, path))
    return dw.cpu().numpy()


def _ulp_gap(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in FP32 ulps (ordered-integer view, both signs)."""
    def key(v):
        i = v.astype(np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(key(a) - key(b))


@pytest.mark.parametrize("path", [R.PATH_SMALL, R.PATH_LARGE], ids=["small", "large"])
@pytest.mark.parametrize("H", [512, 1536, 4096, 5120, 6144])
def test_det_dw_single_row_is_the_exact_term_rounded_once(H, path):
    p = synth.make(1, H, seed=21, w_dtype="f32")
    r32 = _host_rstd(p)
    terms = _terms(p, r32)
    assert terms.shape == (1, H)
    want = terms[0].astype(np.float32)  # exact term, one RNE rounding
    got = _gpu_det_dw(p, r32, path)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("path", [R.PATH_SMALL, R.PATH_LARGE], ids=["small", "large"])
@pytest.mark.parametrize("T,H,heads", [(203, 512, 1), (203, 6144, 1), (203, 256, 24)])
def test_det_dw_small_T_within_one_ulp_of_exact_sum(T, H, heads, path):
    p = synth.make(T, H, seed=22, heads=heads, w_dtype="f32")
    r32 = _host_rstd(p)
    terms = _terms(p, r32)
    exact = np.array([math.fsum(terms[:, j]) for j in range(H)])
    got = _gpu_det_dw(p, r32, path)
    assert _ulp_gap(got, exact.astype(np.float32)).max() <= 1


@pytest.mark.parametrize("family", ["normal", "spread"])
@pytest.mark.parametrize("T,H", [(4099, 512), (4099, 4096), (2053, 5120), (1500, 6144), (1000, 1536)])
def test_det_dw_large_path_within_one_ulp_of_exact_sum(T, H, family):
    p = synth.make(T, H, seed=23, family=family, w_dtype="f32")
    r32 = _host_rstd(p)
    terms = _terms(p, r32)
    exact = np.array([math.fsum(terms[:, j]) for j in range(H)])
    got = _gpu_det_dw(p, r32, R.PATH_LARGE)
    gap = _ulp_gap(got, exact.astype(np.float32))
    assert gap.max() <= 1, f"det dw is {gap.max()} FP32 ulp from the exact sum"


# ---------------------------------------------------------- dw in BF16 --
# With dw_dtype BF16 the FP64 value is rounded once, straight to BF16.

def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("path", [R.PATH_SMALL, R.PATH_LARGE], ids=["small", "large"])
@pytest.mark.parametrize("H", [512, 4096, 6144])
def test_det_bf16_dw_single_row_is_the_exact_term_rounded_once(H, path):
    p = synth.make(1, H, seed=24, w_dtype="bf16")
    r32 = _host_rstd(p)
    want = oracle.f64_to_bf16(_terms(p, r32)[0])
    g = OnGpu(p)
    r = torch.from_numpy(np.ascontiguousarray(r32)).cuda()
    _, dw = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, True, launch=R.Launch(0, 0, path),
                                dw_dtype=torch.bfloat16)
    assert dw.dtype == torch.bfloat16
    assert np.array_equal(_bits16(dw), want)


@pytest.mark.parametrize("path", [R.PATH_SMALL, R.PATH_LARGE], ids=["small", "large"])
@pytest.mark.parametrize("T,H,heads", [(203, 1536, 1), (203, 256, 24), (4099, 5120, 1)])
def test_det_bf16_dw_is_the_exact_sum_rounded_once(T, H, heads, path):
    p = synth.make(T, H, seed=25, heads=heads, w_dtype="bf16")
    r32 = _host_rstd(p)
    terms = _terms(p, r32)
    exact = np.array([math.fsum(terms[:, j]) for j in range(H)])
    g = OnGpu(p)
    r = torch.from_numpy(np.ascontiguousarray(r32)).cuda()
    _, dw = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, True, launch=R.Launch(0, 0, path),
                                dw_dtype=torch.bfloat16)
    # the FP64 fold is within ~1e-15 relative of the exact sum, so one rounding
    # of either to BF16 agrees except at a rounding boundary: allow one ulp
    from helpers import bf16_ulp_distance
    gap = bf16_ulp_distance(_bits16(dw), oracle.f64_to_bf16(exact))
    assert gap.max() <= 1
    assert (gap == 0).mean() > 0.99
