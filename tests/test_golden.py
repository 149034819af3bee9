"""The pages' printed worked example, as a stored fixture (tests/golden/).

review_8848_cancellation.txt: the column terms 65536, 2^-10, -65536 of the
PR #8848 page's review comment. Exact arithmetic gives dw = 2^-10; one FP32
sum over a block of rows gives 0. The fixture's rows realise those terms in
every column (x = 1, eps = 0, w = 1, dy = the term).

CPU: the oracle (FP64, ascending rows) must return the exact 2^-10, and a
plain FP32 sum of the terms returns 0, as the page says.
GPU: the deterministic backward (exact products, TwoSum, FP64 fold) returns
2^-10 bit for bit on both paths; the non-deterministic backward, whose dw is
the page's 8-row FP32 blocks, returns 0 when the three rows fall into one
block of one sub-chain (width 6144: one row per tile, one chunk), which pins
that mode to the blocked design the review criticises.
"""
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = os.path.join(HERE, "golden", "review_8848_cancellation.txt")


def load_fixture(path=FIXTURE):
    fx = {"rows": []}
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "row":
                fx["rows"].append(tuple(float.fromhex(v) for v in vals))
            elif key == "width":
                fx[key] = int(vals[0])
            else:
                fx[key] = float.fromhex(vals[0])
    return fx


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """Exact BF16 values (float64) -> BF16 bit patterns (asserts exactness)."""
    f32 = np.asarray(values, np.float32)
    assert np.array_equal(f32.astype(np.float64), values)
    u = f32.view(np.uint32)
    assert not np.any(u & 0xFFFF), "fixture value is not a BF16 value"
    return (u >> 16).astype(np.uint16)


def fixture_arrays(fx, width=None):
    W = width or fx["width"]
    xs = np.array([[r[0]] * W for r in fx["rows"]], np.float64)
    dys = np.array([[r[1]] * W for r in fx["rows"]], np.float64)
    return W, bf16_bits(xs), bf16_bits(dys)


def test_fixture_oracle_returns_the_exact_sum():
    fx = load_fixture()
    W, xb, dyb = fixture_arrays(fx)
    w = np.full(W, fx["w"])
    dx, dw = oracle.bwd(oracle.View.dense(dyb), oracle.View.dense(xb), w, fx["eps"])
    assert np.all(dw == fx["dw_exact"])
    assert np.all(dx == fx["dx_exact"])


def test_fixture_plain_fp32_block_loses_the_small_term():
    fx = load_fixture()
    s = np.float32(0.0)
    for _, dy in fx["rows"]:
        s = np.float32(s + np.float32(dy))  # xhat = 1: each term is dy
    assert float(s) == fx["dw_fp32_block"] != fx["dw_exact"]


def _gpu_dw(fx, W, det, path):
    import rmsnorm_train_fwd_amd as R

    _, xb, dyb = fixture_arrays(fx, W)
    w = np.full(W, fx["w"])
    _, rstd = oracle.fwd(oracle.View.dense(xb), w, fx["eps"])
    dev = torch.device("cuda:0")
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    dy = torch.from_numpy(dyb.view(np.int16)).view(torch.bfloat16).to(dev)
    r = torch.from_numpy(rstd.astype(np.float32)).to(dev)
    wt = torch.from_numpy(w.astype(np.float32)).to(dev)
    dx, dw = R.rmsnorm_train_bwd(dy, x, r, wt, det, launch=R.Launch(0, 0, path))
    return dx.float().cpu().numpy(), dw.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["small", "large"])
@pytest.mark.parametrize("W", [512, 4096, 6144])
def test_fixture_det_dw_is_exact_on_the_gpu(W, path):
    import rmsnorm_train_fwd_amd as R

    fx = load_fixture()
    dx, dw = _gpu_dw(fx, W, True, R.PATH_SMALL if path == "small" else R.PATH_LARGE)
    want = np.float32(fx["dw_exact"])
    assert np.array_equal(dw.view(np.uint32), np.full(W, want).view(np.uint32))
    assert np.all(dx == fx["dx_exact"])


@pytest.mark.gpu
def test_fixture_nondet_dw_is_the_blocked_fp32_sum():
    import rmsnorm_train_fwd_amd as R

    fx = load_fixture()
    plan = R.rmsnorm_train_bwd_query(torch.empty((3, 6144), dtype=torch.bfloat16), False,
                                     launch=R.Launch(0, 0, R.PATH_LARGE))
    assert (plan.subchains, plan.chunks) == (1, 1)  # all three rows in one 8-row block
    _, dw = _gpu_dw(fx, 6144, False, R.PATH_LARGE)
    assert np.all(dw == np.float32(fx["dw_fp32_block"]))
