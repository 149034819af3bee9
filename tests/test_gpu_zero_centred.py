"""Zero-centred-weight RMSNorm on the GPU (the related-PR title "zero-centred
input RMSNorm" on the PR #8512 page, read as the RMSNorm whose stored weight is
centred on zero and used as 1 + w).

Parity: every form and mode against the FP64 oracle given the effective weight
1 + w, under the pages' budget. Identity: a zero-centred call equals, bit for
bit, the plain call given the FP32 weight 1 + w rounded once (torch's FP32 add
rounds to nearest even, as the kernels do when they load the weight).
"""
import pytest
import torch

import rmsnorm_train_fwd_amd as R
import synth

from test_gpu_parity import run_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [
    ("plain", 8, 512, 1), ("plain", 4099, 4096, 1), ("plain", 64, 256, 24),
    ("plain", 4096, 256, 24), ("residual", 777, 6144, 1), ("residual", 32, 6144, 1),
    ("gate", 3534, 4096, 1), ("gate", 300, 256, 48),
], ids=lambda c: f"{c[0]}-{c[1]}x{c[3]}x{c[2]}")
def test_zero_centred_parity(case, w_dtype):
    form, T, W, heads = case
    print(f"[zero-centred] {form} [{T},{heads},{W}] w {w_dtype}", flush=True)
    p = synth.make(T, W, seed=11, heads=heads, w_dtype=w_dtype, form=form, w_centre=0.0)
    run_case(p, det=(False, True), form=form, zero_centred=True,
             nsample=48 if T * heads > 4096 else None)


@pytest.mark.parametrize("w_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("form", ["plain", "residual", "gate"])
def test_zero_centred_equals_plain_with_one_plus_w(form, w_dtype):
    T, W = 1000, 2048
    g = torch.Generator(device="cuda").manual_seed(5)
    mk = lambda: torch.randn(T, W, device="cuda", generator=g).to(torch.bfloat16)
    x, dy, e, dh = mk(), mk(), mk(), mk()
    w = (0.1 * torch.randn(W, device="cuda", generator=g)).to(w_dtype)
    w_plus = 1.0 + w.float()                       # FP32, rounded once
    outs = []
    for weight, zc in ((w, True), (w_plus, False)):
        if form == "residual":
            y, rstd, h = R.rmsnorm_train_fwd(x, weight, residual=e, zero_centred=zc)
            res = [y, rstd, h]
            for det in (True, False):
                res += list(R.rmsnorm_train_bwd(dy, h, rstd, weight, det, dh=dh, zero_centred=zc))
        elif form == "gate":
            y, rstd = R.rmsnorm_silu_gate_train_fwd(x, e, weight, zero_centred=zc)
            res = [y, rstd]
            for det in (True, False):
                res += list(R.rmsnorm_silu_gate_train_bwd(dy, x, e, rstd, weight, det,
                                                          zero_centred=zc))
        else:
            y, rstd = R.rmsnorm_train_fwd(x, weight, zero_centred=zc)
            res = [y, rstd]
            for det in (True, False):
                res += list(R.rmsnorm_train_bwd(dy, x, rstd, weight, det, zero_centred=zc))
        outs.append(res)
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert a.dtype == b.dtype and torch.equal(a.view(torch.uint8), b.view(torch.uint8))
