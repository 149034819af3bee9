"""The Python binding refuses calls that the kernels could not run safely:
tensors off the GPU or on another device than x, wrong dtypes or shapes, a
non-contiguous workspace. Every refusal happens in Python before the library
is called, so nothing is launched (the GPU cases only need tensors that live
on a GPU)."""
import pytest
import torch

import rmsnorm_train_fwd_amd as R


def test_cpu_tensors_raise_without_a_cpu_path():
    x = torch.zeros(4, 512, dtype=torch.bfloat16)
    w = torch.ones(512)
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        R.rmsnorm_train_fwd(x, w)
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        R.rmsnorm_silu_gate_train_fwd(x, x, w)
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        R.rmsnorm_train_bwd(x, x, torch.ones(4), w, True)
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        R.rmsnorm_silu_gate_train_bwd(x, x, x, torch.ones(4), w, True)


@pytest.mark.gpu
def test_mixed_devices_and_bad_arguments_are_refused():
    dev = torch.device("cuda:0")
    x = torch.randn(64, 512, device=dev).to(torch.bfloat16)
    w = torch.ones(512, device=dev)
    y, rstd = R.rmsnorm_train_fwd(x, w)
    torch.cuda.synchronize()
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="same GPU"):
        R.rmsnorm_train_fwd(x, w.to(cpu))
    with pytest.raises(ValueError, match="same GPU"):
        R.rmsnorm_train_fwd(x, w, residual=x.to(cpu))
    with pytest.raises(ValueError, match="same GPU"):
        R.rmsnorm_silu_gate_train_fwd(x, x.to(cpu), w)
    with pytest.raises(ValueError, match="same GPU"):
        R.rmsnorm_train_bwd(x, x, rstd.to(cpu), w, True)
    with pytest.raises(ValueError, match="same GPU"):
        R.rmsnorm_train_bwd(x, x, rstd, w, True, dh=x.to(cpu))
    with pytest.raises(ValueError, match="same GPU"):
        R.rmsnorm_silu_gate_train_bwd(x, x, x, rstd, w.to(cpu), True)
    with pytest.raises(TypeError):
        R.rmsnorm_train_fwd(x.float(), w)
    with pytest.raises(ValueError, match="rstd"):
        R.rmsnorm_train_bwd(x, x, rstd.double(), w, True)
    with pytest.raises(ValueError, match="w must be"):
        R.rmsnorm_train_fwd(x, w[:256])
    big = R.rmsnorm_train_bwd_query(torch.empty(4096, 512, dtype=torch.bfloat16, device=dev), False)
    assert big.workspace_bytes > 0
    xb = torch.randn(4096, 512, device=dev).to(torch.bfloat16)
    _, rb = R.rmsnorm_train_fwd(xb, w)
    ws = torch.empty(2 * big.workspace_bytes, dtype=torch.uint8, device=dev)[::2]
    with pytest.raises(ValueError, match="workspace"):
        R.rmsnorm_train_bwd(xb, xb, rb, w, False, workspace=ws)
    torch.cuda.synchronize()


def test_last_dim_strided_companion_tensors_are_refused():
    # residual, z and dh are read with the strides of x (or dy) as rows of
    # 16-byte vectors; a view whose last dimension is strided must be refused
    # before anything is called (the check runs before the device check, so
    # CPU tensors reach it).
    x = torch.zeros(8, 512, dtype=torch.bfloat16)
    w = torch.ones(512)
    rstd = torch.ones(8)
    strided = torch.zeros(8, 1024, dtype=torch.bfloat16)[:, ::2]     # strides (1024, 2)
    assert strided.shape == x.shape and strided.stride(-1) == 2
    with pytest.raises(ValueError, match="residual: the last dimension"):
        R.rmsnorm_train_fwd(x, w, residual=strided)
    with pytest.raises(ValueError, match="z: the last dimension"):
        R.rmsnorm_silu_gate_train_fwd(x, strided, w)
    with pytest.raises(ValueError, match="z: the last dimension"):
        R.rmsnorm_silu_gate_train_bwd(x, x, strided, rstd, w, True)
    with pytest.raises(ValueError, match="dh: the last dimension"):
        R.rmsnorm_train_bwd(x, x, rstd, w, True, dh=strided)
    # per-head [T, 24, 256] views with a strided last dimension
    xh = torch.zeros(4, 24, 256, dtype=torch.bfloat16)
    sh = torch.zeros(4, 24, 512, dtype=torch.bfloat16)[:, :, ::2]
    with pytest.raises(ValueError, match="residual: the last dimension"):
        R.rmsnorm_train_fwd(xh, torch.ones(256), residual=sh)
    with pytest.raises(ValueError, match="x: the last dimension"):
        R.rmsnorm_train_fwd(sh, torch.ones(256))
    # companion tensors with the right inner stride but other token strides
    other = torch.zeros(8, 1024, dtype=torch.bfloat16)[:, :512]
    with pytest.raises(ValueError, match="shape and strides"):
        R.rmsnorm_train_fwd(x, w, residual=other)
    # well-formed CPU tensors pass every metadata check and stop at the device
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        R.rmsnorm_train_fwd(x, w, residual=x.clone())
