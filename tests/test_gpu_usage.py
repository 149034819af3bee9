"""GPU usage properties of the library beyond elementwise parity.

- FP32 weight: the deterministic dw must be at least as accurate as an
  eager FP32 computation on the same inputs (PR #8848 page, "Measurement":
  with FP32 weight no point exceeds the dw error of FP32 eager).
- The calls are capturable in a HIP graph and every replay equals the eager
  result bit for bit (the library issues kernels only: no allocation, no
  memset, no synchronisation).
- Calls honour the caller's stream.
- Another stream keeping the GPU busy does not change any bit of the result
  (no workgroup ever waits for another: the pages' "stall" concern).
- The backward workspace needs no initialisation: whatever it holds on entry
  (NaN bytes, another call's partials) the results are the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_train_fwd_amd as R
import synth

from helpers import OnGpu, bits, oview, w_f64

pytestmark = pytest.mark.gpu


def _eager_fp32_dw(p: synth.Problem) -> np.ndarray:
    """The plain FP32 computation a framework would run eagerly: FP32 rstd,
    FP32 xhat, FP32 column sum (torch's CPU reduction)."""
    x = p.view(p.x).reshape(-1, p.width).float()
    dy = p.view(p.dy).reshape(-1, p.width).float()
    rstd = torch.rsqrt(x.pow(2).mean(dim=1, keepdim=True) + p.eps)
    return (dy * (x * rstd)).sum(dim=0).double().numpy()


@pytest.mark.parametrize("T,H,family", [(65537, 4096, "normal"), (131072, 2048, "normal"),
                                        (32768, 6144, "spread"), (16384, 512, "cancel")])
def test_det_dw_no_worse_than_fp32_eager(T, H, family):
    p = synth.make(T, H, seed=3, family=family, w_dtype="f32")
    g = OnGpu(p)
    _, rstd = R.rmsnorm_train_fwd(g.x, g.w, p.eps)
    _, dw = R.rmsnorm_train_bwd(g.dy, g.x, rstd, g.w, True)
    _, ref = oracle.bwd(oview(p, p.dy), oview(p, p.x), w_f64(p.w), p.eps, want_rows=False)
    tol = 1e-4 + 1e-4 * np.abs(ref)
    ours = np.max(np.abs(dw.cpu().double().numpy() - ref) / tol)
    eager = np.max(np.abs(_eager_fp32_dw(p) - ref) / tol)
    assert ours <= 1.0
    assert ours <= eager, f"deterministic dw error {ours:.3g} > FP32 eager error {eager:.3g} (x tol)"


@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("T,H,form", [(4099, 4096, "plain"), (100, 512, "plain"),
                                      (777, 6144, "residual"), (300, 4096, "gate")])
def test_graph_replays_match_eager(T, H, form, det):
    p = synth.make(T, H, seed=4, w_dtype="f32", form=form)
    g = OnGpu(p)

    def step():
        if form == "residual":
            y, r, h = R.rmsnorm_train_fwd(g.x, g.w, p.eps, residual=g.e)
            dx, dw = R.rmsnorm_train_bwd(g.dy, h, r, g.w, det, dh=g.dh)
            return [y, r, h, dx, dw]
        if form == "gate":
            y, r = R.rmsnorm_silu_gate_train_fwd(g.x, g.e, g.w, p.eps)
            dx, dz, dw = R.rmsnorm_silu_gate_train_bwd(g.dy, g.x, g.e, r, g.w, det)
            return [y, r, dx, dz, dw]
        y, r = R.rmsnorm_train_fwd(g.x, g.w, p.eps)
        dx, dw = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, det)
        return [y, r, dx, dw]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"


def test_calls_run_on_the_callers_stream():
    p = synth.make(2048, 4096, seed=5, w_dtype="f32")
    g = OnGpu(p)
    y0, r0 = R.rmsnorm_train_fwd(g.x, g.w)
    dx0, dw0 = R.rmsnorm_train_bwd(g.dy, g.x, r0, g.w, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y, r = R.rmsnorm_train_fwd(g.x, g.w)
        dx, dw = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, True)
    s.synchronize()
    assert torch.equal(bits_t(y), bits_t(y0)) and torch.equal(dx.view(torch.int16), dx0.view(torch.int16))
    assert torch.equal(dw, dw0) and torch.equal(r, r0)


def bits_t(t):
    return t.view(torch.int16)


def test_busy_gpu_does_not_change_results():
    # A long matrix product on another stream occupies the CUs while the
    # backward runs; every bit of dx and the deterministic dw must stay.
    p = synth.make(65536, 4096, seed=6, w_dtype="f32")
    g = OnGpu(p)
    _, r = R.rmsnorm_train_fwd(g.x, g.w)
    dx0, dw0 = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, True)
    torch.cuda.synchronize()
    a = torch.randn(8192, 8192, device="cuda")
    other = torch.cuda.Stream()
    with torch.cuda.stream(other):
        for _ in range(4):
            a = a @ a
            a = a / a.abs().max()
    for _ in range(3):
        dx, dw = R.rmsnorm_train_bwd(g.dy, g.x, r, g.w, True)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16))
    assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))
    assert torch.isfinite(a).all()


@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("T,H", [(4099, 4096), (65537, 1536), (3000, 256)])
def test_workspace_contents_on_entry_do_not_matter(T, H, det):
    p = synth.make(T, H, seed=12, w_dtype="f32")
    q = synth.make(T, H, seed=13, w_dtype="f32")
    g, h = OnGpu(p), OnGpu(q)
    _, rstd_p = R.rmsnorm_train_fwd(g.x, g.w, p.eps)
    _, rstd_q = R.rmsnorm_train_fwd(h.x, h.w, q.eps)
    plan = R.rmsnorm_train_bwd_query(g.x, det)
    assert plan.path == R.PATH_LARGE and plan.workspace_bytes > 0
    fresh = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    dx0, dw0 = R.rmsnorm_train_bwd(g.dy, g.x, rstd_p, g.w, det, workspace=fresh)
    nan_bytes = torch.full((plan.workspace_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    dx1, dw1 = R.rmsnorm_train_bwd(g.dy, g.x, rstd_p, g.w, det, workspace=nan_bytes)
    # the same workspace, first used by a call on other inputs
    used = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    R.rmsnorm_train_bwd(h.dy, h.x, rstd_q, h.w, det, workspace=used)
    dx2, dw2 = R.rmsnorm_train_bwd(g.dy, g.x, rstd_p, g.w, det, workspace=used)
    torch.cuda.synchronize()
    for dx, dw in ((dx1, dw1), (dx2, dw2)):
        assert np.array_equal(bits(dx), bits(dx0))
        assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))
