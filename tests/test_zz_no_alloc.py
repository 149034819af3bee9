"""rmsnorm_train_bwd_noalloc (the backward for callers that cannot allocate)
against rmsnorm_train_bwd on the same inputs, called through the C ABI.

Both run the same kernels over the same dw tree, so the deterministic mode
must agree bit for bit; the non-deterministic mode is held to the pages' budget
(dx atol = rtol = 1e-2, dw atol 1e-4 + rtol 1e-4 against the other call's dw).
Two large-path calls run back to back, the second on a smaller input (its
workspace is a smaller part of the same device array, which still holds the
first call's partials), then a small-path call that needs no workspace.
"""
import ctypes as C

import pytest
import torch

import rmsnorm_train_fwd_amd as R

pytestmark = pytest.mark.gpu


def _inputs(T, H, seed, w_dtype, residual):
    g = torch.Generator(device="cuda").manual_seed(seed)
    mk = lambda: torch.randn(T, H, device="cuda", generator=g).to(torch.bfloat16)
    x, dy = mk(), mk()
    dh = mk() if residual else None
    w = (1 + 0.1 * torch.randn(H, device="cuda", generator=g)).to(w_dtype)
    _, rstd = R.rmsnorm_train_fwd(x, w)
    return x, dy, dh, w, rstd


def _noalloc(dy, x, dh, w, rstd, det):
    """The no-allocation entry point, called through ctypes with outputs made here."""
    T, H = x.shape
    L = R.Layout(T, 1, H, H, H, H, H)
    dx = torch.empty_like(x)
    dw = torch.empty(H, dtype=torch.float32, device=x.device)
    wd = R.RMSN_F32 if w.dtype == torch.float32 else R.RMSN_BF16
    st = R.lib().rmsnorm_train_bwd_noalloc(
        dy.data_ptr(), x.data_ptr(), dh.data_ptr() if dh is not None else None, w.data_ptr(), wd,
        rstd.data_ptr(), int(det), C.byref(L), dx.data_ptr(), dw.data_ptr(), R.RMSN_F32, None,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, R.lib().rmsn_status_str(st).decode()
    return dx, dw


def _compare(a, b, det, what):
    (dxa, dwa), (dxb, dwb) = a, b
    if det:
        assert torch.equal(dxa.view(torch.int16), dxb.view(torch.int16)), f"{what}: dx bits"
        assert torch.equal(dwa.view(torch.int32), dwb.view(torch.int32)), f"{what}: dw bits"
    else:
        da, db = dxa.double(), dxb.double()
        assert ((da - db).abs() <= 1e-2 + 1e-2 * db.abs()).all(), f"{what}: dx"
        wa, wb = dwa.double(), dwb.double()
        assert ((wa - wb).abs() <= 1e-4 + 1e-4 * wb.abs()).all(), f"{what}: dw"


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
def test_noalloc_matches_the_workspace_entry_point(det):
    cases = [
        # (T, H, residual, w dtype): workspace 12 MiB (the whole array), then
        # 4 MiB of it on a smaller input, then the small path (none)
        (65537, 6144, False, torch.float32),
        (4099, 2048, True, torch.bfloat16),
        (64, 512, False, torch.float32),
    ]
    for i, (T, H, residual, wdt) in enumerate(cases):
        print(f"[noalloc] det={det} [{T}, {H}] residual={residual}", flush=True)
        x, dy, dh, w, rstd = _inputs(T, H, 100 + i, wdt, residual)
        plan = R.rmsnorm_train_bwd_query(x, det)
        assert plan.workspace_bytes <= 256 * 6144 * 8
        got = _noalloc(dy, x, dh, w, rstd, det)
        ref = R.rmsnorm_train_bwd(dy, x, rstd, w, det, dh=dh)
        again = _noalloc(dy, x, dh, w, rstd, det)    # array reused with its last contents
        torch.cuda.synchronize()
        _compare(got, ref, det, f"[{T}, {H}]")
        _compare(again, ref, det, f"[{T}, {H}] repeated")


def test_noalloc_rejects_what_the_workspace_entry_point_rejects():
    x = torch.zeros(4096, 512, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, device="cuda")
    rstd = torch.ones(4096, device="cuda")
    L = R.Layout(4096, 1, 512, 512, 512, 512, 512)
    lib = R.lib()
    # dw sharing storage with w, and a bad mode flag: refused before any launch
    st = lib.rmsnorm_train_bwd_noalloc(x.data_ptr(), x.data_ptr(), None, w.data_ptr(), R.RMSN_F32,
                                       rstd.data_ptr(), 1, C.byref(L), x.data_ptr() + 0, w.data_ptr(),
                                       R.RMSN_F32, None, None)
    assert st != 0
    dx = torch.empty_like(x)
    dw = torch.empty(512, device="cuda")
    st = lib.rmsnorm_train_bwd_noalloc(x.data_ptr(), x.data_ptr(), None, w.data_ptr(), R.RMSN_F32,
                                       rstd.data_ptr(), 2, C.byref(L), dx.data_ptr(), dw.data_ptr(),
                                       R.RMSN_F32, None, None)
    assert st == 9  # RMSN_E_ARG
    torch.cuda.synchronize()


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
def test_noalloc_inside_a_graph_matches_eager(det):
    # The callers this entry point is for include code under HIP graph
    # capture: the captured call (outputs made before capture, through the C
    # ABI) replays several times, with eager work on the same GPU in between,
    # and every replay equals the eager call bit for bit.
    T, H = 4099, 4096
    x, dy, dh, w, rstd = _inputs(T, H, 7, torch.float32, residual=True)
    L = R.Layout(T, 1, H, H, H, H, H)
    dx = torch.empty_like(x)
    dw = torch.empty(H, dtype=torch.float32, device=x.device)
    ref = R.rmsnorm_train_bwd(dy, x, rstd, w, det, dh=dh)

    def call(stream):
        st = R.lib().rmsnorm_train_bwd_noalloc(
            dy.data_ptr(), x.data_ptr(), dh.data_ptr(), w.data_ptr(), R.RMSN_F32,
            rstd.data_ptr(), int(det), C.byref(L), dx.data_ptr(), dw.data_ptr(), R.RMSN_F32,
            None, stream)
        assert st == 0, R.lib().rmsn_status_str(st).decode()

    call(torch.cuda.current_stream().cuda_stream)      # first call on this device, outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream().cuda_stream)
    for i in range(3):
        dx.zero_()
        dw.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _compare((dx, dw), ref, det, f"replay {i}")    # bits in the deterministic mode
        _ = R.rmsnorm_train_bwd(dy[:2000], x[:2000], rstd[:2000], w, det)   # eager work between
        torch.cuda.synchronize()
