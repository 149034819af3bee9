"""Host-only tests of the C ABI (no GPU needed).

The library must load, export every function include/rmsnorm_train.h
declares, and reject every malformed call before touching the GPU: the
checks run on the host and never dereference device pointers, so fake
pointer values exercise them here. Also covers the backward plan: the
canonical chunking of the deterministic dw tree, the path choice and the
workspace size.
"""
import ctypes as C
import os
import re

import pytest

import rmsnorm_train_fwd_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm_train.h")

OK, E_NULL, E_DTYPE, E_SHAPE, E_STRIDE, E_ALIGN, E_ALIAS, E_WS, E_LAUNCH, E_ARG, E_HIP = range(11)
MB = 1 << 20


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = R.lib()
    names = declared_functions()
    assert set(names) == set(R.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"


def test_status_strings():
    lib = R.lib()
    for code in range(11):
        assert lib.rmsn_status_str(code)
    assert lib.rmsn_status_str(99) == b"unknown status"


def lay(T, W, heads=1, st=None, sh=None, gst=None, gsh=None):
    sh = W if sh is None else sh
    st = heads * sh if st is None else st
    return R.Layout(T, heads, W, st, sh, st if gst is None else gst, sh if gsh is None else gsh)


class Bufs:
    """Disjoint fake device addresses, 16-byte aligned."""

    def __init__(self):
        self.next = 1 << 32

    def __call__(self, nbytes):
        a = self.next
        self.next += ((nbytes + 4095) // 4096 + 1) * 4096
        return a


def fwd(L, x, res, w, y, h, rstd, wd=R.RMSN_F32, eps=1e-6):
    return R.lib().rmsnorm_train_fwd(x, res, w, wd, eps, C.byref(L) if L else None, y, h, rstd, None)


def bwd(L, dy, x, dh, w, rstd, dx, dw, ws=None, wsb=0, det=1, wd=R.RMSN_F32, launch=None,
        dwd=R.RMSN_F32):
    return R.lib().rmsnorm_train_bwd(dy, x, dh, w, wd, rstd, det, C.byref(L) if L else None, dx,
                                     dw, dwd, ws, wsb, C.byref(launch) if launch else None, None)


def gpu_visible():
    import torch
    return torch.cuda.is_available()


def setup_fwd(T=8, W=512):
    b = Bufs()
    n = T * W * 2
    return dict(x=b(n), res=b(n), w=b(W * 4), y=b(n), h=b(n), rstd=b(T * 4))


def test_fwd_validation_errors():
    L = lay(8, 512)
    a = setup_fwd()
    assert fwd(None, a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_NULL
    assert fwd(L, None, None, a["w"], a["y"], None, a["rstd"]) == E_NULL
    assert fwd(L, a["x"], None, None, a["y"], None, a["rstd"]) == E_NULL
    assert fwd(L, a["x"], None, a["w"], None, None, a["rstd"]) == E_NULL
    assert fwd(L, a["x"], None, a["w"], a["y"], None, None) == E_NULL
    assert fwd(L, a["x"], a["res"], a["w"], a["y"], None, a["rstd"]) == E_NULL  # residual w/o h_out
    assert fwd(L, a["x"], None, a["w"], a["y"], a["h"], a["rstd"]) == E_ARG     # h_out w/o residual
    assert fwd(L, a["x"], None, a["w"], a["y"], None, a["rstd"], wd=7) == E_DTYPE
    assert fwd(L, a["x"], None, a["w"], a["y"], None, a["rstd"], wd=4) == E_DTYPE
    if not gpu_visible():  # both zero-centred codes pass validation
        for wd in (R.RMSN_BF16_ZERO_CENTRED, R.RMSN_F32_ZERO_CENTRED):
            assert fwd(L, a["x"], None, a["w"], a["y"], None, a["rstd"], wd=wd) == E_HIP
    for eps in (float("nan"), float("inf"), -1e-6):
        assert fwd(L, a["x"], None, a["w"], a["y"], None, a["rstd"], eps=eps) == E_ARG
    for W in (0, 128, 1000, 4097, 8192):
        assert fwd(lay(8, W), a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_SHAPE
    assert fwd(R.Layout(-1, 1, 512, 512, 512, 512, 512), a["x"], None, a["w"], a["y"], None,
               a["rstd"]) == E_SHAPE
    assert fwd(R.Layout(8, 0, 512, 512, 512, 512, 512), a["x"], None, a["w"], a["y"], None,
               a["rstd"]) == E_SHAPE
    assert fwd(R.Layout(1 << 31, 1, 512, 512, 512, 512, 512), a["x"], None, a["w"], a["y"], None,
               a["rstd"]) == E_SHAPE
    # misaligned pointers
    assert fwd(L, a["x"] + 2, None, a["w"], a["y"], None, a["rstd"]) == E_ALIGN
    assert fwd(L, a["x"], None, a["w"] + 4, a["y"], None, a["rstd"]) == E_ALIGN
    assert fwd(L, a["x"], None, a["w"], a["y"] + 8, None, a["rstd"]) == E_ALIGN
    assert fwd(L, a["x"], None, a["w"], a["y"], None, a["rstd"] + 2) == E_ALIGN
    # aliasing: output over input, output over output
    assert fwd(L, a["x"], None, a["w"], a["x"], None, a["rstd"]) == E_ALIAS
    assert fwd(L, a["x"], None, a["w"], a["y"], None, a["y"] + 512) == E_ALIAS
    assert fwd(L, a["x"], a["res"], a["w"], a["y"], a["res"], a["rstd"]) == E_ALIAS
    assert fwd(L, a["x"], None, a["w"], a["y"], None, a["w"] + 16) == E_ALIAS


def test_stride_validation():
    a = setup_fwd(T=4, W=256)
    # per-head rows must not overlap: head stride >= width, token stride covers all heads
    assert fwd(lay(4, 256, heads=24, sh=128), a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_STRIDE
    assert fwd(lay(4, 256, heads=24, sh=256, st=256 * 23), a["x"], None, a["w"], a["y"], None,
               a["rstd"]) == E_STRIDE
    assert fwd(lay(4, 256, heads=24, sh=260), a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_ALIGN
    assert fwd(lay(4, 512, st=516), a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_ALIGN
    assert fwd(lay(4, 512, st=-512), a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_STRIDE
    # strides are ignored where they are unused (T == 1; heads == 1): the call gets
    # past the layout checks to the (deliberately misaligned) output, so nothing
    # is launched with these fake addresses
    assert fwd(lay(1, 512, st=3), a["x"], None, a["w"], a["y"] + 8, None, a["rstd"]) == E_ALIGN
    # a view whose byte extent exceeds the address space (T * stride_t would
    # overflow 64-bit arithmetic) is rejected, not wrapped around
    huge = R.Layout((1 << 31) - 1, 1, 512, 1 << 40, 512, 1 << 40, 512)
    assert fwd(huge, a["x"], None, a["w"], a["y"], None, a["rstd"]) == E_SHAPE


def setup_bwd(T=8, W=512):
    b = Bufs()
    n = T * W * 2
    return dict(dy=b(n), x=b(n), dh=b(n), w=b(W * 4), rstd=b(T * 4), dx=b(n), dw=b(W * 4),
                ws=b(64 * MB))


def test_bwd_validation_errors():
    L = lay(8, 512)
    a = setup_bwd()
    args = lambda **kw: {**dict(L=L, dy=a["dy"], x=a["x"], dh=None, w=a["w"], rstd=a["rstd"],
                                dx=a["dx"], dw=a["dw"]), **kw}
    assert bwd(**args(L=None)) == E_NULL
    for k in ("dy", "x", "w", "rstd", "dx", "dw"):
        assert bwd(**args(**{k: None})) == E_NULL, k
    assert bwd(**args(det=2)) == E_ARG
    assert bwd(**args(wd=5)) == E_DTYPE
    assert bwd(**args(wd=4)) == E_DTYPE
    assert bwd(**args(wd=-1)) == E_DTYPE
    assert bwd(**args(dwd=2)) == E_DTYPE               # dw is FP32 or BF16
    assert bwd(**args(dwd=R.RMSN_F32_ZERO_CENTRED)) == E_DTYPE
    # the zero-centred weight codes keep their storage size: a dw right after a
    # BF16 w's 512 elements touches a FP32 w's extent only
    W = 512
    assert bwd(**args(dw=a["w"] + 2 * W, wd=R.RMSN_F32_ZERO_CENTRED)) == E_ALIAS
    if not gpu_visible():
        assert bwd(**args(dw=a["w"] + 2 * W, wd=R.RMSN_BF16_ZERO_CENTRED)) == E_HIP
        assert bwd(**args(wd=R.RMSN_F32_ZERO_CENTRED)) == E_HIP
    # the dw extent follows its dtype: 512 FP32 values starting 1 KiB below rstd
    # reach into rstd, 512 BF16 values end exactly at it
    assert bwd(**args(dw=a["rstd"] - 1024)) == E_ALIAS
    if not gpu_visible():  # a call that passes validation must not launch on fake addresses
        assert bwd(**args(dw=a["rstd"] - 1024, dwd=R.RMSN_BF16)) == E_HIP
    assert bwd(**args(dw=a["w"])) == E_ALIAS          # dw sharing storage with w is rejected
    assert bwd(**args(dw=a["w"] + 1024)) == E_ALIAS
    assert bwd(**args(dx=a["dy"])) == E_ALIAS
    assert bwd(**args(dx=a["x"] + 4096)) == E_ALIAS
    assert bwd(**args(dw=a["dx"])) == E_ALIAS
    assert bwd(**args(dw=a["rstd"])) == E_ALIAS
    assert bwd(**args(dx=a["dx"] + 8)) == E_ALIGN
    assert bwd(**args(dw=a["dw"] + 4)) == E_ALIGN
    # launch override: non-negative 1-D counts, known paths only
    for bad in (R.Launch(-1, 0, 0), R.Launch(0, -3, 0), R.Launch(0, 0, 3), R.Launch(1 << 25, 0, 0)):
        assert bwd(**args(launch=bad)) == E_LAUNCH


def test_bwd_workspace_rules():
    T, W = 4096, 4096
    a = setup_bwd(T, W)
    L = lay(T, W)
    plan = R.BwdPlan()
    assert R.lib().rmsnorm_train_bwd_query(C.byref(L), 1, None, C.byref(plan)) == OK
    assert plan.path == R.PATH_LARGE and plan.workspace_bytes == plan.chunks * W * 8
    base = dict(L=L, dy=a["dy"], x=a["x"], dh=None, w=a["w"], rstd=a["rstd"], dx=a["dx"], dw=a["dw"])
    assert bwd(**base, ws=None, wsb=0) == E_WS
    assert bwd(**base, ws=a["ws"], wsb=plan.workspace_bytes - 1) == E_WS
    assert bwd(**base, ws=a["ws"] + 8, wsb=plan.workspace_bytes) == E_ALIGN
    assert bwd(**base, ws=a["dx"], wsb=plan.workspace_bytes) == E_ALIAS   # workspace over dx
    assert bwd(**base, ws=a["x"], wsb=plan.workspace_bytes) == E_ALIAS


def query(T, W, heads=1, det=1, launch=None):
    plan = R.BwdPlan()
    L = lay(T, W, heads=heads)
    rc = R.lib().rmsnorm_train_bwd_query(C.byref(L), det, C.byref(launch) if launch else None,
                                         C.byref(plan))
    assert rc == OK
    return plan


SUBCHAINS = {256: 16, 512: 8, 1536: 4, 2048: 4, 4096: 2, 5120: 2, 6144: 1}
SMALL_ROWS = {256: 1280, 512: 960, 1536: 640, 2048: 640, 4096: 512, 5120: 512, 6144: 384}


@pytest.mark.parametrize("W", [256, 512, 1536, 2048, 4096, 5120, 6144])
@pytest.mark.parametrize("rows", [1, 15, 16, 17, 203, 256, 257, 300, 384, 385, 512, 513, 640, 641, 768, 769,
                                  960, 961, 1024, 1025, 1280, 1281, 2048, 2049, 16384, 16385, 65537, 98304, 131072,
                                  113536, 786432, 3145728])
def test_dw_tree_chunking(rows, W):
    p = query(rows, W)
    assert p.subchains == SUBCHAINS[W] and p.fold_group == 32
    tiles = -(-rows // p.subchains)
    assert 1 <= p.chunks <= tiles          # every chunk holds at least one tile
    if rows <= SMALL_ROWS[W]:
        # as few chunks as hold at most 8 tiles each; at most two fold groups
        assert p.chunks == -(-tiles // 8) and p.chunks <= 64
        assert p.path == R.PATH_SMALL and p.workspace_bytes == 0
    else:
        # one chunk per workgroup a 256-CU part holds at once (one per CU)
        assert p.chunks == min(tiles, 256)
        assert p.path == R.PATH_LARGE
    # the tree depends on the row count and the width only: not on the mode,
    # the grid or the path
    for other in (query(rows, W, det=0), query(rows, W, launch=R.Launch(5, 2, R.PATH_LARGE)),
                  query(rows, W, launch=R.Launch(3, 1, R.PATH_SMALL))):
        assert (other.chunks, other.subchains) == (p.chunks, p.subchains)


def test_plan_headline_and_paths():
    p = query(131072, 4096)
    assert (p.chunks, p.subchains, p.fold_group) == (256, 2, 32)
    assert p.workspace_bytes == 256 * 4096 * 8 and p.grid == 256 and p.fold_grid == 128
    s = query(8, 512)
    assert s.path == R.PATH_SMALL and s.workspace_bytes == 0 and s.subchains == 8
    assert query(4, 256, heads=24).subchains == 16
    z = query(0, 6144)
    assert z.path == R.PATH_SMALL and z.grid == 0 and z.workspace_bytes == 0
    forced = query(100, 2048, launch=R.Launch(0, 0, R.PATH_LARGE))
    assert forced.path == R.PATH_LARGE and forced.workspace_bytes == forced.chunks * 2048 * 8


def test_bandwidth_probe_library_loads_and_rejects_bad_arguments():
    # The probe that bench.py times beside the kernels (a separate library, not
    # part of the normalisation ABI). Only argument errors are exercised here:
    # they return before any HIP call, so nothing launches.
    path = os.path.join(ROOT, "probe", "librmsn_probe.so")
    f = C.CDLL(path).rmsn_stream_probe
    f.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int,
                  C.c_void_p]
    f.restype = C.c_int
    invalid = 1  # hipErrorInvalidValue
    a, b, o = 1 << 20, 2 << 20, 3 << 20  # 16-byte aligned stand-ins, never dereferenced
    tile = 16 << 10
    assert f(3, 0, a, b, o, tile, 256, None) == invalid       # nin out of range
    assert f(2, 3, a, b, o, tile, 256, None) == invalid       # pattern out of range
    assert f(2, 0, a, None, o, tile, 256, None) == invalid    # two inputs need b
    assert f(1, 0, a, None, None, tile, 256, None) == invalid  # no output
    assert f(1, 0, a, None, o, tile + 16, 256, None) == invalid  # not whole 16 KiB tiles
    assert f(1, 0, a, None, o, 0, 256, None) == invalid       # empty
    assert f(1, 0, a, None, o, tile, 0, None) == invalid      # no workgroups
    assert f(1, 0, a + 8, None, o, tile, 256, None) == invalid  # misaligned


@pytest.mark.gpu
def test_pending_unrelated_hip_error_does_not_fail_a_good_call():
    # An earlier, unrelated HIP error left in the thread's last-error state
    # (here: hipSetDevice on a device index that does not exist, a pure argument
    # error) must not turn a valid call into RMSN_E_HIP: each call reports the
    # status of its own launches and leaves that state to the caller.
    import torch

    hip = C.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [C.c_int]
    hip.hipGetLastError.restype = C.c_int
    x = torch.randn(64, 512, device="cuda").to(torch.bfloat16)
    xl = torch.cat([x] * 64)                       # 4096 rows: the large path + fold
    w = torch.ones(512, device="cuda")
    _, rstd_l = R.rmsnorm_train_fwd(xl, w)
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0
    # No torch kernel may run while the error is pending (torch checks the
    # last-error state after its own launches); the binding's calls only
    # allocate and call the library.
    assert hip.hipSetDevice(1 << 20) != 0          # leaves an error pending on this thread
    try:
        y, rstd = R.rmsnorm_train_fwd(x, w)        # raises RmsnError on any non-OK status
        dx, dw = R.rmsnorm_train_bwd(x, x, rstd, w, True)
        dxl, dwl = R.rmsnorm_train_bwd(xl, xl, rstd_l, w, False)
    finally:
        hip.hipGetLastError()                      # clear it, so later torch calls do not see it
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(dw).all()
    assert torch.isfinite(dwl).all()
