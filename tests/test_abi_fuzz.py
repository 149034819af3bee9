"""Randomised host tests of the C ABI's layout rules and backward plan (no GPU).

The rules come from include/rmsnorm_train.h ("Sizes", "Strides", "Alignment"
and the description of the deterministic tree under rmsnorm_train_bwd); a
small model written from that text decides which rules a drawn layout breaks.
The query (host-only) must then return OK exactly when none is broken, and
otherwise one of the broken rules' codes (the order in which the library
checks them is not part of the contract). On OK the plan must describe the
documented tree and path.
"""
import ctypes as C

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import rmsnorm_train_fwd_amd as R

OK, E_NULL, E_DTYPE, E_SHAPE, E_STRIDE, E_ALIGN, E_ALIAS, E_WS, E_LAUNCH, E_ARG, E_HIP = range(11)
WIDTHS = (256, 512, 1536, 2048, 4096, 5120, 6144)
SUBCHAINS = {256: 16, 512: 8, 1536: 4, 2048: 4, 4096: 2, 5120: 2, 6144: 1}
SMALL_ROWS = {256: 1280, 512: 960, 1536: 640, 2048: 640, 4096: 512, 5120: 512, 6144: 384}
MAX_ROWS = 2**31 - 1
MAX_STRIDE = 2**40


def broken_rules(T, heads, W, pairs):
    """Codes of the header's rules this layout breaks (empty: valid)."""
    bad = set()
    if T < 0 or heads < 1 or W not in WIDTHS:
        return {E_SHAPE}
    if T > MAX_ROWS or heads > MAX_ROWS or T * heads > MAX_ROWS:
        bad.add(E_SHAPE)
    for s_t, s_h in pairs:
        if heads > 1:
            if s_h < W or s_h > MAX_STRIDE:
                bad.add(E_STRIDE)
            elif s_h % 8:
                bad.add(E_ALIGN)
        if T > 1:
            need = (heads - 1) * (s_h if heads > 1 else 0) + W
            if s_t < need or s_t > MAX_STRIDE:
                bad.add(E_STRIDE)
            elif s_t % 8:
                bad.add(E_ALIGN)
        if T > 0:
            last = ((T - 1) * s_t if T > 1 else 0) + ((heads - 1) * s_h if heads > 1 else 0) + W
            if 2 * last > 2**48:
                bad.add(E_SHAPE)
    return bad


def query(T, heads, W, xs, gs, det=1, launch=None):
    L = R.Layout(T, heads, W, xs[0], xs[1], gs[0], gs[1])
    plan = R.BwdPlan()
    rc = R.lib().rmsnorm_train_bwd_query(C.byref(L), det, C.byref(launch) if launch else None,
                                         C.byref(plan))
    return rc, plan


def stride_pair(W, heads):
    # mostly valid strides (padded by multiples of 8), sometimes anything
    valid = st.tuples(st.integers(0, 64), st.integers(0, 64)).map(
        lambda p: (heads * (W + 8 * p[1]) + 8 * p[0], W + 8 * p[1]))
    wild = st.tuples(st.integers(-2**41, 2**41), st.integers(-2**41, 2**41))
    edge = st.tuples(st.sampled_from([0, 1, 7, 8, W - 8, W, W + 1, W + 4, 2**40, 2**40 + 8]),
                     st.sampled_from([0, 8, W - 8, W, W + 3, W + 8, 2**40, 2**40 + 8]))
    return st.one_of(valid, valid, valid, valid, wild, edge)


@st.composite
def layouts(draw):
    # mostly valid sizes, with a share of unsupported or extreme ones
    widths = st.sampled_from(WIDTHS)
    W = draw(st.one_of(widths, widths, widths, widths, st.integers(-8, 8192)))
    hs = st.integers(1, 48)
    heads = draw(st.one_of(hs, hs, hs, st.sampled_from([1, 0, -1, 2**31, 2**20, 2**30 - 1, 2**30])))
    ts = st.integers(0, 200000)
    T = draw(st.one_of(ts, ts, ts, st.sampled_from([-1, 1, 2, 3, 2**24, 2**31 - 1, 2**31, 2**62])))
    Wv = W if W in WIDTHS else 256
    hv = max(1, min(heads, 64))
    xs = draw(stride_pair(Wv, hv))
    gs = draw(st.one_of(st.just(xs), stride_pair(Wv, hv)))
    return T, heads, W, xs, gs


@st.composite
def valid_layouts(draw):
    W = draw(st.sampled_from(WIDTHS))
    heads = draw(st.one_of(st.just(1), st.integers(1, 48)))
    T = draw(st.integers(0, 300000))
    pad = st.integers(0, 64)
    sh = W + 8 * draw(pad) if heads > 1 else W
    xs = (heads * sh + 8 * draw(pad), sh)
    sh2 = W + 8 * draw(pad) if heads > 1 else W
    gs = draw(st.one_of(st.just(xs), st.just((heads * sh2 + 8 * draw(pad), sh2))))
    return T, heads, W, xs, gs


@settings(max_examples=1500, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.one_of(layouts(), valid_layouts()))
def test_query_status_follows_the_header_rules(lay):
    T, heads, W, xs, gs = lay
    rc, plan = query(T, heads, W, xs, gs)
    bad = broken_rules(T, heads, W, [xs, gs])
    if bad:
        assert rc in bad, f"status {rc}, broken rules {sorted(bad)}"
        return
    assert rc == OK, f"status {rc} for a layout that breaks no rule"
    rows = T * heads
    Rr = SUBCHAINS[W]
    tiles = -(-rows // Rr)
    assert plan.rows == rows and plan.subchains == Rr and plan.fold_group == 32
    if rows == 0:
        assert plan.path == R.PATH_SMALL and plan.grid == 0 and plan.workspace_bytes == 0
        return
    if rows <= SMALL_ROWS[W]:
        assert plan.chunks == -(-tiles // 8) and plan.path == R.PATH_SMALL
        assert plan.workspace_bytes == 0
    else:
        assert plan.chunks == min(tiles, 256) and plan.path == R.PATH_LARGE
        assert plan.workspace_bytes == plan.chunks * W * 8
    # the tree depends on the row count and the width only
    other, p2 = query(T, heads, W, xs, gs, det=0, launch=R.Launch(3, 2, R.PATH_LARGE))
    assert other == OK and (p2.chunks, p2.subchains) == (plan.chunks, plan.subchains)
    assert p2.path == R.PATH_LARGE and p2.grid == 3 and p2.fold_grid == 2


@settings(max_examples=600, deadline=None)
@given(st.integers(-2**31, 2**31 - 1), st.integers(-2**31, 2**31 - 1), st.integers(-5, 5),
       st.integers(-3, 3))
def test_query_launch_override_and_flag_rules(grid, fold_grid, path, det):
    launch = R.Launch(grid, fold_grid, path)
    rc, plan = query(1000, 1, 4096, (4096, 4096), (4096, 4096), det=det, launch=launch)
    bad = set()
    if det not in (0, 1):
        bad.add(E_ARG)
    if grid < 0 or fold_grid < 0 or grid > 2**24 or fold_grid > 2**24 or path not in (0, 1, 2):
        bad.add(E_LAUNCH)
    if bad:
        assert rc in bad
        return
    assert rc == OK
    want_path = path if path else R.PATH_LARGE  # 1000 rows at 4096: above the single-launch limit
    assert plan.path == want_path
    if grid:
        assert plan.grid == grid
    if fold_grid:
        assert plan.fold_grid == fold_grid


def test_huge_head_count_with_the_largest_head_stride_is_rejected():
    # (heads - 1) * stride_h exceeds 64 bits here; the check must still
    # reject the layout (the token stride cannot cover the heads) without
    # overflowing.
    W, heads, sh = 256, 2**30 - 1, 2**40
    rc, _ = query(2, heads, W, (2**40, sh), (2**40, sh))
    assert rc == E_STRIDE


# ---------------------------------------------------------------- backward call --
#
# Fake device addresses (never dereferenced: validation runs on the host and a
# call that passes it returns RMSN_E_HIP here, where no GPU is visible). Each
# buffer gets its own 1 MiB-aligned region; a draw may then move an output into
# another buffer's extent, misalign a pointer, or drop it.

def _extent(T, heads, W, s_t, s_h):
    if T == 0:
        return 0
    last = ((T - 1) * s_t if T > 1 else 0) + ((heads - 1) * s_h if heads > 1 else 0) + W
    return 2 * last


def _overlap(a, b):
    (pa, na), (pb, nb) = a, b
    return pa is not None and pb is not None and na > 0 and nb > 0 and pa < pb + nb and pb < pa + na


@st.composite
def bwd_calls(draw):
    T, heads, W, xs, gs = draw(valid_layouts().filter(lambda l: l[0] * l[1] <= 20000))
    form = draw(st.sampled_from(["plain", "residual", "gate"]))
    wd = draw(st.sampled_from([0, 1, 2, 3, 0, 1, 4, -1]))
    dwd = draw(st.sampled_from([0, 1, 0, 1, 2]))
    det = draw(st.sampled_from([0, 1, 0, 1, 2]))
    rows = T * heads
    w_bytes = W * (4 if wd in (1, 3) else 2)
    sizes = {
        "dy": _extent(T, heads, W, *gs), "x": _extent(T, heads, W, *xs),
        "e": (_extent(T, heads, W, *gs) if form == "residual" else _extent(T, heads, W, *xs))
        if form != "plain" else 0,
        "w": w_bytes, "rstd": 4 * rows, "dx": 2 * rows * W,
        "dz": 2 * rows * W if form == "gate" else 0, "dw": W * (4 if dwd == 1 else 2),
    }
    ptr = {k: (1 + i) << 40 for i, k in enumerate(sizes)}
    if form == "plain":
        ptr["e"] = None
    if form != "gate":
        ptr["dz"] = None
    ws_need = None
    rc, plan = query(T, heads, W, xs, gs, det=det if det in (0, 1) else 1)
    ws_need = plan.workspace_bytes if rc == OK else 0
    ws = (20 << 40) if ws_need else None
    ws_bytes = ws_need
    # perturbations
    for _ in range(draw(st.integers(0, 2))):
        kind = draw(st.sampled_from(["null", "misalign", "alias", "ws_small", "ws_null"]))
        key = draw(st.sampled_from(sorted(sizes)))
        if kind == "null" and ptr.get(key) is not None:
            ptr[key] = None
        elif kind == "misalign" and ptr.get(key) is not None:
            ptr[key] += draw(st.sampled_from([2, 4, 8]))
        elif kind == "alias":
            out = draw(st.sampled_from(["dx", "dz", "dw"]))
            if ptr.get(out) is not None and ptr.get(key) is not None and sizes[key] > 0:
                ptr[out] = ptr[key] + 16 * draw(st.integers(0, max(0, sizes[key] // 16 - 1)))
        elif kind == "ws_small" and ws_need:
            ws_bytes = draw(st.integers(0, ws_need - 1))
        elif kind == "ws_null" and ws_need:
            ws = None
    return dict(T=T, heads=heads, W=W, xs=xs, gs=gs, form=form, wd=wd, dwd=dwd, det=det,
                sizes=sizes, ptr=ptr, ws=ws, ws_bytes=ws_bytes, ws_need=ws_need)


def bwd_broken_rules(c):
    """Codes of the header rules a backward call breaks (the layout is valid)."""
    bad = set()
    p, n = c["ptr"], c["sizes"]
    rows = c["T"] * c["heads"]
    gate = c["form"] == "gate"
    if c["wd"] not in (0, 1, 2, 3) or c["dwd"] not in (0, 1):
        bad.add(E_DTYPE)
    if c["det"] not in (0, 1):
        bad.add(E_ARG)
    if p["w"] is None or p["dw"] is None:
        bad.add(E_NULL)
    if rows > 0:
        if any(p[k] is None for k in ("dy", "x", "rstd", "dx")):
            bad.add(E_NULL)
        if gate and (p["e"] is None or p["dz"] is None):
            bad.add(E_NULL)
        if c["form"] == "residual" and p["e"] is None:
            pass  # dh NULL selects the plain form: no rule broken by itself
    al16 = [k for k in ("w", "dw") if p[k] is not None and p[k] % 16]
    if rows > 0:
        al16 += [k for k in ("dy", "x", "dx", "e", "dz") if p.get(k) is not None and p[k] % 16]
        if p["rstd"] is not None and p["rstd"] % 4:
            al16.append("rstd")
    if al16:
        bad.add(E_ALIGN)
    if c["ws_need"]:
        if c["ws"] is None or c["ws_bytes"] < c["ws_need"]:
            bad.add(E_WS)
    # overlaps: outputs against inputs and each other
    ins = [(p[k], n[k]) for k in ("dy", "x", "e", "w", "rstd")]
    outs = [(p[k], n[k]) for k in ("dx", "dz", "dw")] + [(c["ws"], c["ws_need"] if c["ws"] else 0)]
    for i, o in enumerate(outs):
        if any(_overlap(o, b) for b in ins) or any(_overlap(o, b) for j, b in enumerate(outs) if j != i):
            bad.add(E_ALIAS)
    return bad


@settings(max_examples=800, deadline=None, suppress_health_check=[HealthCheck.too_slow,
                                                                   HealthCheck.filter_too_much])
@given(bwd_calls())
def test_bwd_call_status_follows_the_header_rules(c):
    import torch
    if torch.cuda.is_available():
        return  # a valid call would launch on fake addresses
    p = c["ptr"]
    L = R.Layout(c["T"], c["heads"], c["W"], c["xs"][0], c["xs"][1], c["gs"][0], c["gs"][1])
    args = (p["dy"], p["x"])
    if c["form"] == "gate":
        rc = R.lib().rmsnorm_silu_gate_train_bwd(p["dy"], p["x"], p["e"], p["w"], c["wd"], p["rstd"],
                                                  c["det"], C.byref(L), p["dx"], p["dz"], p["dw"],
                                                  c["dwd"], c["ws"], c["ws_bytes"], None, None)
    else:
        dh = p["e"] if c["form"] == "residual" else None
        rc = R.lib().rmsnorm_train_bwd(*args, dh, p["w"], c["wd"], p["rstd"], c["det"], C.byref(L),
                                       p["dx"], p["dw"], c["dwd"], c["ws"], c["ws_bytes"], None,
                                       None)
    bad = bwd_broken_rules(c)
    if bad:
        assert rc in bad, f"status {rc}, broken rules {sorted(bad)}"
    else:
        assert rc == E_HIP, f"status {rc} for a call that breaks no rule"


# ----------------------------------------------------------------- forward call --

@st.composite
def fwd_calls(draw):
    T, heads, W, xs, _ = draw(valid_layouts().filter(lambda l: l[0] * l[1] <= 20000))
    form = draw(st.sampled_from(["plain", "residual", "gate"]))
    wd = draw(st.sampled_from([0, 1, 2, 3, 0, 1, 5]))
    eps = draw(st.sampled_from([1e-6, 0.0, 1e-5, -1e-6, float("nan"), float("inf")]))
    rows = T * heads
    sizes = {"x": _extent(T, heads, W, *xs), "e": _extent(T, heads, W, *xs) if form != "plain" else 0,
             "w": W * (4 if wd in (1, 3) else 2), "y": 2 * rows * W,
             "h": 2 * rows * W if form == "residual" else 0, "rstd": 4 * rows}
    ptr = {k: (1 + i) << 40 for i, k in enumerate(sizes)}
    if form == "plain":
        ptr["e"] = None
    if form != "residual":
        ptr["h"] = None
    if form == "plain" and draw(st.integers(0, 9)) == 0:
        ptr["h"] = 7 << 40  # h_out without a residual
    for _ in range(draw(st.integers(0, 2))):
        kind = draw(st.sampled_from(["null", "misalign", "alias"]))
        key = draw(st.sampled_from(sorted(sizes)))
        if kind == "null" and ptr.get(key) is not None:
            ptr[key] = None
        elif kind == "misalign" and ptr.get(key) is not None:
            ptr[key] += draw(st.sampled_from([2, 4, 8]))
        elif kind == "alias":
            out = draw(st.sampled_from(["y", "h", "rstd"]))
            if ptr.get(out) is not None and ptr.get(key) is not None and sizes[key] > 0:
                ptr[out] = ptr[key] + 16 * draw(st.integers(0, max(0, sizes[key] // 16 - 1)))
    return dict(T=T, heads=heads, W=W, xs=xs, form=form, wd=wd, eps=eps, sizes=sizes, ptr=ptr)


def fwd_broken_rules(c):
    bad = set()
    p, n = c["ptr"], c["sizes"]
    rows = c["T"] * c["heads"]
    gate = c["form"] == "gate"
    if c["wd"] not in (0, 1, 2, 3):
        bad.add(E_DTYPE)
    if not (c["eps"] >= 0.0 and c["eps"] != float("inf")):
        bad.add(E_ARG)
    # the plain and residual forms are one entry point: residual == NULL selects plain
    residual = not gate and p["e"] is not None
    if not gate and not residual and p["h"] is not None:
        bad.add(E_ARG)  # h_out only with a residual
    if p["w"] is None:
        bad.add(E_NULL)
    if rows > 0:
        if any(p[k] is None for k in ("x", "y", "rstd")) or (gate and p["e"] is None):
            bad.add(E_NULL)
        if residual and p["h"] is None:
            bad.add(E_NULL)
    mis = p["w"] is not None and p["w"] % 16
    if rows > 0:
        mis = mis or any(p.get(k) is not None and p[k] % 16 for k in ("x", "y", "e", "h"))
        mis = mis or (p["rstd"] is not None and p["rstd"] % 4)
    if mis:
        bad.add(E_ALIGN)
    ins = [(p[k], n[k]) for k in ("x", "e", "w")]
    outs = [(p[k], n[k]) for k in ("y", "h", "rstd")]
    for i, o in enumerate(outs):
        if any(_overlap(o, b) for b in ins) or any(_overlap(o, b) for j, b in enumerate(outs) if j != i):
            bad.add(E_ALIAS)
    return bad


@settings(max_examples=800, deadline=None, suppress_health_check=[HealthCheck.too_slow,
                                                                   HealthCheck.filter_too_much])
@given(fwd_calls())
def test_fwd_call_status_follows_the_header_rules(c):
    import torch
    if torch.cuda.is_available():
        return  # a valid call would launch on fake addresses
    p = c["ptr"]
    L = R.Layout(c["T"], c["heads"], c["W"], c["xs"][0], c["xs"][1], c["xs"][0], c["xs"][1])
    if c["form"] == "gate":
        rc = R.lib().rmsnorm_silu_gate_train_fwd(p["x"], p["e"], p["w"], c["wd"], c["eps"],
                                                  C.byref(L), p["y"], p["rstd"], None)
    else:
        rc = R.lib().rmsnorm_train_fwd(p["x"], p["e"], p["w"], c["wd"], c["eps"], C.byref(L),
                                       p["y"], p["h"], p["rstd"], None)
    bad = fwd_broken_rules(c)
    rows = c["T"] * c["heads"]
    if bad:
        assert rc in bad, f"status {rc}, broken rules {sorted(bad)}"
    elif rows == 0:
        assert rc == OK  # nothing to enqueue
    else:
        assert rc == E_HIP, f"status {rc} for a call that breaks no rule"
