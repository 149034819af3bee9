"""Pins of the FP64 CPU oracle to facts other than itself (CPU only).

Every check here would catch a plausible slip in oracle/rmsn_oracle.c: a
dropped term, a wrong sign, width-1 instead of width, eps outside the root, a
wrong rounding rule, a transposed operand. The references are closed forms,
complex-step and central finite-difference derivatives of the forward (which
tie the backward to the forward), the scale-invariance identity, exact (fsum)
summation, the IEEE round-to-nearest-even definition evaluated with exact
rationals, and torch's CPU BF16 casts.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

EPS = 1e-6


# ---------------------------------------------------------------- formats ---

def _bf16_bits_torch(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_to_f64_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def _rne_bf16_exact(d: float) -> int:
    """Brute-force IEEE round-to-nearest-even of a finite double to BF16,
    over exact rationals: scan every candidate neighbour."""
    if d == 0.0:
        return 0x8000 if math.copysign(1.0, d) < 0 else 0
    sign = 0x8000 if d < 0 else 0
    a = Fraction(abs(d))
    # candidates: all finite non-negative BF16 values bracketing a
    best = None
    lo, hi = 0, 0x7F7F
    while lo < hi:  # largest finite bf16 <= a (values increase with bit pattern)
        mid = (lo + hi + 1) // 2
        v = Fraction(struct.unpack("<f", struct.pack("<I", mid << 16))[0])
        if v <= a:
            lo = mid
        else:
            hi = mid - 1
    below = lo
    vb = Fraction(struct.unpack("<f", struct.pack("<I", below << 16))[0])
    if vb == a:
        return sign | below
    above = below + 1  # 0x7F80 (inf) when below is the largest finite value
    if above == 0x7F80:
        # overflow threshold: max + half ulp rounds to inf (ties to even -> inf)
        half = Fraction(2) ** 127 * Fraction(2) ** -8
        return sign | (0x7F80 if a >= vb + half else below)
    va = Fraction(struct.unpack("<f", struct.pack("<I", above << 16))[0])
    if a - vb < va - a:
        best = below
    elif a - vb > va - a:
        best = above
    else:
        best = below if below % 2 == 0 else above
    return sign | best


def test_bf16_rounding_matches_exact_rne_definition():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(400) * 10.0 ** rng.integers(-40, 39, 400))
    vals += [1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2**-133, 2**-134, 3 * 2**-134,
             2**-126 * (1 - 2**-9), 3.3895313892515355e38, 3.3961e38, 3.4e38, 1e-45, 2**-149,
             65536 + 2**-10, 1.0 - 2**-9, 1.0 - 2**-10, 255.5, 256.5, 257.0]
    # doubles with bits below FP32 precision: exercises rounding of the full double
    vals += list(rng.standard_normal(200) * (1 + 2.0**-30))
    for d in vals:
        assert int(oracle.f64_to_bf16([d])[0]) == _rne_bf16_exact(float(d)), d


def test_bf16_rounding_matches_torch_cast_for_float32():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(oracle.f64_to_bf16(f.astype(np.float64)), _bf16_bits_torch(f))


# ---------------------------------------------------------- closed forms ---

def test_zero_row():
    # x = 0: rstd = 1/sqrt(eps) = 1000, y = 0; xhat = 0 so c = 0 and dx = rstd*g.
    n = 16
    x = np.zeros((1, n))
    w = np.linspace(0.5, 1.5, n)
    dy = np.linspace(-1, 1, n)[None, :]
    y, r = oracle.rmsnorm_fwd_f64(x, w, EPS)
    assert r[0] == pytest.approx(1000.0, rel=1e-15)
    assert np.all(y == 0)
    dx, dw = oracle.rmsnorm_bwd_f64(dy, x, w, EPS)
    assert np.allclose(dx[0], 1000.0 * dy[0] * w, rtol=1e-15, atol=0)
    assert np.all(dw == 0)


def test_constant_and_one_hot_rows():
    n = 32
    w = np.ones(n)
    for a in (3.0, -0.125, 1e-3):
        y, r = oracle.rmsnorm_fwd_f64(np.full((1, n), a), w, EPS)
        assert r[0] == pytest.approx(1 / math.sqrt(a * a + EPS), rel=1e-15)
        x = np.zeros((1, n))
        x[0, 5] = a
        y, r = oracle.rmsnorm_fwd_f64(x, w, EPS)
        # mean over the width n (not n-1), eps inside the root
        assert r[0] == pytest.approx(1 / math.sqrt(a * a / n + EPS), rel=1e-15)
        assert y[0, 5] == pytest.approx(a * r[0], rel=1e-15)


def test_scale_invariance_is_exact_for_eps_zero():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    w = 1 + 0.1 * rng.standard_normal(64)
    dy = rng.standard_normal((5, 64))
    y1, r1 = oracle.rmsnorm_fwd_f64(x, w, 0.0)
    y2, r2 = oracle.rmsnorm_fwd_f64(x * 8.0, w, 0.0)
    assert np.array_equal(y1, y2)
    assert np.array_equal(r1, r2 * 8.0)
    dx1, dw1 = oracle.rmsnorm_bwd_f64(dy, x, w, 0.0)
    dx2, dw2 = oracle.rmsnorm_bwd_f64(dy, x * 8.0, w, 0.0)
    assert np.array_equal(dx1, dx2 * 8.0)
    assert np.array_equal(dw1, dw2)


def test_unit_mean_square_for_eps_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 100)) * 3
    w = 1 + 0.1 * rng.standard_normal(100)
    y, _ = oracle.rmsnorm_fwd_f64(x, w, 0.0)
    ms = ((y / w) ** 2).mean(axis=1)
    assert np.allclose(ms, 1.0, rtol=0, atol=1e-14)


# ------------------------------------------------------- derivatives ---

def _fwd_complex(x, w, eps, z=None):
    """The forward written over complex numbers for complex-step derivatives."""
    n = x.shape[-1]
    r = 1.0 / np.sqrt((x * x).sum(axis=-1, keepdims=True) / n + eps)
    y = x * r * w
    if z is not None:
        y = y * (z / (1.0 + np.exp(-z)))
    return y


def _complex_step_grad(fn, arr, h=1e-30):
    g = np.zeros(arr.shape)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        a = arr.astype(np.complex128)
        a[idx] += 1j * h
        g[idx] = fn(a).imag / h
    return g


@pytest.mark.parametrize("eps", [EPS, 0.3])
def test_dx_dw_match_complex_step(eps):
    rng = np.random.default_rng(4)
    rows, n = 3, 12
    x = rng.standard_normal((rows, n))
    w = 1 + 0.1 * rng.standard_normal(n)
    dy = rng.standard_normal((rows, n))
    dx, dw = oracle.rmsnorm_bwd_f64(dy, x, w, eps)
    gx = _complex_step_grad(lambda xc: (dy * _fwd_complex(xc, w, eps)).sum(), x)
    gw = _complex_step_grad(lambda wc: (dy * _fwd_complex(x, wc, eps)).sum(), w)
    assert np.allclose(dx, gx, rtol=1e-12, atol=1e-14)
    assert np.allclose(dw, gw, rtol=1e-12, atol=1e-14)


def test_dx_dw_match_finite_differences_of_oracle_forward():
    # Central differences of the oracle's own forward tie its backward to it.
    rng = np.random.default_rng(5)
    rows, n = 2, 10
    x = rng.standard_normal((rows, n))
    w = 1 + 0.1 * rng.standard_normal(n)
    dy = rng.standard_normal((rows, n))
    dx, dw = oracle.rmsnorm_bwd_f64(dy, x, w, EPS)

    def loss(xx, ww):
        return float((dy * oracle.rmsnorm_fwd_f64(xx, ww, EPS)[0]).sum())

    h = 1e-6
    for i in range(rows):
        for j in range(n):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            assert (loss(xp, w) - loss(xm, w)) / (2 * h) == pytest.approx(dx[i, j], rel=1e-6, abs=1e-8)
    for j in range(n):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        assert (loss(x, wp) - loss(x, wm)) / (2 * h) == pytest.approx(dw[j], rel=1e-6, abs=1e-8)


@pytest.mark.parametrize("eps", [EPS, 1e-2])
def test_scale_invariance_identity(eps):
    # sum_j dx_j x_j = eps * rstd^3 * sum_j g_j x_j  (exact form of "~0 up to eps")
    rng = np.random.default_rng(6)
    rows, n = 6, 256
    x = rng.standard_normal((rows, n))
    w = 1 + 0.1 * rng.standard_normal(n)
    dy = rng.standard_normal((rows, n))
    dx, _ = oracle.rmsnorm_bwd_f64(dy, x, w, eps)
    _, r = oracle.rmsnorm_fwd_f64(x, w, eps)
    lhs = (dx * x).sum(axis=1)
    rhs = eps * r**3 * ((dy * w) * x).sum(axis=1)
    scale = np.abs(dx * x).sum(axis=1)
    assert np.all(np.abs(lhs - rhs) <= 1e-13 * scale)


def test_dw_is_exact_row_sum_of_dy_times_xhat():
    # with w = 1 the forward output is xhat itself; dw must be sum_i dy * xhat
    rng = np.random.default_rng(7)
    rows, n = 300, 8
    x = rng.standard_normal((rows, n))
    dy = rng.standard_normal((rows, n)) * 10.0 ** rng.integers(-3, 4, (rows, 1))
    w = np.ones(n)
    xhat, _ = oracle.rmsnorm_fwd_f64(x, w, EPS)
    _, dw = oracle.rmsnorm_bwd_f64(dy, x, w, EPS)
    for j in range(n):
        terms = dy[:, j] * xhat[:, j]
        exact = math.fsum(terms)
        bound = rows * 2**-53 * math.fsum(abs(terms))
        assert abs(dw[j] - exact) <= bound


# ------------------------------------------------------------- gated form ---

def test_gate_matches_complex_step():
    rng = np.random.default_rng(8)
    rows, n = 3, 9
    x = rng.standard_normal((rows, n))
    z = rng.standard_normal((rows, n)) * 2
    w = 1 + 0.1 * rng.standard_normal(n)
    dy = rng.standard_normal((rows, n))
    y, r = oracle.gate_fwd_f64(x, z, w, EPS)
    assert np.allclose(y, _fwd_complex(x, w, EPS, z).real, rtol=1e-14, atol=1e-15)
    dx, dz, dw = oracle.gate_bwd_f64(dy, x, z, w, EPS)
    gx = _complex_step_grad(lambda c: (dy * _fwd_complex(c, w, EPS, z)).sum(), x)
    gz = _complex_step_grad(lambda c: (dy * _fwd_complex(x, w, EPS, c)).sum(), z)
    gw = _complex_step_grad(lambda c: (dy * _fwd_complex(x, c, EPS, z)).sum(), w)
    assert np.allclose(dx, gx, rtol=1e-12, atol=1e-14)
    assert np.allclose(dz, gz, rtol=1e-12, atol=1e-14)
    assert np.allclose(dw, gw, rtol=1e-12, atol=1e-14)


def test_gate_special_cases_reduce_to_plain_form():
    rng = np.random.default_rng(9)
    rows, n = 4, 32
    x = rng.standard_normal((rows, n))
    w = 1 + 0.1 * rng.standard_normal(n)
    dy = rng.standard_normal((rows, n))
    # z = 0: silu = 0, so y = 0, dx = 0, dw = 0 and dz = dy * xhat * w * 1/2
    zero = np.zeros((rows, n))
    y, _ = oracle.gate_fwd_f64(x, zero, w, EPS)
    dx, dz, dw = oracle.gate_bwd_f64(dy, x, zero, w, EPS)
    xhat, _ = oracle.rmsnorm_fwd_f64(x, np.ones(n), EPS)
    assert np.all(y == 0) and np.all(dx == 0) and np.all(dw == 0)
    assert np.allclose(dz, dy * xhat * w * 0.5, rtol=1e-15, atol=0)
    # z = 40: sigmoid rounds to exactly 1, silu = z; the gate is a scalar factor
    big = np.full((rows, n), 40.0)
    yg, rg = oracle.gate_fwd_f64(x, big, w, EPS)
    yp, rp = oracle.rmsnorm_fwd_f64(x, w, EPS)
    assert np.array_equal(rg, rp)
    assert np.array_equal(yg, yp * 40.0)
    dxg, _, dwg = oracle.gate_bwd_f64(dy, x, big, w, EPS)
    dxp, dwp = oracle.rmsnorm_bwd_f64(dy * 40.0, x, w, EPS)
    assert np.allclose(dxg, dxp, rtol=1e-14, atol=0)
    assert np.allclose(dwg, dwp, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- views ---

def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_bf16_views_equal_dense_core_on_converted_inputs():
    # The BF16 entry points over a strided per-head view equal the dense FP64
    # core applied to the gathered rows (the view plumbing adds nothing).
    rng = np.random.default_rng(10)
    T, heads, width, st, sh = 5, 3, 16, 100, 32
    buf = rng.standard_normal(T * st).astype(np.float32)
    xb = _bits(torch.from_numpy(buf).to(torch.bfloat16))
    dyb = _bits(torch.from_numpy(rng.standard_normal(T * st).astype(np.float32)).to(torch.bfloat16))
    w = 1 + 0.1 * rng.standard_normal(width)
    xv = oracle.View(xb, T, heads, width, st, sh)
    dyv = oracle.View(dyb, T, heads, width, st, sh)
    gather = lambda b: np.stack([oracle.bf16_to_f64(b[t * st + h * sh: t * st + h * sh + width])
                                 for t in range(T) for h in range(heads)])
    xd, dyd = gather(xb), gather(dyb)
    y, r = oracle.fwd(xv, w, EPS)
    y2, r2 = oracle.rmsnorm_fwd_f64(xd, w, EPS)
    assert np.array_equal(y, y2) and np.array_equal(r, r2)
    dx, dw = oracle.bwd(dyv, xv, w, EPS)
    dx2, dw2 = oracle.rmsnorm_bwd_f64(dyd, xd, w, EPS)
    assert np.array_equal(dx, dx2) and np.array_equal(dw, dw2)
    sel = [14, 0, 7]
    dxs, _ = oracle.bwd(dyv, xv, w, EPS, sel=sel, want_dw=False)
    assert np.array_equal(dxs, dx[sel])


def test_residual_h_is_rounded_exact_sum():
    rng = np.random.default_rng(11)
    n = 4096
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 10.0 ** rng.integers(-6, 6, n)).to(torch.bfloat16)
    res = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 10.0 ** rng.integers(-6, 6, n)).to(torch.bfloat16)
    # hand-made edges: ties to even, huge exponent gaps, exact cancellation
    edge_x = [1.0, 1.0 + 2**-7, 2.0**20, 3.0, -2.5, 2.0**-130]
    edge_r = [2**-8, 2**-8, 2**-10, -3.0, 2.5, 2.0**-130]
    x[: len(edge_x)] = torch.tensor(edge_x).to(torch.bfloat16)
    res[: len(edge_r)] = torch.tensor(edge_r).to(torch.bfloat16)
    xb, rb = _bits(x), _bits(res)
    h, _, _ = oracle.res_fwd(oracle.View.dense(xb[None]), oracle.View.dense(rb[None]), np.ones(n), EPS)
    ref = _bits((x.float() + res.float()).to(torch.bfloat16))
    assert np.array_equal(h[0], ref)
    assert oracle.bf16_to_f64(h[0, :6]).tolist() == [1.0, 1.0 + 2**-6, 2.0**20, 0.0, 0.0, 2.0**-129]


# ------------------------------------------------ the dw budget discriminates ---

def test_plain_fp32_column_sum_fails_budget_on_cancellation_family():
    # The dw budget (PR #8848 page, "Measurement": atol 1e-4 + rtol 1e-4 vs
    # FP64) must reject a plain sequential FP32 column sum on the cancellation
    # family, while the FP64 oracle sits far inside it (review on the PR #8512
    # page asks for exactly this check).
    import synth

    p = synth.make(8192, 512, seed=0, family="cancel", w_dtype="f32")
    xb = _bits(p.x).reshape(p.T, p.width)
    dyb = _bits(p.dy).reshape(p.T, p.width)
    w = p.w.double().numpy()
    _, dw = oracle.bwd(oracle.View.dense(dyb), oracle.View.dense(xb), w, p.eps, want_rows=False)
    x = oracle.bf16_to_f64(xb)
    dy = oracle.bf16_to_f64(dyb)
    xhat, _ = oracle.rmsnorm_fwd_f64(x, np.ones(p.width), p.eps)
    terms32 = (dy * xhat).astype(np.float32)
    plain32 = terms32.sum(axis=0, dtype=np.float32)  # axis-0 reduce: sequential over rows
    tol = 1e-4 + 1e-4 * np.abs(dw)
    assert np.max(np.abs(plain32 - dw) / tol) > 1.0
    exact = np.array([math.fsum(dy[:, j] * xhat[:, j]) for j in range(0, p.width, 37)])
    assert np.max(np.abs(dw[::37] - exact) / (1e-4 + 1e-4 * np.abs(exact))) < 1e-6


def test_residual_backward_matches_complex_step():
    # Residual form (PR #8512 page, "Residual rows"): the loss sees h both
    # through y = RMSNorm(h) w and directly (the h output), so the gradient of
    # h is d/dh [sum dy*y + sum dh*h].
    rng = np.random.default_rng(12)
    T, n = 3, 16
    mk = lambda: _bits(torch.from_numpy(rng.standard_normal((T, n)).astype(np.float32)).to(torch.bfloat16))
    hb, dyb, dhb = mk(), mk(), mk()
    w = 1 + 0.1 * rng.standard_normal(n)
    gh, dw = oracle.bwd(oracle.View.dense(dyb), oracle.View.dense(hb), w, EPS,
                        dh=oracle.View.dense(dhb))
    h, dy, dh = (oracle.bf16_to_f64(b) for b in (hb, dyb, dhb))
    ref = _complex_step_grad(lambda c: (dy * _fwd_complex(c, w, EPS)).sum() + (dh * c).sum(), h)
    refw = _complex_step_grad(lambda c: (dy * _fwd_complex(h, c, EPS)).sum(), w)
    assert np.allclose(gh, ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(dw, refw, rtol=1e-12, atol=1e-14)


# ----------------------------------- residual forward and gated views ---

def _mk_bits(rng, shape, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return _bits(torch.from_numpy(a).to(torch.bfloat16))


def test_residual_forward_normalises_the_rounded_h():
    # PR #8512 page, description, "Residual rows": the forward returns h = x +
    # residual and y = RMSNorm(h); PR #8848 page, "Key": h_new = BF16(h + u).
    # So y and rstd are the plain forward of the BF16 h the call returns.
    # The addends are scaled so that rounding x + residual to BF16 moves each
    # row's rstd by far more than 1e-12 relative: normalising x, or the
    # unrounded sum, instead of h fails.
    rng = np.random.default_rng(13)
    T, n = 6, 64
    xb = _mk_bits(rng, (T, n), 3.0)
    rb = _mk_bits(rng, (T, n), 0.37)
    w = 1 + 0.1 * rng.standard_normal(n)
    h, y, r = oracle.res_fwd(oracle.View.dense(xb), oracle.View.dense(rb), w, EPS)
    # the pinned plain forward, applied to the returned h
    y2, r2 = oracle.fwd(oracle.View.dense(h), w, EPS)
    assert np.array_equal(y, y2) and np.array_equal(r, r2)
    # the closed form on h, evaluated here in numpy (rstd to 1e-15 relative)
    hd = oracle.bf16_to_f64(h)
    r_ref = 1.0 / np.sqrt((hd * hd).mean(axis=1) + EPS)
    assert np.allclose(r, r_ref, rtol=1e-15, atol=0)
    assert np.allclose(y, hd * r_ref[:, None] * w, rtol=1e-14, atol=0)
    # the test inputs discriminate: rstd of the unrounded sum differs by > 1e-12
    s = oracle.bf16_to_f64(xb) + oracle.bf16_to_f64(rb)
    r_unrounded = 1.0 / np.sqrt((s * s).mean(axis=1) + EPS)
    assert np.all(np.abs(r_unrounded / r_ref - 1.0) > 1e-12)
    r_x = 1.0 / np.sqrt((oracle.bf16_to_f64(xb) ** 2).mean(axis=1) + EPS)
    assert np.all(np.abs(r_x / r_ref - 1.0) > 1e-3)


def test_residual_forward_row_selection_over_a_per_head_view():
    # Rows chosen by `sel` are the same rows of the full output, in the order
    # asked for, and h is always written for every row (strided per-head view).
    rng = np.random.default_rng(14)
    T, heads, n, st, sh = 4, 3, 32, 160, 48
    xb = _mk_bits(rng, T * st)
    rb = _mk_bits(rng, T * st)
    w = 1 + 0.1 * rng.standard_normal(n)
    xv = oracle.View(xb, T, heads, n, st, sh)
    rv = oracle.View(rb, T, heads, n, st, sh)
    h, y, r = oracle.res_fwd(xv, rv, w, EPS)
    sel = [11, 0, 5, 5, 7]
    hs, ys, rs = oracle.res_fwd(xv, rv, w, EPS, sel=sel)
    assert np.array_equal(hs, h)
    assert np.array_equal(ys, y[sel]) and np.array_equal(rs, r[sel])
    # and the full output's rows are the rows of the view, in row order
    for t in range(T):
        for hh in range(heads):
            o = t * st + hh * sh
            ref = _bits((torch.from_numpy(oracle.bf16_to_f64(xb[o:o + n]).astype(np.float32)) +
                         torch.from_numpy(oracle.bf16_to_f64(rb[o:o + n]).astype(np.float32)))
                        .to(torch.bfloat16))
            assert np.array_equal(h[t * heads + hh], ref)


def _gather(b, T, heads, n, st, sh):
    return np.stack([oracle.bf16_to_f64(b[t * st + h * sh: t * st + h * sh + n])
                     for t in range(T) for h in range(heads)])


def test_gate_view_entry_points_equal_dense_cores_with_separate_z():
    # PR #8656 page, description: y = RMSNorm(x) w silu(z) with z its own
    # tensor. Over a strided per-head view whose z buffer differs from x (and
    # has its own padding), the BF16 entry points equal the pinned dense FP64
    # cores applied to the gathered rows of x, z and dy.
    rng = np.random.default_rng(15)
    T, heads, n, st, sh = 5, 3, 24, 120, 40
    xb, dyb = _mk_bits(rng, T * st), _mk_bits(rng, T * st)
    zb = _mk_bits(rng, T * st, 2.0)
    w = 1 + 0.1 * rng.standard_normal(n)
    xv, zv, dyv = (oracle.View(b, T, heads, n, st, sh) for b in (xb, zb, dyb))
    xd, zd, dyd = (_gather(b, T, heads, n, st, sh) for b in (xb, zb, dyb))
    y, r = oracle.gate_fwd(xv, zv, w, EPS)
    y2, r2 = oracle.gate_fwd_f64(xd, zd, w, EPS)
    assert np.array_equal(y, y2) and np.array_equal(r, r2)
    dx, dz, dw = oracle.gate_bwd(dyv, xv, zv, w, EPS)
    dx2, dz2, dw2 = oracle.gate_bwd_f64(dyd, xd, zd, w, EPS)
    assert np.array_equal(dx, dx2) and np.array_equal(dz, dz2) and np.array_equal(dw, dw2)
    # row selection: the chosen rows of the full output; dw still over all rows
    sel = [14, 2, 9]
    ys, rs = oracle.gate_fwd(xv, zv, w, EPS, sel=sel)
    assert np.array_equal(ys, y[sel]) and np.array_equal(rs, r[sel])
    dxs, dzs, dws = oracle.gate_bwd(dyv, xv, zv, w, EPS, sel=sel)
    assert np.array_equal(dxs, dx[sel]) and np.array_equal(dzs, dz[sel])
    assert np.array_equal(dws, dw)
    # the inputs discriminate: with z read through x's view the results move
    y_xz, _ = oracle.gate_fwd_f64(xd, xd, w, EPS)
    assert not np.allclose(y_xz, y)


# --------------------------------------------------- zero-centred weight ---
# The related-PR title "zero-centred input RMSNorm" on the PR #8512 page, read
# as the RMSNorm whose stored weight is centred on zero and enters as 1 + w.

def test_zero_centred_weight_zero_is_the_unit_gain_norm():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((4, 48))
    dy = rng.standard_normal((4, 48))
    w_eff = oracle.zero_centred_weight(np.zeros(48))
    assert np.array_equal(w_eff, np.ones(48))
    y, r = oracle.rmsnorm_fwd_f64(x, w_eff, EPS)
    # closed form: y = x / sqrt(mean x^2 + eps)
    ref = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + EPS)
    assert np.allclose(y, ref, rtol=1e-15, atol=0)
    # and the stored value enters once, as 1 + w
    w = rng.standard_normal(48) * 0.1
    assert np.array_equal(oracle.zero_centred_weight(w), 1.0 + w)


def test_zero_centred_weight_matches_complex_step_of_its_own_loss():
    # loss = sum dy * xhat * (1 + w), written here over complex numbers; its
    # derivatives w.r.t. x and the stored w are the oracle's dx and dw taken
    # with the effective weight 1 + w (plain and gated forms)
    rng = np.random.default_rng(17)
    rows, n = 3, 10
    x = rng.standard_normal((rows, n))
    z = rng.standard_normal((rows, n))
    dy = rng.standard_normal((rows, n))
    w = 0.1 * rng.standard_normal(n)

    def fwd_zc(xc, wc, zc=None):
        r = 1.0 / np.sqrt((xc * xc).sum(axis=-1, keepdims=True) / n + EPS)
        y = xc * r * (1.0 + wc)
        return y if zc is None else y * (zc / (1.0 + np.exp(-zc)))

    dx, dw = oracle.rmsnorm_bwd_f64(dy, x, oracle.zero_centred_weight(w), EPS)
    gx = _complex_step_grad(lambda c: (dy * fwd_zc(c, w)).sum(), x)
    gw = _complex_step_grad(lambda c: (dy * fwd_zc(x, c)).sum(), w)
    assert np.allclose(dx, gx, rtol=1e-12, atol=1e-14)
    assert np.allclose(dw, gw, rtol=1e-12, atol=1e-14)
    dxg, dzg, dwg = oracle.gate_bwd_f64(dy, x, z, oracle.zero_centred_weight(w), EPS)
    assert np.allclose(dxg, _complex_step_grad(lambda c: (dy * fwd_zc(c, w, z)).sum(), x),
                       rtol=1e-12, atol=1e-14)
    assert np.allclose(dzg, _complex_step_grad(lambda c: (dy * fwd_zc(x, w, c)).sum(), z),
                       rtol=1e-12, atol=1e-14)
    assert np.allclose(dwg, _complex_step_grad(lambda c: (dy * fwd_zc(x, c, z)).sum(), w),
                       rtol=1e-12, atol=1e-14)
