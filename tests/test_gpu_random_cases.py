"""GPU parity on seeded random call shapes: width, form, token count (ragged,
1 to ~2500), heads and padded strides, weight dtype, zero-centred weight,
input family and a forced path, all drawn from one fixed generator, so the
cases are the same on every run. Each case runs the forward and both backward
modes and checks every row and column against the FP64 oracle within the same
budgets as the configuration tests. The shapes are small enough for the
oracle to take well under a second each.
"""
import numpy as np
import pytest

import rmsnorm_train_fwd_amd as R
import synth

from test_gpu_parity import run_case

pytestmark = pytest.mark.gpu

WIDTHS = (256, 512, 1536, 2048, 4096, 5120, 6144)
N_CASES = 120


def draw_cases(n=N_CASES, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        W = int(rng.choice(WIDTHS))
        form = str(rng.choice(["plain", "plain", "residual", "gate"]))
        heads = 1 if rng.random() < 0.6 else int(rng.integers(2, 7))
        # token count log-uniform, rows kept to a few thousand
        T = int(np.exp(rng.uniform(0.0, np.log(2500 / heads))))
        T = max(T, 1)
        hs = W + 8 * int(rng.integers(0, 4)) if heads > 1 else W
        rs = heads * hs + 8 * int(rng.integers(0, 4))
        w_dtype = str(rng.choice(["f32", "bf16"]))
        zero_centred = bool(rng.random() < 0.2)
        family = str(rng.choice(["normal", "normal", "spread"]))
        path = int(rng.choice([R.PATH_AUTO, R.PATH_AUTO, R.PATH_SMALL, R.PATH_LARGE]))
        cases.append(dict(i=i, W=W, form=form, heads=heads, T=T, hs=hs, rs=rs, w_dtype=w_dtype,
                          zero_centred=zero_centred, family=family, path=path))
    return cases


CASES = draw_cases()


def test_the_draw_covers_every_width_form_and_path():
    assert {c["W"] for c in CASES} == set(WIDTHS)
    assert {c["form"] for c in CASES} == {"plain", "residual", "gate"}
    assert {c["path"] for c in CASES} == {R.PATH_AUTO, R.PATH_SMALL, R.PATH_LARGE}
    assert any(c["heads"] > 1 for c in CASES) and any(c["zero_centred"] for c in CASES)


@pytest.mark.parametrize("c", CASES, ids=lambda c: (f"{c['i']}-{c['form']}-[{c['T']},{c['heads']},"
                                                     f"{c['W']}]-{c['w_dtype']}"))
def test_random_case_matches_the_oracle(c):
    p = synth.make(c["T"], c["W"], seed=c["i"], heads=c["heads"], w_dtype=c["w_dtype"],
                   family=c["family"], form=c["form"], row_stride=c["rs"],
                   head_stride=c["hs"] if c["heads"] > 1 else None,
                   w_centre=0.0 if c["zero_centred"] else 1.0)
    launch = None if c["path"] == R.PATH_AUTO else R.Launch(0, 0, c["path"])
    run_case(p, det=(True, False), form=c["form"], launch=launch,
             zero_centred=c["zero_centred"])
