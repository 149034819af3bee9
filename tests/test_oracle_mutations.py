"""Plant plausible mistakes in copies of the oracle and check that the pins
in test_oracle_pins.py catch every one (CPU only; the copies live in a temp
directory and are loaded through RMSN_ORACLE_LIB in a child pytest)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rmsn_oracle.c")

MUTATIONS = {
    "mean_over_n_minus_1": ("ss / (double)n + eps", "ss / (double)(n - 1) + eps"),
    "eps_outside_root": ("1.0 / sqrt(ss / (double)n + eps)", "1.0 / sqrt(ss / (double)n) + eps"),
    "dx_sign": ("dx[j] = r * (g - xh * c)", "dx[j] = r * (g + xh * c)"),
    "dx_drops_mean_term": ("dx[j] = r * (g - xh * c)", "dx[j] = r * g"),
    "c_not_divided": ("c /= (double)n;", "c /= 1.0;"),
    "dw_uses_x_not_xhat": ("dw[j] += dy[j] * xh * silu", "dw[j] += dy[j] * x[j] * silu"),
    "dw_uses_g": ("dw[j] += dy[j] * xh * silu", "dw[j] += g * xh"),
    "dz_missing_factor": ("s * (1.0 + gate[j] * (1.0 - s))", "s"),
    "gate_uses_sigmoid_not_silu": ("y[i * width + j] = (xi[j] * r) * w[j] * (zi[j] * sigmoid(zi[j]))",
                                   "y[i * width + j] = (xi[j] * r) * w[j] * sigmoid(zi[j])"),
    "bf16_round_truncates": ("double r = nearbyint(n);", "double r = trunc(n);"),
    "bf16_round_ties_away": ("double r = nearbyint(n);", "double r = round(n);"),
    "view_head_stride_ignored": ("v->p + t * v->st + h * v->sh", "v->p + t * v->st + h * v->width"),
    "residual_not_rounded": ("h[r * n + j] = orc_f64_to_bf16(a[j] + b[j])", "h[r * n + j] = orc_f64_to_bf16(a[j])"),
    "grad_h_drops_dh": ("dxi[j] = hr[j] + dxi[j]", "dxi[j] = dxi[j]"),
    "residual_y_from_x_not_h": ("orc_bf16_to_f64_array(h + r * n, n, a);", "load_row(x, r, a);"),
    "residual_y_from_unrounded_sum": ("orc_bf16_to_f64_array(h + r * n, n, a);",
                                      "load_row(x, r, a); load_row(res, r, b); "
                                      "for (int64_t j = 0; j < n; ++j) a[j] += b[j];"),
    "residual_sel_ignored": ("int64_t r = sel ? sel[i] : i;\n    orc_bf16_to_f64_array(h + r * n",
                             "int64_t r = i;\n    orc_bf16_to_f64_array(h + r * n"),
    "gate_fwd_view_z_from_x": ("load_row(z, r, zr);\n    orc_gate_fwd_f64",
                               "load_row(x, r, zr);\n    orc_gate_fwd_f64"),
    "gate_bwd_view_z_from_x": ("if (z) load_row(z, r, zr);", "if (z) load_row(x, r, zr);"),
    "gate_bwd_view_dw_z_from_x": ("if (z) load_row(z, r, zr);\n      row_bwd(n, gr, xr, z ? zr : NULL, w, eps, NULL, NULL, dw);",
                                  "if (z) load_row(x, r, zr);\n      row_bwd(n, gr, xr, z ? zr : NULL, w, eps, NULL, NULL, dw);"),
    "zero_centred_offset_missing": ("out[j] = 1.0 + w[j];", "out[j] = w[j];"),
    "zero_centred_offset_doubled": ("out[j] = 1.0 + w[j];", "out[j] = 2.0 + w[j];"),
    "gate_fwd_sel_ignored": ("int64_t r = sel ? sel[i] : i;\n    load_row(x, r, xr);\n    load_row(z, r, zr);",
                             "int64_t r = i;\n    load_row(x, r, xr);\n    load_row(z, r, zr);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor missing: {old}"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), str(mut), "-lm"], check=True)
    env = dict(os.environ, RMSN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"
