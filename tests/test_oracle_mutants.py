"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that the pins in
test_oracle_pins.py and test_oracle_scales.py catch every one of them: a pin suite that a
dropped term, a flipped sign, a wrong index, a missing rounding point or a wrong tolerance
scale would pass is not a pin."""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement).  Each text must occur in the source.
MUTANTS = [
    ("dyt_fwd_beta_sign", "if (y) y[i * N + j] = g * t + b;", "if (y) y[i * N + j] = g * t - b;"),
    ("dyt_fwd_gamma_beta_swapped", "double g = load_elem(gamma, pdt, j), b = load_elem(beta, pdt, j);\n            double t = tanh",
     "double g = load_elem(beta, pdt, j), b = load_elem(gamma, pdt, j);\n            double t = tanh"),
    ("dyt_fwd_gamma_row_index", "double g = load_elem(gamma, pdt, j), b = load_elem(beta, pdt, j);\n            double t = tanh",
     "double g = load_elem(gamma, pdt, (i + j) % N), b = load_elem(beta, pdt, j);\n            double t = tanh"),
    ("dyt_dx_drops_alpha", "return s == 0.0 ? 0.0 : alpha * s;", "return s;"),
    ("dyt_dx_inf_times_zero", "return s == 0.0 ? 0.0 : alpha * s;", "return alpha * s;"),
    ("dyt_dgamma_drops_dy", "terms[j] = g * tanh(z);", "terms[j] = tanh(z);"),
    ("dyt_dalpha_drops_x", "double t = g * load_elem(c->gamma, c->pdt, j) * xv * s;", "double t = g * load_elem(c->gamma, c->pdt, j) * s;"),
    ("dyt_dalpha_drops_gamma", "double t = g * load_elem(c->gamma, c->pdt, j) * xv * s;", "double t = g * xv * s;"),
    ("ln_unbiased_variance", "    v /= (double)N;\n", "    v /= (double)(N > 1 ? N - 1 : 1);\n"),
    ("ln_eps_outside_sqrt", "*rstd_out = 1.0 / sqrt(v + eps);", "*rstd_out = 1.0 / (sqrt(v) + eps);"),
    ("ln_dx_sign", "if (dx) dx[i * N + j] = r * (g - c1 - xh * c2);", "if (dx) dx[i * N + j] = r * (g - c1 + xh * c2);"),
    ("ln_c1_uses_dy", "                c1 += g;\n", "                c1 += load_elem(dy, xdt, i * N + j);\n"),
    ("ln_dgamma_drops_rstd", "terms[j] = g * (xv - mu) * r;", "terms[j] = g * (xv - mu);"),
    ("rms_n_not_rounded", "            double n = round_to(xdt, h);\n", "            double n = h;\n"),
    ("rms_g_not_rounded", "double g = round_to(xdt, round_arith(xdt, load_elem(dy, xdt, i * N + j) * load_elem(w, wdt, j)));\n                double h",
     "double g = round_arith(xdt, load_elem(dy, xdt, i * N + j) * load_elem(w, wdt, j));\n                double h"),
    ("rms_dw_term_not_rounded", "double t = round_to(c->wdt, round_arith(c->xdt, g * n));",
     "double t = round_arith(c->xdt, g * n);"),
    ("rms_dx_sign", "if (dx) dx[i * N + j] = r * (g - h * c);", "if (dx) dx[i * N + j] = r * (g + h * c);"),
    ("rms_sum_not_mean", "return 1.0 / sqrt(s / (double)N + eps);", "return 1.0 / sqrt(s + eps);"),
    ("colsum_drops_block_tail", "int64_t i1 = (b + 1) * ORA_ROW_BLOCK < M ? (b + 1) * ORA_ROW_BLOCK : M;",
     "int64_t i1 = ((b + 1) * ORA_ROW_BLOCK < M ? (b + 1) * ORA_ROW_BLOCK : M) - 1;"),
    ("bf16_ties_away", "double r = ldexp(nearbyint(ldexp(v, -q)), q);", "double r = ldexp(round(ldexp(v, -q)), q);"),
    ("bf16_seven_bits", "int q = e - 8;", "int q = e - 7;"),
    ("rms_form_drops_one", "return form == 2 ? round_arith(xdt, 1.0 + wj) : wj;", "return wj;"),
    ("rms_form_rounds_g", "double g = load_elem(dy, xdt, i * N + j) * rms_form_scale(form, xdt, load_elem(w, wdt, j));\n                double h = load_elem(x, xdt, i * N + j) * r;\n                if (dx)",
     "double g = round_to(xdt, load_elem(dy, xdt, i * N + j) * rms_form_scale(form, xdt, load_elem(w, wdt, j)));\n                double h = load_elem(x, xdt, i * N + j) * r;\n                if (dx)"),
    ("rms_form_rounds_h", "double v = rms_form_scale(form, xdt, load_elem(w, wdt, j)) * (load_elem(x, xdt, i * N + j) * r);",
     "double v = rms_form_scale(form, xdt, load_elem(w, wdt, j)) * round_to(xdt, load_elem(x, xdt, i * N + j) * r);"),
    ("rms_form_dw_drops_rstd", "terms[j] = load_elem(c->dy, c->xdt, i * c->N + j) * (load_elem(c->x, c->xdt, i * c->N + j) * r);",
     "terms[j] = load_elem(c->dy, c->xdt, i * c->N + j) * load_elem(c->x, c->xdt, i * c->N + j);"),
    ("f16_nine_fraction_bits", "int q = e - 11;", "int q = e - 10;"),
    ("f16_subnormal_spacing", "if (q < -24) q = -24;", "if (q < -25) q = -25;"),
    ("f16_no_overflow", "if (fabs(r) > 65504.0) r = copysign(INFINITY, v);", ""),
    ("f16_exponent_bias", "else v = ldexp((double)(1024 + f), e - 25);", "else v = ldexp((double)(1024 + f), e - 24);"),
    ("f16_subnormal_read", "if (e == 0) v = ldexp((double)f, -24);", "if (e == 0) v = ldexp((double)(1024 + f), -25);"),
    # --- mistakes in the tolerance scales (magnitude sums) and the admissible-rounding window
    ("scale_param_abs_sums_x10", "pa[c] += fabs(terms[c]);", "pa[c] += 10.0 * fabs(terms[c]);"),
    ("scale_dyt_y_drops_beta", "y_scale[i * N + j] = fabs(g * t) + fabs(b);", "y_scale[i * N + j] = fabs(g * t);"),
    ("scale_dyt_y_x10", "y_scale[i * N + j] = fabs(g * t) + fabs(b);", "y_scale[i * N + j] = 10.0 * (fabs(g * t) + fabs(b));"),
    ("scale_dyt_dx_x10", "if (dx_scale) dx_scale[i * N + j] = fabs(v);", "if (dx_scale) dx_scale[i * N + j] = 10.0 * fabs(v);"),
    ("scale_dyt_dalpha_row_sums", "daa += fabs(t);", "daa += t;"),
    ("scale_ln_y_drops_am", "y_scale[i * N + j] = r * fabs(g) * (fabs(xv) + am) + fabs(b);",
     "y_scale[i * N + j] = r * fabs(g) * fabs(xv) + fabs(b);"),
    ("scale_ln_y_times_N", "y_scale[i * N + j] = r * fabs(g) * (fabs(xv) + am) + fabs(b);",
     "y_scale[i * N + j] = (double)N * (r * fabs(g) * (fabs(xv) + am) + fabs(b));"),
    ("scale_ln_dx_drops_r", "dx_scale[i * N + j] = r * (fabs(g) + a1 + r * (fabs(xv) + am) * a2);",
     "dx_scale[i * N + j] = r * (fabs(g) + a1 + (fabs(xv) + am) * a2);"),
    ("scale_ln_dx_drops_am", "a2 += fabs(g) * r * (fabs(xv) + am);", "a2 += fabs(g) * r * fabs(xv);"),
    ("scale_ln_dx_times_N", "dx_scale[i * N + j] = r * (fabs(g) + a1 + r * (fabs(xv) + am) * a2);",
     "dx_scale[i * N + j] = (double)N * r * (fabs(g) + a1 + r * (fabs(xv) + am) * a2);"),
    ("scale_ln_dgamma_drops_am", "terms[2 * c->N + j] = fabs(g) * r * (fabs(xv) + am);",
     "terms[2 * c->N + j] = fabs(g * (xv - mu) * r);"),
    ("scale_ln_mean_x10", "if (mean_scale) mean_scale[i] = am;", "if (mean_scale) mean_scale[i] = 10.0 * am;"),
    ("scale_ln_rstd_drops_am", "double m = fabs(load_elem(x, xdt, i * N + j)) + am;",
     "double m = fabs(load_elem(x, xdt, i * N + j));"),
    ("scale_rms_dx_abs_of_mean", "a += fabs(g * load_elem(x, xdt, i * N + j) * r);", "a += g * load_elem(x, xdt, i * N + j) * r;"),
    ("scale_rms_dx_drops_r", "if (dx_scale) dx_scale[i * N + j] = r * (fabs(g) + fabs(h) * a);",
     "if (dx_scale) dx_scale[i * N + j] = fabs(g) + fabs(h) * a;"),
    ("scale_rms_y_x10", "if (y_scale) y_scale[i * N + j] = fabs(v);\n            if (y_alt)",
     "if (y_scale) y_scale[i * N + j] = 10.0 * fabs(v);\n            if (y_alt)"),
    ("scale_rms_form_dx_times_N", "a += fabs(g * h);", "a += (double)N * fabs(g * h);"),
    ("tie_window_2e-14", "double tol = ldexp(fabs(h), -18);", "double tol = ldexp(fabs(h), -14);"),
    ("tie_window_2e-20", "double tol = ldexp(fabs(h), -18);", "double tol = ldexp(fabs(h), -20);"),
    ("dw_slack_doubled", "terms[c->N + j] = fabs(ta - t);", "terms[c->N + j] = 2.0 * fabs(ta - t);"),
]
PIN_FILES = ["test_oracle_pins.py", "test_oracle_scales.py"]


def _kill(mutant, tmp):
    name, old, new = mutant
    with open(SRC) as f:
        src = f.read()
    assert old in src, f"mutant {name}: text not found in oracle.c"
    lib = oracle.build_variant(src.replace(old, new, 1), os.path.join(tmp, f"lib_{name}.so"))
    env = dict(os.environ, ORACLE_LIBRARY=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _kill(m, tmp), MUTANTS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"


def test_unmutated_copy_passes_the_pins():
    with tempfile.TemporaryDirectory() as tmp:
        name, rc = _kill(("identity", "#include <math.h>", "#include <math.h>"), tmp)
    assert rc == 0
