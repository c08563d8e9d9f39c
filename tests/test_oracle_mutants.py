"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that the pins in
test_oracle_pins.py catch every one of them: a pin suite that a dropped term, a flipped sign,
a wrong index or a missing rounding point would pass is not a pin."""
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
    ("dyt_dalpha_drops_x", "da += g * load_elem(c->gamma, c->pdt, j) * xv * s;", "da += g * load_elem(c->gamma, c->pdt, j) * s;"),
    ("dyt_dalpha_drops_gamma", "da += g * load_elem(c->gamma, c->pdt, j) * xv * s;", "da += g * xv * s;"),
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
]


def _kill(mutant, tmp):
    name, old, new = mutant
    with open(SRC) as f:
        src = f.read()
    assert old in src, f"mutant {name}: text not found in oracle.c"
    lib = oracle.build_variant(src.replace(old, new, 1), os.path.join(tmp, f"lib_{name}.so"))
    env = dict(os.environ, ORACLE_LIBRARY=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
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
