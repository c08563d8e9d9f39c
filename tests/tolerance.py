"""Element-by-element comparison of GPU results with the oracle's exact values.

Bounds (the oracle returns the exact value before the final cast plus a magnitude sum S):
  float32 outputs and dx:      |gpu - exact| <= 1e-5 * S_e                    (+ a 4*FLT_MIN floor)
  bfloat16 / float16 outputs and dx:
                               |gpu - exact| <= ulp + 1e-5 * S_e              (1 ulp of the dtype after fp32 compute)
  parameter gradients:         |gpu - exact| <= 1e-4 * sum_i |term_ij| + ulp_param_dtype
                               (+ RMSNorm: the summed change of terms whose normalized value
                               has two admissible roundings)
S_e is the sum of the magnitudes of the terms forming the element, so where nothing cancels
the float32 bound is a plain relative error.  A NaN or Inf where the oracle is finite fails;
NaN where the oracle is NaN passes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

FLT_MIN = float(np.finfo(np.float32).tiny)
REL_ELEM = 1e-5
REL_PARAM = 1e-4


def ulp(v: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Spacing of dtype's values at |v| (binade-based; subnormal spacing below the normal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    mant, emin = {torch.bfloat16: (7, -126), torch.float16: (10, -14)}.get(dtype, (23, -126))
    # frexp: a = f * 2^k with f in [0.5, 1), so the binade exponent is k - 1
    _, k = np.frexp(np.where(np.isfinite(a) & (a > 0), a, 1.0))
    e = np.maximum(k.astype(np.int64) - 1, emin)
    return np.where(np.isfinite(a), np.ldexp(1.0, e - mant), np.inf)


@dataclasses.dataclass
class Report:
    name: str
    n: int
    bad: int
    max_ratio: float        # max of err / bound
    max_ulp: float          # max error in output-dtype ulps
    within_1ulp: float      # fraction of elements within one ulp
    worst: Optional[tuple]
    outside_policy: int = 0  # elements outside |gpu - exact| <= 2^-6 + 2^-6 |exact| (the BF16 policy)

    def ok(self) -> bool:
        return self.bad == 0

    def __str__(self):
        return (f"{self.name}: n={self.n} bad={self.bad} max_err/bound={self.max_ratio:.3g} "
                f"max_ulp={self.max_ulp:.3g} within_1ulp={self.within_1ulp:.5f} "
                f"outside_bf16_policy={self.outside_policy} worst={self.worst}")


def compare(name: str, gpu: torch.Tensor, exact: np.ndarray, scale: np.ndarray, out_dtype: torch.dtype,
            rel: float = REL_ELEM, alt: Optional[np.ndarray] = None) -> Report:
    g = gpu.detach().to("cpu", torch.float64).numpy().reshape(exact.shape)
    ex = np.asarray(exact, dtype=np.float64)
    err = np.abs(g - ex)
    if alt is not None:
        err = np.minimum(err, np.abs(g - np.asarray(alt, dtype=np.float64)))
    u = ulp(np.maximum(np.abs(g), np.abs(ex)), out_dtype)
    if out_dtype in (torch.bfloat16, torch.float16):
        bound = u + rel * np.asarray(scale, dtype=np.float64)
    else:
        bound = rel * np.asarray(scale, dtype=np.float64) + 4 * FLT_MIN
    both_nan = np.isnan(g) & np.isnan(ex)
    same_inf = np.isinf(g) & np.isinf(ex) & (np.sign(g) == np.sign(ex))
    good = (err <= bound) | both_nan | same_inf
    bad = int((~good).sum())
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(good & ~(both_nan | same_inf), err / np.maximum(bound, 1e-300), 0.0)
        ratio = np.where(good, ratio, np.inf)
        ulps = np.where(both_nan | same_inf, 0.0, err / u)
    worst = None
    if err.size:
        k = int(np.nanargmax(np.where(np.isfinite(ratio), ratio, 1e300)))
        idx = np.unravel_index(k, err.shape)
        worst = (tuple(int(i) for i in idx), float(g.reshape(err.shape)[idx]), float(ex[idx]), float(bound[idx]))
    policy_bad = int((~((err <= 2.0 ** -6 + 2.0 ** -6 * np.abs(ex)) | both_nan | same_inf)).sum())
    return Report(name, int(err.size), bad,
                  float(np.max(ratio)) if ratio.size else 0.0,
                  float(np.nanmax(ulps)) if ulps.size else 0.0,
                  float(np.mean(ulps <= 1.0)) if ulps.size else 1.0, worst, policy_bad)


def compare_param(name: str, gpu: torch.Tensor, exact: np.ndarray, abs_sum: np.ndarray,
                  param_dtype: torch.dtype, slack: Optional[np.ndarray] = None) -> Report:
    """Parameter gradients: |gpu - exact| <= 1e-4 * sum|terms| + one ulp of the param dtype
    (+ the oracle's slack for admissible alternative roundings inside the terms)."""
    g = gpu.detach().to("cpu", torch.float64).numpy().reshape(-1)
    ex = np.asarray(exact, dtype=np.float64).reshape(-1)
    err = np.abs(g - ex)
    u = ulp(np.maximum(np.abs(g), np.abs(ex)), param_dtype)
    bound = REL_PARAM * np.asarray(abs_sum, dtype=np.float64).reshape(-1) + u
    if slack is not None:
        bound = bound + np.asarray(slack, dtype=np.float64).reshape(-1)
    good = err <= bound
    bad = int((~good).sum())
    ratio = np.where(good, err / np.maximum(bound, 1e-300), np.inf)
    worst = None
    if err.size:
        k = int(np.argmax(np.where(np.isfinite(ratio), ratio, 1e300)))
        worst = (k, float(g[k]), float(ex[k]), float(bound[k]))
    return Report(name, int(err.size), bad, float(np.max(ratio)) if ratio.size else 0.0,
                  float(np.max(err / u)) if err.size else 0.0,
                  float(np.mean(err <= u)) if err.size else 1.0, worst,
                  int((err > 2.0 ** -6 + 2.0 ** -6 * np.abs(ex)).sum()))


def merge(reports) -> Report:
    """One report over the union of several reports' elements (e.g. row chunks of a tensor)."""
    reports = list(reports)
    n = sum(r.n for r in reports)
    worst = max(reports, key=lambda r: r.max_ratio)
    return Report(reports[0].name, n, sum(r.bad for r in reports), max(r.max_ratio for r in reports),
                  max(r.max_ulp for r in reports),
                  sum(r.within_1ulp * r.n for r in reports) / n if n else 1.0, worst.worst,
                  sum(r.outside_policy for r in reports))


def assert_reports(reports) -> None:
    failed = [str(r) for r in reports if not r.ok()]
    assert not failed, "\n".join(failed)
