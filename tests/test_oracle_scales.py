"""Pins of the oracle's tolerance scales (CPU).

Every GPU-vs-oracle bound is 1e-5 (elements) or 1e-4 (parameter gradients) times a magnitude
sum S that the oracle returns beside each exact value: the sum of the magnitudes of the terms
that form the value, which is what bounds the float32 rounding error of any evaluation order.
These tests fix S independently of the oracle's hand-expanded formulas:

1. Absolute-value evaluation.  Each layer's defining expression is evaluated once more with
   ``Mag`` numbers, which carry beside every value the same expression evaluated with each leaf
   replaced by its magnitude and each subtraction by an addition.  That is the magnitude sum by
   definition; it must equal every ``*_scale`` output.  The leaves are the quantities a kernel
   reads or forms in one rounding (inputs, parameters, rstd, tanh and sech^2, the RMSNorm
   rounding points).
2. Closed forms for the admissible-rounding window of RMSNorm (``y_alt``, ``dweight_slack``):
   inputs whose normalized value sits a known distance from a bfloat16 / float16 midpoint.
3. Controls.  Not too tight: an independent float32 implementation (torch eager, with autograd)
   on inputs with cancellation (odd widths, a large row mean, 1% x10 outliers) passes every
   bound.  Not too loose: results with a planted error (a dropped term, a relative error of a
   few 1e-5, an extra row) fail.

tests/test_oracle_mutants.py plants mistakes in the scales (a dropped term, x10, xN, an
absolute value in the wrong place, a wider tie window) and checks that these tests catch them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests import tolerance as tol

F64 = np.float64


# ----------------------------------------------------------------------- Mag numbers

class Mag:
    """A value and the magnitude sum of the terms that form it (elementwise numpy arrays)."""

    __array_priority__ = 100

    def __init__(self, v, m=None):
        self.v = np.asarray(v, dtype=F64)
        self.m = np.abs(self.v) if m is None else np.asarray(m, dtype=F64)

    @staticmethod
    def lift(o):
        return o if isinstance(o, Mag) else Mag(o)

    def __add__(self, o):
        o = Mag.lift(o)
        return Mag(self.v + o.v, self.m + o.m)

    __radd__ = __add__

    def __sub__(self, o):
        o = Mag.lift(o)
        return Mag(self.v - o.v, self.m + o.m)

    def __rsub__(self, o):
        return Mag.lift(o) - self

    def __mul__(self, o):
        o = Mag.lift(o)
        return Mag(self.v * o.v, self.m * o.m)

    __rmul__ = __mul__

    def sum(self, axis=None, keepdims=False):
        return Mag(self.v.sum(axis=axis, keepdims=keepdims), self.m.sum(axis=axis, keepdims=keepdims))

    def mean(self, axis, keepdims=False):
        n = self.v.shape[axis]
        return self.sum(axis, keepdims) * (1.0 / n)


def vals(t: torch.Tensor) -> np.ndarray:
    """The exact float64 values of a host tensor's elements."""
    return t.to(torch.float64).numpy()


def close(a, b):
    np.testing.assert_allclose(np.asarray(a, F64), np.asarray(b, F64), rtol=1e-10, atol=0)


def _data(M, N, xdt, seed, mean=0.0, std=1.0, outliers=0.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, N, generator=g, dtype=torch.float64) * std + mean
    if outliers:
        x = torch.where(torch.rand(M, N, generator=g, dtype=torch.float64) < outliers, x * 10, x)
    dy = torch.randn(M, N, generator=g, dtype=torch.float64)
    gam = 1 + 0.3 * torch.randn(N, generator=g, dtype=torch.float64)
    bet = 0.3 * torch.randn(N, generator=g, dtype=torch.float64)
    return x.to(xdt), dy.to(xdt), gam, bet


CASES = [  # (M, N, x dtype, param dtype, row mean, std, outlier fraction)
    (7, 5, torch.float32, torch.float32, 0.0, 3.0, 0.0),
    (9, 33, torch.float32, torch.float32, 40.0, 0.5, 0.0),
    (6, 1025, torch.bfloat16, torch.float32, 0.0, 1.0, 0.01),
    (5, 64, torch.bfloat16, torch.bfloat16, -3.0, 0.25, 0.0),
    (4, 31, torch.float16, torch.float16, 2.0, 2.0, 0.02),
]


@pytest.mark.parametrize("M,N,xdt,pdt,mu,sd,out", CASES)
def test_dyt_scales_are_magnitude_sums(M, N, xdt, pdt, mu, sd, out):
    x, dy, gam, bet = _data(M, N, xdt, M * N, mu, sd, out)
    gam, bet = gam.to(pdt), bet.to(pdt)
    alpha = torch.tensor([0.7], dtype=pdt)
    a = float(alpha.double())
    X, DY, G, B = Mag(vals(x)), Mag(vals(dy)), Mag(vals(gam)), Mag(vals(bet))
    z = a * vals(x)
    T = Mag(np.tanh(z))                       # one rounding each: leaves
    AS = Mag(a / np.cosh(z) ** 2)             # alpha * sech^2
    S = Mag(1.0 / np.cosh(z) ** 2)
    y = G * T + B
    dx = DY * G * AS
    dgamma = (DY * T).sum(0)
    dbeta = DY.sum(0)
    dalpha = (DY * G * X * S).sum()
    f = oracle.dyt_fwd(x, alpha, gam, bet)
    b = oracle.dyt_bwd(x, dy, alpha, gam)
    close(f["y_scale"], y.m)
    close(b["dx_scale"], dx.m)
    close(b["dgamma_scale"], dgamma.m)
    close(b["dbeta_scale"], dbeta.m)
    close(b["dalpha_scale"], [dalpha.m])


@pytest.mark.parametrize("M,N,xdt,pdt,mu,sd,out", CASES)
def test_layernorm_scales_are_magnitude_sums(M, N, xdt, pdt, mu, sd, out):
    x, dy, gam, bet = _data(M, N, xdt, M + N, mu, sd, out)
    gam, bet = gam.to(pdt), bet.to(pdt)
    eps = 1e-5
    xv = vals(x)
    var = ((xv - xv.mean(1, keepdims=True)) ** 2).mean(1, keepdims=True)
    X, DY, G, B = Mag(xv), Mag(vals(dy)), Mag(vals(gam)), Mag(vals(bet))
    R = Mag(1.0 / np.sqrt(var + eps))         # rstd: a leaf (its own error is relative)
    mu_ = X.mean(1, keepdims=True)
    xh = (X - mu_) * R
    y = xh * G + B
    g = DY * G
    c1 = g.mean(1, keepdims=True)
    c2 = (g * xh).mean(1, keepdims=True)
    dx = R * (g - c1 - xh * c2)
    v = ((X - mu_) * (X - mu_)).mean(1)
    f = oracle.layernorm_fwd(x, gam, bet, eps)
    b = oracle.layernorm_bwd(x, dy, gam, eps)
    close(f["y_scale"], y.m)
    close(f["mean_scale"], mu_.m[:, 0])
    # rstd = (var + eps)^(-1/2): relative error half that of var + eps; the scale doubles it
    r = R.v[:, 0]
    close(f["rstd_scale"], r * (v.m + eps) / (v.v + eps))
    close(b["dx_scale"], dx.m)
    close(b["dgamma_scale"], (DY * xh).sum(0).m)
    close(b["dbeta_scale"], DY.sum(0).m)


def _round(v: np.ndarray, dt: torch.dtype) -> np.ndarray:
    """Round float64 values to dt (round to nearest even), via the oracle's pinned rounding."""
    if dt == torch.float32:
        return oracle.round_f32(v)
    return oracle.round_bf16(v) if dt == torch.bfloat16 else oracle.round_f16(v)


@pytest.mark.parametrize("M,N,xdt,pdt,mu,sd,out", CASES)
@pytest.mark.parametrize("form", ["cast_then_weight", "weight_then_cast", "one_plus_weight"])
def test_rmsnorm_scales_are_magnitude_sums(M, N, xdt, pdt, mu, sd, out, form):
    x, dy, w, _ = _data(M, N, xdt, 3 * M + N, mu, sd, out)
    w = w.to(pdt)
    eps = 1e-6
    xv, dyv, wv = vals(x), vals(dy), vals(w)
    X, DY = Mag(xv), Mag(dyv)
    R = Mag(1.0 / np.sqrt((xv * xv).mean(1, keepdims=True) + eps))
    H = X * R
    if form == "cast_then_weight":
        n = _round(H.v, xdt)                                       # the rounding point
        y = Mag(wv) * Mag(n)
        G = Mag(_round(_round(dyv * wv, torch.float32), xdt))      # grad of n, rounded
        dwt = Mag(_round(_round(dyv * n, torch.float32), pdt))     # rounded product per term
        dw = dwt.sum(0)
    else:
        s = wv if form == "weight_then_cast" else _round(1.0 + wv, torch.float32)
        y = Mag(s) * H
        G = DY * Mag(s)
        dw = (DY * H).sum(0)
    c = (G * H).mean(1, keepdims=True)
    dx = R * (G - H * c)
    f = oracle.rmsnorm_fwd(x, w, eps, form=form)
    b = oracle.rmsnorm_bwd(x, dy, w, eps, form=form)
    np.testing.assert_allclose(f["y_scale"], y.m, rtol=2 ** -23)   # |y| vs |float32(y)|
    close(b["dx_scale"], dx.m)
    close(b["dweight_scale"], dw.m)


# ------------------------------------------------ closed forms: the admissible-rounding window

# RMSNorm's n = round(x * rstd) may round either way when x * rstd lies within float32 error of
# a midpoint between two values of x's dtype: |h - mid| <= 2^-18 |h| (a float32 h carries a few
# roundings of ~2^-24 each; the window is wider by a margin).  With x = 1 in every column, eps
# sets h = 1 / sqrt(1 + eps) exactly to a chosen distance from the midpoint below 1.

@pytest.mark.parametrize("xdt,bits", [(torch.bfloat16, 8), (torch.float16, 11)])
@pytest.mark.parametrize("k", [-40, -12, -6, -3, 3, 6, 12, 40])
def test_rmsnorm_tie_window_closed_form(xdt, bits, k):
    lo, hi = 1.0 - 2.0 ** -bits, 1.0                   # neighbours below 1
    mid = 0.5 * (lo + hi)
    h = mid * (1.0 + k * 2.0 ** -20)                  # |h - mid| = |k| 2^-20 mid
    eps = 1.0 / (h * h) - 1.0
    N = 4
    x = torch.ones(1, N, dtype=xdt)
    w = torch.full((N,), 3.0, dtype=xdt)              # exact in both dtypes
    dy = torch.ones(1, N, dtype=xdt)
    f = oracle.rmsnorm_fwd(x, w, eps)
    b = oracle.rmsnorm_bwd(x, dy, w, eps)
    n = lo if k < 0 else hi
    other = hi if k < 0 else lo
    inside = abs(k) * 2.0 ** -20 * mid <= 2.0 ** -18 * h
    assert inside == (abs(k) <= 3)
    np.testing.assert_array_equal(f["y"], np.full((1, N), 3.0 * n))
    np.testing.assert_array_equal(f["y_alt"], np.full((1, N), 3.0 * (other if inside else n)))
    # dweight term = round(dy * n) = n; its other admissible value is `other`
    np.testing.assert_array_equal(b["dweight"], np.full(N, n))
    np.testing.assert_array_equal(b["dweight_slack"], np.full(N, abs(other - n) if inside else 0.0))


# ------------------------------------------------------------------------- controls

def _eager_fp32(layer, x, dy, params, eps, form="cast_then_weight"):
    """An independent implementation: torch eager (CPU) with autograd, float32 arithmetic,
    outputs rounded once to x's dtype and gradients to the parameters' dtype.  The RMSNorm
    Llama form runs its eager expression in x's dtype, rounding points included."""
    xdt = x.dtype
    pdt = next(iter(params.values())).dtype
    xf = x.detach().to(torch.float32, copy=True).requires_grad_(True)
    ps = {k: v.detach().to(torch.float32, copy=True).requires_grad_(True) for k, v in params.items()}
    if layer == "dyt":
        y = ps["gamma"] * torch.tanh(ps["alpha"] * xf) + ps["beta"]
    elif layer == "layernorm":
        y = F.layer_norm(xf, (x.shape[1],), ps["gamma"], ps["beta"], eps)
    elif form == "cast_then_weight":
        xl = x.detach().clone().requires_grad_(True)
        wl = params["weight"].detach().clone().requires_grad_(True)
        xs = xl.float()
        y = wl * (xs * torch.rsqrt(xs.pow(2).mean(-1, keepdim=True) + eps)).to(xdt)
        y = y.to(xdt)
        y.backward(dy.to(y.dtype))
        return {"y": y.detach(), "dx": xl.grad.to(xdt), "dweight": wl.grad.to(pdt)}
    else:
        s = ps["weight"] if form == "weight_then_cast" else 1.0 + ps["weight"]
        y = s * (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps))
    y.backward(dy.float())
    out = {"y": y.detach().to(xdt), "dx": xf.grad.to(xdt)}
    out.update({"d" + k: v.grad.to(pdt) for k, v in ps.items()})
    if layer == "dyt":
        # autograd's tanh derivative is 1 - tanh^2, which cancels in float32 where tanh
        # saturates: relative errors of ~1e-3 on dx at |alpha x| ~ 5, and 0 instead of ~1e-13
        # per term at |alpha x| ~ 15, outside the bounds.  sech^2 = 1 / cosh^2 in float32 has no
        # such cancellation; the gradients are formed from it with float32 torch ops.
        with torch.no_grad():
            a, g = ps["alpha"], ps["gamma"]
            xf32, dyf = x.float(), dy.float()
            s2 = 1.0 / torch.cosh(a * xf32) ** 2
            out["dx"] = (dyf * g * a * s2).to(xdt)
            out["dgamma"] = (dyf * torch.tanh(a * xf32)).sum(0).to(pdt)
            out["dbeta"] = dyf.sum(0).to(pdt)
            out["dalpha"] = (dyf * g * xf32 * s2).sum().reshape(1).to(pdt)
    return out


def _oracle_all(layer, x, dy, params, eps, form="cast_then_weight"):
    if layer == "dyt":
        f = oracle.dyt_fwd(x, params["alpha"], params["gamma"], params["beta"])
        b = oracle.dyt_bwd(x, dy, params["alpha"], params["gamma"])
    elif layer == "layernorm":
        f = oracle.layernorm_fwd(x, params["gamma"], params["beta"], eps)
        b = oracle.layernorm_bwd(x, dy, params["gamma"], eps)
    else:
        f = oracle.rmsnorm_fwd(x, params["weight"], eps, form=form)
        b = oracle.rmsnorm_bwd(x, dy, params["weight"], eps, form=form)
    return {**f, **b}


def _reports(layer, got, o, xdt, pdt):
    reps = [tol.compare(f"{layer}.y", got["y"], o["y"], o["y_scale"], xdt, alt=o.get("y_alt")),
            tol.compare(f"{layer}.dx", got["dx"], o["dx"], o["dx_scale"], xdt)]
    for n in {"dyt": ["dgamma", "dbeta", "dalpha"], "layernorm": ["dgamma", "dbeta"], "rmsnorm": ["dweight"]}[layer]:
        reps.append(tol.compare_param(f"{layer}.{n}", got[n], o[n], o[n + "_scale"], pdt, slack=o.get(n + "_slack")))
    return reps


def _params(layer, N, pdt, seed):
    g = torch.Generator().manual_seed(seed)
    p = {"gamma": (1 + 0.1 * torch.randn(N, generator=g)).to(pdt), "beta": (0.1 * torch.randn(N, generator=g)).to(pdt)}
    if layer == "dyt":
        p["alpha"] = torch.tensor([0.5]).to(pdt)
    if layer == "rmsnorm":
        p = {"weight": p["gamma"]}
    return p


CONTROL = [  # (M, N, x dtype, param dtype, row mean, std, outliers)
    (64, 1025, torch.float32, torch.float32, 0.0, 1.0, 0.01),
    (64, 1025, torch.bfloat16, torch.float32, 0.0, 1.0, 0.01),
    (48, 771, torch.float32, torch.float32, 30.0, 1.0, 0.0),
    (48, 771, torch.bfloat16, torch.bfloat16, 30.0, 1.0, 0.0),
    (2048, 24, torch.float32, torch.float32, 0.0, 2.0, 0.0),
    (32, 333, torch.float16, torch.float16, 1.0, 1.0, 0.01),
]


@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("M,N,xdt,pdt,mu,sd,out", CONTROL)
def test_independent_float32_path_passes_every_bound(layer, M, N, xdt, pdt, mu, sd, out):
    """Not too tight: torch eager in float32 (or the pages' eager RMSNorm expression in x's
    dtype) is a correct float32 implementation with its own summation orders; every bound
    admits it, also where rows cancel (large mean, outliers, odd widths)."""
    x, dy, _, _ = _data(M, N, xdt, M * 7 + N, mu, sd, out)
    params = _params(layer, N, pdt, N)
    eps = {"dyt": 0.0, "layernorm": 1e-5, "rmsnorm": 1e-6}[layer]
    got = _eager_fp32(layer, x, dy, params, eps)
    o = _oracle_all(layer, x, dy, params, eps)
    reps = _reports(layer, got, o, xdt, pdt)
    tol.assert_reports(reps)


@pytest.mark.parametrize("form", ["weight_then_cast", "one_plus_weight"])
def test_independent_float32_path_passes_rmsnorm_forms(form):
    x, dy, _, _ = _data(48, 771, torch.bfloat16, 5, 0.0, 1.0, 0.01)
    params = _params("rmsnorm", 771, torch.float32, 9)
    got = _eager_fp32("rmsnorm", x, dy, params, 1e-6, form=form)
    o = _oracle_all("rmsnorm", x, dy, params, 1e-6, form=form)
    tol.assert_reports(_reports("rmsnorm", got, o, torch.bfloat16, torch.float32))


def _fails(reps) -> bool:
    return any(not r.ok() for r in reps)


@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
def test_planted_errors_fail_the_bounds(layer):
    """Not too loose: each planted error makes some bound fail."""
    M, N = 4, 96
    x, dy, _, _ = _data(M, N, torch.float32, 77, 0.0, 1.0, 0.0)
    if layer == "dyt":
        dy = dy.abs() * torch.sign(x)       # same-signed dalpha terms: the sum does not cancel
    params = _params(layer, N, torch.float32, 3)
    eps = {"dyt": 0.0, "layernorm": 1e-5, "rmsnorm": 1e-6}[layer]
    o = _oracle_all(layer, x, dy, params, eps)
    exact = {k: torch.from_numpy(np.asarray(o[k])) for k in o if not k.endswith(("_scale", "_slack", "_alt"))}
    gnames = {"dyt": ["dgamma", "dbeta", "dalpha"], "layernorm": ["dgamma", "dbeta"], "rmsnorm": ["dweight"]}[layer]

    def with_(k, v):
        d = {n: exact[n] for n in ["y", "dx"] + gnames}
        d[k] = v
        return _reports(layer, d, o, torch.float32, torch.float32)

    assert not _fails(with_("y", exact["y"]))                          # the exact values pass
    assert _fails(with_("y", exact["y"] * (1 + 5e-5)))                 # 5e-5 relative on y
    assert _fails(with_("dx", exact["dx"] * (1 + 5e-5)))               # 5e-5 relative on dx
    for n in gnames:
        assert _fails(with_(n, exact[n] * (1 + 5e-4))), n              # 5e-4 relative on a gradient
    # a gradient missing one row's terms, or taking one more
    xr, dyr = x[1:], dy[1:]
    o1 = _oracle_all(layer, xr, dyr, params, eps)
    for n in gnames:
        assert _fails(with_(n, torch.from_numpy(np.asarray(o1[n])))), n
    # a dropped term in dx
    if layer == "layernorm":
        xv, dyv, gv = vals(x), vals(dy), vals(params["gamma"])
        mu_ = xv.mean(1, keepdims=True)
        r = 1 / np.sqrt(((xv - mu_) ** 2).mean(1, keepdims=True) + eps)
        g = dyv * gv
        assert _fails(with_("dx", torch.from_numpy(r * (g - g.mean(1, keepdims=True)))))          # no x_hat * c2
        assert _fails(with_("dx", torch.from_numpy(r * (g - ((xv - mu_) * r) * (g * (xv - mu_) * r).mean(1, keepdims=True)))))  # no c1
    if layer == "rmsnorm":
        xv, dyv, wv = vals(x), vals(dy), vals(params["weight"])
        r = 1 / np.sqrt((xv * xv).mean(1, keepdims=True) + eps)
        assert _fails(with_("dx", torch.from_numpy(r * _round(_round(dyv * wv, torch.float32), torch.float32))))  # no h * c
    if layer == "dyt":
        assert _fails(with_("dx", exact["dx"] / 0.5))                  # alpha dropped


def test_rmsnorm_bf16_weight_gradient_needs_its_rounded_terms():
    """Not too loose for the rounding points: with few rows, summing the unrounded products
    dy * n instead of their bfloat16 roundings fails the weight-gradient bound."""
    x, dy, w, _ = _data(2, 512, torch.bfloat16, 11, 0.0, 1.0, 0.0)
    w = w.to(torch.bfloat16)
    o = oracle.rmsnorm_bwd(x, dy, w, 1e-6)
    f = oracle.rmsnorm_fwd(x, w, 1e-6)
    n = _round(vals(x) * f["rstd"][:, None], torch.bfloat16)
    unrounded = (vals(dy) * n).sum(0)
    got = torch.from_numpy(_round(unrounded, torch.bfloat16))
    rep = tol.compare_param("rmsnorm.dweight", got, o["dweight"], o["dweight_scale"], torch.bfloat16,
                            slack=o["dweight_slack"])
    assert not rep.ok()
