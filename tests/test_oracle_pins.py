"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against one of: a textbook identity, a closed form the pages
print, finite differences of the oracle's own forward, torch's library routines in float64,
exact rational arithmetic on tiny inputs, or an invariant of the mathematics.  Together they
are chosen so that a dropped term, a wrong sign or index, a missing rounding point or a
transposed operand in the oracle fails at least one of them (test_oracle_mutants.py plants
such mistakes and checks exactly that).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _randn(shape, seed, dtype=torch.float64, scale=1.0, shift=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * scale + shift).to(dtype)


# ------------------------------------------------------------------------ bfloat16 rounding

def test_round_bf16_matches_torch_rne_on_float32_values():
    """Every float32 value rounds to the same bfloat16 as torch's float32 -> bfloat16 cast
    (round to nearest, ties to even), including exact ties, subnormals and overflow."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=300000, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi | 0x0001, hi | 0xFFFF])
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0x00000001,
                        0x80000000, 0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32)
    vals = np.concatenate([bits, ties, special]).view(np.float32)
    vals = vals[np.isfinite(vals)]
    expect = torch.from_numpy(vals.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(vals.astype(np.float64))
    assert np.array_equal(got, expect)


def test_round_bf16_rounds_doubles_directly_not_through_float32():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1).  A double just above the tie must
    # round up, although its float32 rounding would land exactly on the tie.
    assert oracle.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7
    assert oracle.round_bf16(np.array([-(1 + 2 ** -8 + 2 ** -40)]))[0] == -(1 + 2 ** -7)
    assert oracle.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])
    assert oracle.round_bf16(np.array([2.0 ** 128]))[0] == np.inf


# ------------------------------------------------------------------------- float16 values

def _all_f16():
    return torch.arange(0, 2 ** 16, dtype=torch.int32).to(torch.int16).view(torch.float16)


def test_f16_values_read_exactly():
    """Every binary16 bit pattern reads as the value torch's exact float16 -> float64
    conversion gives (subnormals, infinities and NaNs included)."""
    h = _all_f16()
    got = oracle.load_values(h)
    expect = h.to(torch.float64).numpy()
    nan = np.isnan(expect)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], expect[~nan])


def _f16_nearest_brute_force(vals):
    """Round to nearest float16, ties to the even bit pattern, by search over every finite
    float16 value; beyond 65504 the next step (65536) stands for infinity."""
    h = _all_f16()
    v = h.to(torch.float64).numpy()
    bits = h.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    fin = np.isfinite(v) & (bits < 0x8000)            # non-negative finite values, ascending
    mags, mbits = v[fin], bits[fin]
    order = np.argsort(mags, kind="stable")
    mags, mbits = mags[order], mbits[order]
    mags = np.append(mags, 65536.0)
    mbits = np.append(mbits, 0x7C00)
    out = []
    for x in vals:
        a = abs(x)
        k = int(np.searchsorted(mags, a, side="left"))
        if k == len(mags):
            r = 65536.0
        elif mags[k] == a:
            r = mags[k]
        else:
            lo, hi = mags[k - 1], mags[k]
            dlo, dhi = a - lo, hi - a
            if dlo < dhi or (dlo == dhi and mbits[k - 1] % 2 == 0):
                r = lo
            else:
                r = hi
        r = np.inf if r == 65536.0 else r
        out.append(math.copysign(r, x))
    return np.array(out)


def test_round_f16_against_brute_force_nearest():
    """Exact ties (midpoints of neighbouring float16 values), values one double ulp either side
    of them, the subnormal range, the overflow threshold and log-uniform random doubles."""
    h = _all_f16().to(torch.float64).numpy()
    pos = np.unique(h[np.isfinite(h) & (h >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2                     # exact in float64
    rng = np.random.default_rng(5)
    pick = rng.choice(len(mids), size=3000, replace=False)
    m = mids[pick]
    rand = np.exp2(rng.uniform(-30, 17, size=3000)) * rng.choice([-1.0, 1.0], size=3000)
    special = np.array([65504.0, 65519.99, 65520.0, 65520.0 - 2 ** -20, 2.0 ** -24, 2.0 ** -25,
                        3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1e9, -1e9])
    vals = np.concatenate([m, np.nextafter(m, 0), np.nextafter(m, np.inf), -m, rand, special])
    got = oracle.round_f16(vals)
    assert np.array_equal(got, _f16_nearest_brute_force(vals))


def test_round_f16_matches_torch_on_float32_values():
    """On float32 inputs the rounding agrees with torch's float32 -> float16 cast."""
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    expect = torch.from_numpy(vals.copy()).to(torch.float16).to(torch.float64).numpy()
    got = oracle.round_f16(vals.astype(np.float64))
    assert np.array_equal(got, expect)


# ---------------------------------------------------------------------------- DyT pins

def _tanh_cases():
    with open(os.path.join(GOLDEN, "tanh_identities.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _tanh_cases(), ids=lambda c: f"a={c['a']}")
def test_dyt_at_closed_form_tanh_points(case):
    """alpha = ln a and x = +-1 give tanh(alpha x) = +-(a^2-1)/(a^2+1) and
    sech^2 = 4a^2/(a^2+1)^2 (closed forms), so y, dx, dgamma, dbeta, dalpha are known."""
    a, t, s2 = case["a"], case["tanh"], case["sech2"]
    alpha = math.log(a)
    x = torch.tensor([[1.0, -1.0, 1.0], [-1.0, 1.0, 1.0]], dtype=torch.float64)
    gamma = torch.tensor([1.5, -0.5, 2.0], dtype=torch.float64)
    beta = torch.tensor([0.25, 0.0, -1.0], dtype=torch.float64)
    dy = torch.tensor([[1.0, 2.0, -1.0], [0.5, -3.0, 1.0]], dtype=torch.float64)
    fw = oracle.dyt_fwd(x, alpha, gamma, beta)
    sign = x.numpy()
    np.testing.assert_allclose(fw["y"], gamma.numpy() * t * sign + beta.numpy(), rtol=1e-14, atol=1e-15)
    bw = oracle.dyt_bwd(x, dy, alpha, gamma)
    np.testing.assert_allclose(bw["dx"], dy.numpy() * gamma.numpy() * alpha * s2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(bw["dgamma"], (dy.numpy() * t * sign).sum(0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(bw["dbeta"], dy.numpy().sum(0), rtol=1e-15)
    np.testing.assert_allclose(bw["dalpha"][0], (dy.numpy() * gamma.numpy() * sign * s2).sum(), rtol=1e-13)


def test_dyt_alpha_zero():
    """alpha = 0: tanh(0) = 0 and sech^2(0) = 1, so y = beta and dx = 0 exactly, dgamma = 0,
    dbeta_j = sum_i dy_ij and dalpha = sum_ij dy * gamma * x (correctly rounded sums)."""
    x, dy = _randn((37, 9), 1), _randn((37, 9), 2)
    gamma, beta = _randn(9, 3, shift=1.0), _randn(9, 4)
    fw = oracle.dyt_fwd(x.float(), 0.0, gamma.float(), beta.float())
    assert np.array_equal(fw["y"], np.broadcast_to(beta.float().double().numpy(), (37, 9)))
    bw = oracle.dyt_bwd(x, dy, 0.0, gamma)
    assert np.all(bw["dx"] == 0.0) and np.all(bw["dgamma"] == 0.0)
    exp_db = [math.fsum(dy[:, j].tolist()) for j in range(9)]
    np.testing.assert_allclose(bw["dbeta"], exp_db, rtol=1e-14)
    exp_da = math.fsum((dy * gamma * x).reshape(-1).tolist())
    np.testing.assert_allclose(bw["dalpha"][0], exp_da, rtol=1e-13)


def test_dyt_alpha_inf_gives_finite_gradients():
    """alpha = +inf, x != 0: y = gamma*sign(x) + beta, dx = 0, dalpha = 0, dgamma_j =
    sum_i dy*sign(x), dbeta_j = sum_i dy -- all finite.  At x = 0 the product inf*0 is NaN
    (Liger-Kernel PR #1617, Summary: tanh(inf * 0) is NaN)."""
    x = _randn((50, 6), 5, dtype=torch.float32)
    assert bool((x != 0).all())
    dy, gamma, beta = _randn((50, 6), 6, torch.float32), _randn(6, 7, torch.float32, shift=1.0), _randn(6, 8, torch.float32)
    fw = oracle.dyt_fwd(x, math.inf, gamma, beta)
    sg = np.sign(x.double().numpy())
    np.testing.assert_array_equal(fw["y"], gamma.double().numpy() * sg + beta.double().numpy())
    bw = oracle.dyt_bwd(x, dy, math.inf, gamma)
    assert np.all(bw["dx"] == 0.0) and bw["dalpha"][0] == 0.0
    dyd = dy.double().numpy()
    np.testing.assert_allclose(bw["dgamma"], [math.fsum((dyd[:, j] * sg[:, j]).tolist()) for j in range(6)], rtol=1e-14)
    np.testing.assert_allclose(bw["dbeta"], [math.fsum(dyd[:, j].tolist()) for j in range(6)], rtol=1e-14)
    x0 = x.clone()
    x0[3, 2] = 0.0
    assert np.isnan(oracle.dyt_fwd(x0, math.inf, gamma, beta)["y"][3, 2])


def test_dyt_is_odd_around_beta():
    x = _randn((11, 13), 9)
    g, b = _randn(13, 10), _randn(13, 11)
    yp = oracle.dyt_fwd(x, 0.7, g, b)["y"] - b.numpy()
    ym = oracle.dyt_fwd(-x, 0.7, g, b)["y"] - b.numpy()
    np.testing.assert_allclose(yp, -ym, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ finite differences

def _fd_check(forward, backward, inputs, names, seed, h_rel=1e-6, tol=2e-7):
    """Central differences of L = sum(y * dy) against the oracle's backward, for every
    element of every named input (float64 inputs, no rounding points)."""
    y0 = forward(inputs)
    dy = _randn(y0.shape, seed)
    grads = backward(inputs, dy)

    def loss(inp):
        return float((forward(inp) * dy.numpy()).sum())

    for name in names:
        base = inputs[name]
        flat = base.reshape(-1)
        an = np.asarray(grads[name], dtype=np.float64).reshape(-1)
        for k in range(flat.numel()):
            v = float(flat[k])
            h = h_rel * max(1.0, abs(v))
            up = dict(inputs); dn = dict(inputs)
            pu = base.clone().reshape(-1); pu[k] = v + h
            pd = base.clone().reshape(-1); pd[k] = v - h
            up[name] = pu.reshape(base.shape); dn[name] = pd.reshape(base.shape)
            fd = (loss(up) - loss(dn)) / (2 * h)
            assert abs(fd - an[k]) <= tol * (1.0 + abs(an[k])), (name, k, fd, an[k])


@pytest.mark.parametrize("seed", [11, 12, 13])
@pytest.mark.parametrize("shape", [(3, 5), (2, 1), (1, 7)])
def test_dyt_backward_matches_finite_differences(seed, shape):
    M, N = shape
    inp = {"x": _randn((M, N), seed), "alpha": torch.tensor([0.8]), "gamma": _randn(N, seed + 1, shift=1.0),
           "beta": _randn(N, seed + 2)}
    inp["alpha"] = inp["alpha"].double()

    def fwd(d):
        return oracle.dyt_fwd(d["x"], float(d["alpha"][0]), d["gamma"], d["beta"])["y"]

    def bwd(d, dy):
        r = oracle.dyt_bwd(d["x"], dy, float(d["alpha"][0]), d["gamma"])
        return {"x": r["dx"], "alpha": r["dalpha"], "gamma": r["dgamma"], "beta": r["dbeta"]}

    _fd_check(fwd, bwd, inp, ["x", "alpha", "gamma", "beta"], seed + 100)


@pytest.mark.parametrize("seed", [21, 22, 23])
@pytest.mark.parametrize("shape", [(3, 5), (2, 1), (2, 8)])
def test_layernorm_backward_matches_finite_differences(seed, shape):
    M, N = shape
    inp = {"x": _randn((M, N), seed, scale=2.0, shift=0.3), "gamma": _randn(N, seed + 1, shift=1.0),
           "beta": _randn(N, seed + 2)}
    eps = 1e-3

    def fwd(d):
        return oracle.layernorm_fwd(d["x"], d["gamma"], d["beta"], eps)["y"]

    def bwd(d, dy):
        r = oracle.layernorm_bwd(d["x"], dy, d["gamma"], eps)
        return {"x": r["dx"], "gamma": r["dgamma"], "beta": r["dbeta"]}

    _fd_check(fwd, bwd, inp, ["x", "gamma", "beta"], seed + 100)


@pytest.mark.parametrize("seed", [31, 32, 33])
@pytest.mark.parametrize("shape", [(3, 5), (2, 1), (2, 8)])
def test_rmsnorm_backward_matches_finite_differences(seed, shape):
    M, N = shape
    inp = {"x": _randn((M, N), seed, shift=0.2), "weight": _randn(N, seed + 1, shift=1.0)}
    eps = 1e-2

    def fwd(d):
        return oracle.rmsnorm_fwd(d["x"], d["weight"], eps)["y"]

    def bwd(d, dy):
        r = oracle.rmsnorm_bwd(d["x"], dy, d["weight"], eps)
        return {"x": r["dx"], "weight": r["dweight"]}

    _fd_check(fwd, bwd, inp, ["x", "weight"], seed + 100)


# --------------------------------------------------------- library cross-checks (float64)

@pytest.mark.parametrize("shape", [(17, 24), (5, 1), (3, 257)])
def test_layernorm_matches_torch_layer_norm_float64(shape):
    M, N = shape
    x = _randn((M, N), 41, scale=2.0, shift=-0.7).requires_grad_(True)
    g = _randn(N, 42, shift=1.0).requires_grad_(True)
    b = _randn(N, 43).requires_grad_(True)
    dy = _randn((M, N), 44)
    eps = 1e-5
    y = F.layer_norm(x, (N,), g, b, eps)
    y.backward(dy)
    fw = oracle.layernorm_fwd(x.detach(), g.detach(), b.detach(), eps)
    np.testing.assert_allclose(fw["y"], y.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fw["mean"], x.detach().mean(1).numpy(), rtol=1e-12, atol=1e-14)
    var = x.detach().var(1, unbiased=False).numpy()
    np.testing.assert_allclose(fw["rstd"], 1 / np.sqrt(var + eps), rtol=1e-12)
    bw = oracle.layernorm_bwd(x.detach(), dy, g.detach(), eps)
    np.testing.assert_allclose(bw["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(bw["dgamma"], g.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(bw["dbeta"], b.grad.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", [(17, 24), (5, 1), (3, 257)])
def test_rmsnorm_matches_torch_rms_norm_float64(shape):
    M, N = shape
    x = _randn((M, N), 51, shift=0.1).requires_grad_(True)
    w = _randn(N, 52, shift=1.0).requires_grad_(True)
    dy = _randn((M, N), 53)
    eps = 1e-6
    y = F.rms_norm(x, (N,), w, eps)
    y.backward(dy)
    fw = oracle.rmsnorm_fwd(x.detach(), w.detach(), eps)
    np.testing.assert_allclose(fw["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(fw["y_alt"], fw["y"])
    bw = oracle.rmsnorm_bwd(x.detach(), dy, w.detach(), eps)
    np.testing.assert_allclose(bw["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(bw["dweight"], w.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_dyt_matches_torch_autograd_float64():
    x = _randn((9, 33), 61).requires_grad_(True)
    a = torch.tensor([0.6], dtype=torch.float64, requires_grad=True)
    g = _randn(33, 62, shift=1.0).requires_grad_(True)
    b = _randn(33, 63).requires_grad_(True)
    dy = _randn((9, 33), 64)
    y = g * torch.tanh(a * x) + b
    y.backward(dy)
    bw = oracle.dyt_bwd(x.detach(), dy, 0.6, g.detach())
    np.testing.assert_allclose(bw["dx"], x.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bw["dgamma"], g.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(bw["dbeta"], b.grad.numpy(), rtol=1e-13)
    np.testing.assert_allclose(bw["dalpha"], a.grad.numpy(), rtol=1e-12)


# ---------------------------------------------------------------------- RMSNorm rounding points

def _rne(v: Fraction, bits: int = 8) -> Fraction:
    """Exact round-to-nearest-even of a rational to `bits` significant bits (normal range)."""
    if v == 0:
        return v
    s = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2; e += 1
    while a < 1:
        a *= 2; e -= 1
    scaled = a * 2 ** (bits - 1)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * Fraction(fl, 2 ** (bits - 1)) * Fraction(2) ** e


def test_rmsnorm_bf16_rounding_points_exact():
    """A tiny case worked in exact rational arithmetic with the rounding points of DeepSpeed
    PR #8645, "Semantics": n = bf16(x * rstd); y = bf16(w * n); g = bf16(dy * w);
    dw_j = sum_i bf16(dy * n).  With x = [1, 7], eps = 0: rstd = 1/5 exactly, h = [1/5, 7/5].
    The inputs are chosen so that every rounding point changes the result."""
    xs = [Fraction(1), Fraction(7)]
    ws = [Fraction(3), Fraction(193, 64)]          # 3 and 3.015625, both bfloat16
    dys = [Fraction(3), Fraction(3)]
    r = Fraction(1, 5)
    h = [xv * r for xv in xs]
    n = [_rne(v) for v in h]
    g = [_rne(d * w) for d, w in zip(dys, ws)]
    c = sum(gi * hi for gi, hi in zip(g, h)) / 2
    dx = [r * (gi - hi * c) for gi, hi in zip(g, h)]
    y_exact = [w * ni for w, ni in zip(ws, n)]
    M = 4                                           # identical rows: the column sum shows each rounding
    dw = [M * _rne(d * ni) for d, ni in zip(dys, n)]
    # Each rounding point matters here:
    assert n[0] != h[0] and g[1] != dys[1] * ws[1] and _rne(dys[0] * n[0]) != dys[0] * n[0]
    to_bf16 = lambda vals, m: torch.tensor([[float(v) for v in vals]] * m, dtype=torch.float32).to(torch.bfloat16)
    x = to_bf16(xs, M); dy = to_bf16(dys, M)
    w = torch.tensor([float(v) for v in ws], dtype=torch.float32).to(torch.bfloat16)
    fw = oracle.rmsnorm_fwd(x, w, 0.0)
    np.testing.assert_array_equal(fw["rstd"], [0.2] * M)
    for j in range(2):
        assert fw["y"][0, j] == float(y_exact[j])
    bw = oracle.rmsnorm_bwd(x, dy, w, 0.0)
    for j in range(2):
        assert math.isclose(bw["dx"][0, j], float(dx[j]), rel_tol=1e-13)
        assert bw["dweight"][j] == float(dw[j])


def test_rmsnorm_bf16_matches_eager_expression():
    """The page's eager expression evaluated by torch on the CPU in bfloat16 (float32 statistics)
    against the oracle (float64 statistics): the forward may differ only where float32 and
    float64 statistics put the normalized value on different sides of a bfloat16 rounding
    boundary (<1% of elements, never more than one step), and dx by at most a few ulp."""
    M, N = 64, 96
    xb = _randn((M, N), 71, torch.float32).to(torch.bfloat16)
    wb = _randn(N, 72, torch.float32, scale=0.02, shift=1.0).to(torch.bfloat16)
    dyb = _randn((M, N), 73, torch.float32).to(torch.bfloat16)
    eps = 1e-6
    x = xb.clone().requires_grad_(True)
    w = wb.clone().requires_grad_(True)
    xf = x.float()
    y = w * (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype)
    y.backward(dyb)
    fw = oracle.rmsnorm_fwd(xb, wb, float(np.float32(eps)))
    ora_y = oracle.round_bf16(fw["y"])
    eager_y = y.detach().double().numpy()
    same = ora_y == eager_y
    assert same.mean() >= 0.99
    ulp = np.exp2(np.floor(np.log2(np.abs(eager_y) + 1e-30)) - 7)
    assert np.all(np.abs(ora_y - eager_y) <= ulp * 1.0001)
    bw = oracle.rmsnorm_bwd(xb, dyb, wb, float(np.float32(eps)))
    ora_dx = oracle.round_bf16(bw["dx"])
    eager_dx = x.grad.double().numpy()
    assert (ora_dx == eager_dx).mean() >= 0.9
    ulpx = np.exp2(np.floor(np.log2(np.abs(eager_dx) + 1e-30)) - 7)
    assert np.all(np.abs(ora_dx - eager_dx) <= 4 * ulpx + 1e-6 * bw["dx_scale"])
    ora_dw = oracle.round_bf16(bw["dweight"])
    eager_dw = w.grad.double().numpy()
    ulpw = np.exp2(np.floor(np.log2(np.abs(eager_dw))) - 7)
    assert np.all(np.abs(ora_dw - eager_dw) <= 2 * ulpw)


def test_rmsnorm_f16_matches_eager_expression():
    """The same eager expression in float16 (float32 statistics, float16 rounding points)
    against the oracle: as for bfloat16, only rare one-step differences in y where float32 and
    float64 statistics straddle a float16 rounding boundary."""
    M, N = 64, 96
    xh = _randn((M, N), 91, torch.float32).to(torch.float16)
    wh = _randn(N, 92, torch.float32, scale=0.02, shift=1.0).to(torch.float16)
    dyh = _randn((M, N), 93, torch.float32).to(torch.float16)
    eps = 1e-6
    x = xh.clone().requires_grad_(True)
    w = wh.clone().requires_grad_(True)
    xf = x.float()
    y = w * (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype)
    y.backward(dyh)
    fw = oracle.rmsnorm_fwd(xh, wh, float(np.float32(eps)))
    ora_y = oracle.round_f16(fw["y"])
    eager_y = y.detach().double().numpy()
    assert (ora_y == eager_y).mean() >= 0.99
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.abs(eager_y) + 1e-30)), -14) - 10)
    assert np.all(np.abs(ora_y - eager_y) <= ulp * 1.0001)
    bw = oracle.rmsnorm_bwd(xh, dyh, wh, float(np.float32(eps)))
    ora_dx = oracle.round_f16(bw["dx"])
    eager_dx = x.grad.double().numpy()
    assert (ora_dx == eager_dx).mean() >= 0.9
    ulpx = np.exp2(np.maximum(np.floor(np.log2(np.abs(eager_dx) + 1e-30)), -14) - 10)
    assert np.all(np.abs(ora_dx - eager_dx) <= 4 * ulpx + 1e-6 * bw["dx_scale"])
    ora_dw = oracle.round_f16(bw["dweight"])
    eager_dw = w.grad.double().numpy()
    ulpw = np.exp2(np.floor(np.log2(np.abs(eager_dw))) - 10)
    assert np.all(np.abs(ora_dw - eager_dw) <= 2 * ulpw)


# The two float32 RMSNorm forms (DeepSpeed PR #8645, "Which modules are replaced" and "Not
# covered"): weight before the cast, and (1 + weight).

@pytest.mark.parametrize("form", ["weight_then_cast", "one_plus_weight"])
def test_rmsnorm_float32_forms_match_torch_autograd_float64(form):
    M, N, eps = 9, 40, 1e-6
    x = _randn((M, N), 101).requires_grad_(True)
    w = _randn(N, 102, scale=0.3, shift=0.2).requires_grad_(True)
    dy = _randn((M, N), 103)
    s = w if form == "weight_then_cast" else 1.0 + w
    y = s * (x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + eps))
    y.backward(dy)
    fw = oracle.rmsnorm_fwd(x.detach(), w.detach(), eps, form=form)
    bw = oracle.rmsnorm_bwd(x.detach(), dy, w.detach(), eps, form=form)
    np.testing.assert_allclose(fw["y"], y.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(bw["dx"], x.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(bw["dweight"], w.grad.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("form", ["weight_then_cast", "one_plus_weight"])
def test_rmsnorm_float32_forms_exact_small_case(form):
    """Exact rational arithmetic on x = [1, 7], eps = 0 (rstd = 1/5): no rounding of the
    normalized value or of dy * s before use, and dweight = sum over rows of dy * h."""
    xs = [Fraction(1), Fraction(7)]
    ws = [Fraction(3), Fraction(193, 64)]
    dys = [Fraction(3), Fraction(3)]
    r = Fraction(1, 5)
    sc = ws if form == "weight_then_cast" else [1 + w for w in ws]
    h = [xv * r for xv in xs]
    g = [d * sv for d, sv in zip(dys, sc)]
    c = sum(gi * hi for gi, hi in zip(g, h)) / 2
    dx = [r * (gi - hi * c) for gi, hi in zip(g, h)]
    M = 4
    to_bf16 = lambda vals, m: torch.tensor([[float(v) for v in vals]] * m, dtype=torch.float32).to(torch.bfloat16)
    x = to_bf16(xs, M); dy = to_bf16(dys, M)
    w = torch.tensor([float(v) for v in ws], dtype=torch.float32).to(torch.bfloat16)
    assert _rne(dys[1] * sc[1]) != dys[1] * sc[1]          # rounding g would change it
    fw = oracle.rmsnorm_fwd(x, w, 0.0, form=form)
    bw = oracle.rmsnorm_bwd(x, dy, w, 0.0, form=form)
    for j in range(2):
        assert math.isclose(fw["y"][0, j], float(sc[j] * h[j]), rel_tol=1e-14)
        assert math.isclose(bw["dx"][0, j], float(dx[j]), rel_tol=1e-13)
        assert math.isclose(bw["dweight"][j], float(M * dys[j] * h[j]), rel_tol=1e-14)


@pytest.mark.parametrize("form", ["weight_then_cast", "one_plus_weight"])
def test_rmsnorm_float32_forms_match_eager_bf16(form):
    """The forms' eager expressions in bfloat16 (float32 normalization, one float32 product,
    one cast) against the oracle: y within one bf16 ulp and almost always equal."""
    M, N = 64, 96
    xb = _randn((M, N), 111, torch.float32).to(torch.bfloat16)
    wb = _randn(N, 112, torch.float32, scale=0.1, shift=0.5).to(torch.bfloat16)
    dyb = _randn((M, N), 113, torch.float32).to(torch.bfloat16)
    eps = 1e-6
    x = xb.clone().requires_grad_(True)
    w = wb.clone().requires_grad_(True)
    xf = x.float()
    hf = xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)
    y = (w * hf).to(x.dtype) if form == "weight_then_cast" else (hf * (1.0 + w.float())).type_as(x)
    y.backward(dyb)
    fw = oracle.rmsnorm_fwd(xb, wb, float(np.float32(eps)), form=form)
    ora_y = oracle.round_bf16(fw["y"])
    eager_y = y.detach().double().numpy()
    assert (ora_y == eager_y).mean() >= 0.99
    ulp = np.exp2(np.floor(np.log2(np.abs(eager_y) + 1e-30)) - 7)
    assert np.all(np.abs(ora_y - eager_y) <= ulp * 1.0001)
    bw = oracle.rmsnorm_bwd(xb, dyb, wb, float(np.float32(eps)), form=form)
    ora_dx = oracle.round_bf16(bw["dx"])
    eager_dx = x.grad.double().numpy()
    assert (ora_dx == eager_dx).mean() >= 0.9
    ulpx = np.exp2(np.floor(np.log2(np.abs(eager_dx) + 1e-30)) - 7)
    assert np.all(np.abs(ora_dx - eager_dx) <= 2 * ulpx + 1e-6 * bw["dx_scale"])
    ora_dw = oracle.round_bf16(bw["dweight"])
    eager_dw = w.grad.double().numpy()
    ulpw = np.exp2(np.floor(np.log2(np.abs(eager_dw))) - 7)
    assert np.all(np.abs(ora_dw - eager_dw) <= 2 * ulpw)


def test_rmsnorm_alternative_rounding_is_rare_and_one_step():
    x = _randn((128, 64), 81, torch.float32).to(torch.bfloat16)
    w = _randn(64, 82, torch.float32, shift=1.0).to(torch.bfloat16)
    fw = oracle.rmsnorm_fwd(x, w, 1e-6)
    diff = fw["y_alt"] != fw["y"]
    assert 0 < diff.mean() < 0.01
    rel = np.abs(fw["y_alt"] - fw["y"])[diff] / np.abs(fw["y"][diff])
    assert np.all(rel < 2 ** -6)


# ------------------------------------------------------------------ closed forms and invariants

def test_rmsnorm_width_one_closed_form():
    """DeepSpeed PR #8664: at width one, d n/d x = eps / (x^2 + eps)^(3/2) (eps = 0.25)."""
    with open(os.path.join(GOLDEN, "rmsnorm_width_one.json")) as f:
        gold = json.load(f)
    eps = gold["eps"]
    xs = torch.tensor([[c["x"]] for c in gold["cases"]], dtype=torch.float64)
    w = torch.tensor([1.75], dtype=torch.float64)
    dy = torch.linspace(-2, 3, len(gold["cases"]), dtype=torch.float64).reshape(-1, 1)
    bw = oracle.rmsnorm_bwd(xs, dy, w, eps)
    expect = np.array([c["d_normalized_dx"] for c in gold["cases"]]) * dy.numpy()[:, 0] * 1.75
    np.testing.assert_allclose(bw["dx"][:, 0], expect, rtol=1e-14, atol=1e-15)


def test_layernorm_width_one():
    """N = 1: x - mean = 0, so y = beta exactly and dx = 0."""
    x = _randn((7, 1), 91, torch.float32)
    g, b = torch.tensor([1.3]), torch.tensor([-0.4])
    fw = oracle.layernorm_fwd(x, g, b, 1e-5)
    assert np.all(fw["y"] == np.float64(np.float32(-0.4)))
    bw = oracle.layernorm_bwd(x, _randn((7, 1), 92, torch.float32), g, 1e-5)
    assert np.all(bw["dx"] == 0.0) and np.all(bw["dgamma"] == 0.0)


def test_layernorm_rows_have_mean_zero_and_variance_v_over_v_plus_eps():
    x = _randn((33, 24), 93, torch.float32, scale=2.0, shift=3.0)
    ones, zeros = torch.ones(24), torch.zeros(24)
    eps = 1e-5
    y = oracle.layernorm_fwd(x, ones, zeros, eps)["y"]
    xd = x.double().numpy()
    v = xd.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose(y.var(axis=1), v / (v + eps), rtol=1e-12)


def test_layernorm_dx_rows_sum_to_zero():
    x, dy = _randn((20, 24), 94, torch.float32, scale=2.0), _randn((20, 24), 95, torch.float32)
    g = _randn(24, 96, torch.float32, shift=1.0)
    bw = oracle.layernorm_bwd(x, dy, g, 1e-5)
    np.testing.assert_allclose(bw["dx"].sum(axis=1), 0.0, atol=1e-12 * np.abs(bw["dx"]).sum(axis=1).max())


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_rmsnorm_scale_invariance(k):
    """eps = 0, c = 2^k: y(c x) == y(x) and dx(c x) == dx(x) / c, bitwise (power-of-two
    scaling is exact and sqrt is correctly rounded)."""
    x = _randn((6, 40), 97, torch.float32).to(torch.bfloat16)
    w = _randn(40, 98, torch.float32, shift=1.0).to(torch.bfloat16)
    dy = _randn((6, 40), 99, torch.float32).to(torch.bfloat16)
    c = 2.0 ** k
    xc = (x.float() * c).to(torch.bfloat16)
    a, b = oracle.rmsnorm_fwd(x, w, 0.0), oracle.rmsnorm_fwd(xc, w, 0.0)
    np.testing.assert_array_equal(a["y"], b["y"])
    ga, gb = oracle.rmsnorm_bwd(x, dy, w, 0.0), oracle.rmsnorm_bwd(xc, dy, w, 0.0)
    np.testing.assert_array_equal(ga["dx"], gb["dx"] * c)
    np.testing.assert_array_equal(ga["dweight"], gb["dweight"])


@pytest.mark.parametrize("layer", ["dyt", "layernorm"])
def test_dbeta_is_correctly_rounded_column_sum_over_many_row_blocks(layer):
    """M spans several of the oracle's row blocks: dbeta_j must equal the correctly rounded
    column sum of dy (math.fsum) to double precision."""
    M, N = 3001, 5
    x = _randn((M, N), 101, torch.float32)
    dy = _randn((M, N), 102, torch.float32)
    g = _randn(N, 103, torch.float32, shift=1.0)
    if layer == "dyt":
        bw = oracle.dyt_bwd(x, dy, 0.5, g, want_dx=False)
    else:
        bw = oracle.layernorm_bwd(x, dy, g, 1e-5, want_dx=False)
    d = dy.double().numpy()
    exp = [math.fsum(d[:, j].tolist()) for j in range(N)]
    np.testing.assert_allclose(bw["dbeta"], exp, rtol=1e-14)
    np.testing.assert_allclose(bw["dbeta_scale"], np.abs(d).sum(0), rtol=1e-13)


def test_column_sums_do_not_depend_on_thread_count():
    x = _randn((5000, 7), 111, torch.float32)
    dy = _randn((5000, 7), 112, torch.float32)
    g = _randn(7, 113, torch.float32)
    saved = oracle.max_threads()
    try:
        oracle.set_threads(1)
        a = oracle.layernorm_bwd(x, dy, g, 1e-5, want_dx=False)
        oracle.set_threads(4)
        b = oracle.layernorm_bwd(x, dy, g, 1e-5, want_dx=False)
    finally:
        oracle.set_threads(saved)
    assert np.array_equal(a["dgamma"], b["dgamma"]) and np.array_equal(a["dbeta"], b["dbeta"])
