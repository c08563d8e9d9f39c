"""GPU parity of the strided entry points: row operands and parameters that are views (a slice of
a wider matrix, a head-major [B, S, H, D] tensor, a gradient in another layout than x, a strided
weight) run through the *_strided kernels without copies and match the oracle on the same
logical rows to the parity bars of tests/tolerance.py.

Needs an MI355X.  Every case records that the binding took the strided entry point (no copy
fallback) and writes through outputs whose untouched neighbours are NaN-poisoned.
"""
import pytest
import torch

import row_wise_normalization_dyt_amd as rwn
import workloads
from tests import gpu_cases as gc
from tests import tolerance as tol

pytestmark = pytest.mark.gpu

DEV = "cuda"
PARAMS = {"dyt": ["alpha", "gamma", "beta"], "layernorm": ["gamma", "beta"], "rmsnorm": ["weight"]}


@pytest.fixture
def strided_calls(monkeypatch):
    """Names of the strided entry points the binding called, each of which must have run."""
    calls = []
    real = rwn._try_strided

    def spy(lib, fn, call):
        ran = real(lib, fn, call)
        calls.append((fn, ran))
        return ran

    monkeypatch.setattr(rwn, "_try_strided", spy)
    return calls


def _embed(t: torch.Tensor, make_view):
    """Copies t into a fresh NaN-filled buffer through make_view(buffer) (a view of t's shape),
    returning (view, buffer)."""
    buf, view = make_view(t)
    assert view.shape == t.shape and view.data_ptr() != 0
    view.copy_(t)
    return view, buf


def _run(layer, x, dy, params, eps, form, y_out=None, dx_out=None):
    """Forward then backward through the binding on (possibly strided) views."""
    if layer == "dyt":
        y = rwn.dyt_fwd(x, params["alpha"], params["gamma"], params["beta"], y=y_out)
        dx, da, dg, db = rwn.dyt_bwd(x, dy, params["alpha"], params["gamma"], dx=dx_out)
        return {"y": y, "dx": dx, "dalpha": da, "dgamma": dg, "dbeta": db}
    if layer == "layernorm":
        y, mean, rstd = rwn.layernorm_fwd(x, params["gamma"], params["beta"], eps, y=y_out)
        dx, dg, db = rwn.layernorm_bwd(x, dy, mean, rstd, params["gamma"], eps, dx=dx_out)
        return {"y": y, "dx": dx, "dgamma": dg, "dbeta": db, "mean": mean, "rstd": rstd}
    y, rstd = rwn.rmsnorm_fwd(x, params["weight"], eps, form=form, y=y_out)
    dx, dw = rwn.rmsnorm_bwd(x, dy, rstd, params["weight"], eps, form=form, dx=dx_out)
    return {"y": y, "dx": dx, "dweight": dw, "rstd": rstd}


def _check(layer, xdt, pdt, M, N, x_view, dy_view, params, logical, wl, calls, y_out=None, dx_out=None):
    """Runs the views and compares every output, on the logical [M, N] rows, with the oracle."""
    calls.clear()
    got = _run(layer, x_view, dy_view, params, wl.eps, wl.form, y_out=y_out, dx_out=dx_out)
    torch.cuda.synchronize()
    assert calls and all(ran for _, ran in calls), calls
    g = {k: (v.reshape(M, N) if k in ("y", "dx") else v) for k, v in got.items()}
    ora = gc.oracle_run(layer, logical, wl.eps, form=wl.form)
    tol.assert_reports(gc.compare(layer, g, ora, gc.DT[xdt], gc.DT[pdt]))
    return got


def _inputs(layer, M, N, xdt, pdt, seed, **kw):
    wl = workloads.small(layer, M, N, xdt, pdt, seed=seed, **kw)
    print("case:", wl, flush=True)
    return wl, workloads.make_inputs(wl)


def _dev_params(layer, inp):
    return {k: inp[k].to(DEV) for k in PARAMS[layer]}


@pytest.mark.parametrize("xdt,pdt", [("bf16", "f32"), ("f16", "f16")])
@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("which", ["x", "dy", "both"])
def test_head_major_rows(layer, xdt, pdt, which, strided_calls):
    """[B, S, H, D] = [2, 300, 32, 128] with x, the upstream gradient or both head-major (the
    transposed view of a contiguous [B, H, S, D] tensor, as attention produces)."""
    B, S, H, D = 2, 300, 32, 128
    M = B * S * H
    wl, inp = _inputs(layer, M, D, xdt, pdt, seed=H + S)

    def head_major(t):
        buf = torch.empty(B, H, S, D, dtype=t.dtype, device=DEV)
        return buf, buf.permute(0, 2, 1, 3)

    x4 = inp["x"].reshape(B, S, H, D).to(DEV)
    dy4 = inp["dy"].reshape(B, S, H, D).to(DEV)
    xv = _embed(x4, head_major)[0] if which in ("x", "both") else x4
    dyv = _embed(dy4, head_major)[0] if which in ("dy", "both") else dy4
    assert not (xv.is_contiguous() and dyv.is_contiguous())
    _check(layer, xdt, pdt, M, D, xv, dyv, _dev_params(layer, inp), inp, wl, strided_calls)


# (M, N, dtype, pad, offset): x and dy are [:, offset:offset + N] column slices of a
# [M, N + pad] buffer.  A pad and offset that are multiples of the chunk keep every row on the
# same 16-byte phase (chunked kernels, aligned or shifted); others give rows of mixed alignment
# (element-wise kernels).
SLICES = [(300, 4096, "f32", 4, 0), (515, 1025, "bf16", 7, 0), (1001, 24, "f32", 1, 0),
          (257, 1000, "bf16", 8, 3), (129, 130, "f16", 16, 8), (77, 2048, "bf16", 5, 1),
          (33, 8192, "bf16", 8, 0), (65, 3001, "f32", 3, 2)]


@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("M,N,xdt,pad,off", SLICES)
def test_column_slices_and_poisoned_strided_outputs(layer, M, N, xdt, pad, off, strided_calls):
    """Column slices of wider matrices as x and dy, with y and dx written into column slices of
    NaN-filled buffers: every row element is written, nothing outside the slices is."""
    pdt = "f32"
    wl, inp = _inputs(layer, M, N, xdt, pdt, seed=M + pad)

    def sliced(t):
        buf = torch.full((t.shape[0], N + pad), float("nan"), dtype=t.dtype, device=DEV)
        return buf, buf[:, off:off + N]

    xv, _ = _embed(inp["x"].to(DEV), sliced)
    dyv, _ = _embed(inp["dy"].to(DEV), sliced)
    y_buf, y_out = sliced(inp["x"])
    dx_buf, dx_out = sliced(inp["x"])
    _check(layer, xdt, pdt, M, N, xv, dyv, _dev_params(layer, inp), inp, wl, strided_calls, y_out=y_out,
           dx_out=dx_out)
    for buf in (y_buf, dx_buf):
        outside = torch.ones_like(buf, dtype=torch.bool)
        outside[:, off:off + N] = False
        assert torch.isnan(buf[outside].float()).all()
        assert not torch.isnan(buf[:, off:off + N].float()).any()


@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("form", ["cast_then_weight", "one_plus_weight"])
def test_strided_parameters(layer, form, strided_calls):
    """Dense x with every parameter vector a stride-3 view: the parameters are read in place."""
    if layer != "rmsnorm" and form != "cast_then_weight":
        pytest.skip("forms are RMSNorm's")
    for (M, N, xdt, pdt) in [(1031, 128, "bf16", "bf16"), (257, 1025, "bf16", "f32"), (4099, 24, "f32", "f32")]:
        wl, inp = _inputs(layer, M, N, xdt, pdt, seed=N, **({"form": form} if layer == "rmsnorm" else {}))
        params = {}
        for k in PARAMS[layer]:
            v = inp[k].to(DEV)
            if v.numel() > 1:
                buf = torch.full((3 * v.numel(),), float("nan"), dtype=v.dtype, device=DEV)
                buf[::3].copy_(v)
                v = buf[::3]
                assert v.stride(0) == 3
            params[k] = v
        _check(layer, xdt, pdt, M, N, inp["x"].to(DEV), inp["dy"].to(DEV), params, inp, wl, strided_calls)


@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
def test_mixed_alignment_and_merged_dimensions(layer, strided_calls):
    """x a [5, 1, 7, 33, N] view with size-1 and mergeable dimensions; dy offset by one element
    from x's 16-byte phase (rows of mixed alignment: element-wise kernels)."""
    N, xdt, pdt = 200, "bf16", "f32"
    M = 5 * 7 * 33
    wl, inp = _inputs(layer, M, N, xdt, pdt, seed=11)
    xb = torch.empty(5, 33, 1, 7, N + 8, dtype=torch.bfloat16, device=DEV)
    xv = xb.permute(0, 2, 3, 1, 4)[..., :N]             # [5, 1, 7, 33, N], rows N + 8 apart
    xv.copy_(inp["x"].reshape(5, 1, 7, 33, N).to(DEV))
    dyb = torch.empty(M * N + 1, dtype=torch.bfloat16, device=DEV)
    dyv = dyb[1:].view(5, 1, 7, 33, N)                    # contiguous, 2 bytes past x's phase
    dyv.copy_(inp["dy"].reshape(5, 1, 7, 33, N).to(DEV))
    got = _check(layer, xdt, pdt, M, N, xv, dyv, _dev_params(layer, inp), inp, wl, strided_calls)
    assert got["y"].shape == xv.shape and got["dx"].shape == xv.shape


def test_strided_matches_dense_bitwise_where_plans_agree(strided_calls):
    """A column slice whose rows take the dense kernel's row shape (aligned, 64 lanes of one
    chunk per row) gives y, rstd and dx bitwise equal to the dense call on a contiguous copy:
    the strided path changes only how rows are addressed."""
    M, N = 4096, 512
    wl, inp = _inputs("rmsnorm", M, N, "bf16", "bf16", seed=2)
    x, dy, w = inp["x"].to(DEV), inp["dy"].to(DEV), inp["weight"].to(DEV)
    for bwd in (False, True):
        dp = rwn.plan("rmsnorm", bwd, M, N, torch.bfloat16, param_dtype=torch.bfloat16)
        sp = rwn.plan("rmsnorm", bwd, M, N, torch.bfloat16, param_dtype=torch.bfloat16, layout=1)
        assert dp["split"] == dp["flat"] == 0
        assert (dp["mode"], dp["tpr"], dp["cpt"]) == (sp["mode"], sp["tpr"], sp["cpt"]) == (0, 64, 1)
    xb = torch.zeros(M, N + 64, dtype=torch.bfloat16, device=DEV)
    dyb = torch.zeros(M, N + 64, dtype=torch.bfloat16, device=DEV)
    xv, dyv = xb[:, 64:], dyb[:, 64:]
    xv.copy_(x)
    dyv.copy_(dy)
    y_d, r_d = rwn.rmsnorm_fwd(x, w, wl.eps)
    dx_d, _ = rwn.rmsnorm_bwd(x, dy, r_d, w, wl.eps)
    strided_calls.clear()
    y_s, r_s = rwn.rmsnorm_fwd(xv, w, wl.eps)
    dx_s, _ = rwn.rmsnorm_bwd(xv, dyv, r_s, w, wl.eps)
    torch.cuda.synchronize()
    assert strided_calls == [("rmsnorm_fwd_strided", True), ("rmsnorm_bwd_strided", True)]
    assert torch.equal(y_s.view(torch.int16), y_d.view(torch.int16))
    assert torch.equal(r_s.view(torch.int32), r_d.view(torch.int32))
    assert torch.equal(dx_s.view(torch.int16), dx_d.view(torch.int16))


@pytest.mark.parametrize("alpha", [float("inf"), 0.0])
def test_strided_dyt_alpha_edges(alpha, strided_calls):
    """DyT with alpha = +inf (tanh saturates, sech^2 = 0 taken as alpha * sech^2 = 0) and alpha = 0
    on a column slice: the strided kernels keep the dense kernels' edge handling."""
    M, N = 1031, 200
    wl, inp = _inputs("dyt", M, N, "bf16", "f32", seed=21, alpha=alpha)

    def sliced(t):
        buf = torch.full((M, N + 24), float("nan"), dtype=t.dtype, device=DEV)
        return buf, buf[:, 16:16 + N]

    xv, _ = _embed(inp["x"].to(DEV), sliced)
    dyv, _ = _embed(inp["dy"].to(DEV), sliced)
    _check("dyt", "bf16", "f32", M, N, xv, dyv, _dev_params("dyt", inp), inp, wl, strided_calls)


@pytest.mark.parametrize("layer", ["layernorm", "rmsnorm"])
def test_strided_backward_recomputes_statistics(layer, strided_calls):
    """Head-major x with the statistics not passed to the backward (recomputed from x there)."""
    B, S, H, D = 2, 97, 8, 256
    M = B * S * H
    wl, inp = _inputs(layer, M, D, "bf16", "f32", seed=5)
    x = inp["x"].reshape(B, S, H, D).to(DEV)
    xv = torch.empty(B, H, S, D, dtype=x.dtype, device=DEV).permute(0, 2, 1, 3)
    xv.copy_(x)
    dy = inp["dy"].reshape(B, S, H, D).to(DEV)
    strided_calls.clear()
    if layer == "layernorm":
        y, _, _ = rwn.layernorm_fwd(xv, inp["gamma"].to(DEV), inp["beta"].to(DEV), wl.eps, want_stats=False)
        dx, dg, db = rwn.layernorm_bwd(xv, dy, None, None, inp["gamma"].to(DEV), wl.eps)
        got = {"y": y, "dx": dx, "dgamma": dg, "dbeta": db}
    else:
        y, _ = rwn.rmsnorm_fwd(xv, inp["weight"].to(DEV), wl.eps, want_stats=False)
        dx, dw = rwn.rmsnorm_bwd(xv, dy, None, inp["weight"].to(DEV), wl.eps)
        got = {"y": y, "dx": dx, "dweight": dw}
    torch.cuda.synchronize()
    assert [fn for fn, ran in strided_calls if ran] == [f"{layer}_fwd_strided", f"{layer}_bwd_strided"]
    got = {k: (v.reshape(M, D) if k in ("y", "dx") else v) for k, v in got.items()}
    tol.assert_reports(gc.compare(layer, got, gc.oracle_run(layer, inp, wl.eps), gc.DT["bf16"], gc.DT["f32"]))


def test_strided_layernorm_single_gradient(strided_calls):
    """dgamma alone on a head-major x: the strided backward forms both gradients' partials and stage 2
    reads only dgamma's columns, which are bitwise the full strided backward's; dx too."""
    B, S, H, D = 2, 300, 32, 128
    wl, inp = _inputs("layernorm", B * S * H, D, "bf16", "f32", seed=8)
    xv = torch.empty(B, H, S, D, dtype=torch.bfloat16, device=DEV).permute(0, 2, 1, 3)
    xv.copy_(inp["x"].reshape(B, S, H, D).to(DEV))
    dy = inp["dy"].reshape(B, S, H, D).to(DEV)
    g = inp["gamma"].to(DEV)
    _, mean, rstd = rwn.layernorm_fwd(xv, g, inp["beta"].to(DEV), wl.eps)
    full = rwn.layernorm_bwd(xv, dy, mean, rstd, g, wl.eps)
    one = rwn.layernorm_bwd(xv, dy, mean, rstd, g, wl.eps, need_dgamma=True, need_dbeta=False)
    torch.cuda.synchronize()
    assert one[2] is None
    assert torch.equal(one[0].view(torch.int16), full[0].view(torch.int16))
    assert torch.equal(one[1].view(torch.int32), full[1].view(torch.int32))
