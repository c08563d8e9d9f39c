"""GPU parity: the HIP path against the CPU oracle, element by element (needs an MI355X).

Bars (tests/tolerance.py): float32 y/dx within 1e-5 of the magnitude sum of their terms;
bfloat16/float16 y/dx within one ulp of the dtype plus that; parameter gradients within 1e-4 of the column's
sum of |terms| plus one ulp of the parameter dtype; NaN/Inf only where the oracle has them.
Parameter gradients must also be bitwise identical from run to run.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import row_wise_normalization_dyt_amd as rwn
from row_wise_normalization_dyt_amd import autograd as ag
import workloads
from tests import gpu_cases as gc
from tests import tolerance as tol

pytestmark = pytest.mark.gpu

DEV = "cuda"
LAYERS = ("dyt", "layernorm", "rmsnorm")
DTYPE_PAIRS = (("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16"))


def _banner(*a):
    print("case:", *a, flush=True)


def _run_small(layer, M, N, xdt, pdt, seed=3, use_stats=True, **kw):
    wl = workloads.small(layer, M, N, xdt, pdt, seed=seed, **kw)
    _banner(wl)
    return gc.check_workload(wl, DEV, use_stats=use_stats)


# ------------------------------------------------------------------ small shapes, all layers

@pytest.mark.parametrize("xdt,pdt", DTYPE_PAIRS)
@pytest.mark.parametrize("layer", LAYERS)
def test_small_shapes_span_tiles_and_ragged_tails(layer, xdt, pdt):
    reps = []
    for (M, N) in [(4099, 24), (1031, 64), (777, 128), (515, 256), (263, 1024), (130, 2048), (67, 4096)]:
        reps += _run_small(layer, M, N, xdt, pdt)
    tol.assert_reports(reps)


EDGE_N = [1, 2, 3, 4, 7, 8, 15, 16, 17, 24, 31, 32, 33, 63, 64, 65, 127, 128, 129, 130, 255, 256, 257,
          512, 1023, 1024, 1025, 2048, 2049]


@pytest.mark.parametrize("xdt,pdt", DTYPE_PAIRS)
@pytest.mark.parametrize("layer", LAYERS)
def test_edge_widths(layer, xdt, pdt):
    """Widths around every chunk, wave and mode boundary, at row counts of 1, 7 and 257."""
    reps = []
    for N in EDGE_N:
        for M in (1, 7, 257):
            reps += _run_small(layer, M, N, xdt, pdt, seed=N * 7 + M)
    tol.assert_reports(reps)


@pytest.mark.parametrize("xdt,pdt", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16")])
@pytest.mark.parametrize("form", ["weight_then_cast", "one_plus_weight"])
def test_rmsnorm_float32_forms(form, xdt, pdt):
    """The weight-before-cast and (1 + weight) RMSNorm forms over aligned, shifted and narrow
    shapes, with the weight's mean at 0 so that (1 + weight) differs from weight."""
    reps = []
    for (M, N) in [(4099, 24), (777, 128), (263, 1024), (67, 4096), (257, 1025), (65, 17), (7, 2049)]:
        wl = workloads.small("rmsnorm", M, N, xdt, pdt, seed=M + N, form=form, gamma_mean=0.0, gamma_std=0.5)
        _banner(wl)
        reps += gc.check_workload(wl, DEV)
    tol.assert_reports(reps)


@pytest.mark.parametrize("layer", LAYERS)
def test_edge_row_counts(layer):
    reps = []
    for M in (2, 3, 65535, 65536, 65537):
        for N in (24, 129):
            reps += _run_small(layer, M, N, "bf16", "f32", seed=M % 1000)
    tol.assert_reports(reps)


@pytest.mark.parametrize("layer", LAYERS)
def test_backward_without_saved_stats(layer):
    if layer == "dyt":
        pytest.skip("DyT has no statistics")
    reps = []
    for (M, N) in [(1001, 24), (257, 1025), (33, 4096)]:
        reps += _run_small(layer, M, N, "bf16", "f32", use_stats=False)
    tol.assert_reports(reps)


@pytest.mark.parametrize("layer", ["layernorm", "rmsnorm"])
def test_backward_recomputing_stats_with_zero_eps(layer):
    """eps = 0 with statistics recomputed in the backward: a padded row's recomputed rstd is
    infinite there, which must not reach the parameter gradients (ragged tiles at every M)."""
    reps = []
    for (M, N) in [(1001, 24), (77, 129), (257, 1025)]:
        reps += _run_small(layer, M, N, "f32", "f32", use_stats=False, eps=0.0)
    tol.assert_reports(reps)


def test_layernorm_without_affine():
    wl = workloads.small("layernorm", 999, 48, "f32", "f32", seed=5)
    inp = workloads.make_inputs(wl)
    del inp["gamma"], inp["beta"]
    _banner(wl, "no affine")
    tol.assert_reports(gc.check_workload(wl, DEV, inputs=inp))


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("offset", [1, 3])
def test_misaligned_operands_take_the_shifted_path(layer, offset, xdt):
    """x and dy are views starting `offset` 16-bit elements past a 16-byte boundary."""
    reps = []
    for (M, N) in [(513, 1025), (100, 999), (37, 129), (65, 24)]:
        wl = workloads.small(layer, M, N, xdt, "f32", seed=M + offset)
        _banner(wl, "offset", offset)
        inp = workloads.make_inputs(wl)
        dev = {}
        for k, v in inp.items():
            if k in ("x", "dy"):
                buf = torch.empty(v.numel() + 16, dtype=v.dtype, device=DEV)
                view = buf[offset:offset + v.numel()].view(v.shape)
                view.copy_(v.to(DEV))
                assert view.data_ptr() % 16 == 2 * offset
                dev[k] = view
            else:
                dev[k] = v.to(DEV)
        g = gc.gpu_run(layer, dev, wl.eps)
        o = gc.oracle_run(layer, inp, wl.eps)
        reps += gc.compare(layer, g, o, gc.DT[xdt], torch.float32)
    tol.assert_reports(reps)


@pytest.mark.parametrize("layer", LAYERS)
def test_narrow_rows_in_shifted_chunks(layer):
    """Narrow rows that are not whole 16-byte chunks move in 16-byte chunks: a power-of-two lane
    group per row, several row slots per workgroup (up to 128 at N = 3), each slot keeping its
    rows' shift while its workgroup walks its tiles.  Row counts give every workgroup of the
    backward's persistent grid at least two tiles; whole tensors compared, parameter gradients
    combined over all slots."""
    reps = []
    for (N, xdt, pdt) in ((100, "bf16", "f32"), (500, "bf16", "bf16"), (17, "f16", "f16"), (3, "bf16", "f32"),
                          (250, "f32", "f32"), (7, "f32", "f32")):
        pb = rwn.plan(layer, True, 1 << 22, N, gc.DT[xdt])
        assert pb["mode"] == 1 and pb["tpr"] <= 64 and not pb["split"], pb
        M = 2 * pb["grid"] * pb["rpp"] + 37
        for _ in range(4):   # the grid follows M (and the kernels' residency): grow M until it holds
            pb = rwn.plan(layer, True, M, N, gc.DT[xdt])
            if pb["ntiles"] >= 2 * pb["grid"]:
                break
            M = 2 * M + 37
        assert pb["ntiles"] >= 2 * pb["grid"], (M, pb)
        wl = workloads.small(layer, M, N, xdt, pdt, seed=M + N)
        _banner(wl, "narrow shifted, tiles per workgroup", pb["ntiles"] / pb["grid"], "slots", pb["rpp"])
        reps += gc.check_workload(wl, DEV)
    tol.assert_reports(reps)


@pytest.mark.parametrize("layer", LAYERS)
def test_float16_outputs_overflow_to_infinity(layer):
    """float16 tops out at 65504: outputs whose exact value rounds beyond it are +-inf, and
    every other element stays within the usual bound (the oracle's exact values rounded to
    float16 decide which elements overflow)."""
    M, N = 257, 136
    wl = workloads.small(layer, M, N, "f16", "f32", seed=5)
    _banner(wl, "overflow")
    inp = workloads.make_inputs(wl)
    big = torch.linspace(30000.0, 70000.0, N)
    if layer == "rmsnorm":
        inp["weight"] = big.to(torch.float32)
    else:
        inp["gamma"] = big.to(torch.float32)
        inp["beta"] = (big / 2).to(torch.float32)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    g = gc.gpu_run(layer, dev, wl.eps)
    torch.cuda.synchronize()
    o = gc.oracle_run(layer, inp, wl.eps, grads=False)
    ry = oracle.round_f16(o["y"])
    gy = g["y"].double().cpu().numpy()
    # Within float32 rounding of the threshold 65520 either side is a correct result.
    edge = np.abs(np.abs(o["y"]) - 65520.0) <= 1e-4 * 65520.0
    over = np.isinf(ry) & ~edge
    fin = ~np.isinf(ry) & ~edge
    assert over.any() and fin.any()
    assert np.array_equal(gy[over], ry[over])
    mask = torch.as_tensor(fin, device=g["y"].device)
    r = tol.compare(f"{layer}.y", g["y"][mask], o["y"][fin], o["y_scale"][fin],
                    torch.float16, alt=None if o.get("y_alt") is None else o["y_alt"][fin])
    tol.assert_reports([r])


def test_non_contiguous_and_batched_inputs():
    """Any leading shape; a transposed (non-contiguous) input is copied by the binding."""
    wl = workloads.small("rmsnorm", 2 * 300 * 32, 128, "bf16", "bf16", seed=11)
    inp = workloads.make_inputs(wl)
    x4 = inp["x"].reshape(2, 300, 32, 128).to(DEV)
    y4, _ = rwn.rmsnorm_fwd(x4, inp["weight"].to(DEV), wl.eps)
    assert y4.shape == x4.shape
    xt = inp["x"].reshape(600, 32, 128).transpose(0, 1).to(DEV)       # non-contiguous
    yt, _ = rwn.rmsnorm_fwd(xt, inp["weight"].to(DEV), wl.eps)
    ref, _ = rwn.rmsnorm_fwd(xt.contiguous(), inp["weight"].to(DEV), wl.eps)
    assert torch.equal(yt, ref)
    o = gc.oracle_run("rmsnorm", inp, wl.eps, grads=False)
    tol.assert_reports([tol.compare("rmsnorm.y", y4.reshape(-1, 128), o["y"], o["y_scale"], torch.bfloat16,
                                    alt=o["y_alt"])])


@pytest.mark.parametrize("layer", LAYERS)
def test_empty_input(layer):
    wl = workloads.small(layer, 0, 64, "bf16", "f32")
    inp = {k: v.to(DEV) for k, v in workloads.make_inputs(wl).items()}
    g = gc.gpu_run(layer, inp, wl.eps)
    torch.cuda.synchronize()
    assert g["y"].numel() == 0 and g["dx"].numel() == 0
    for k in ("dgamma", "dbeta", "dalpha", "dweight"):
        if g.get(k) is not None:
            assert torch.count_nonzero(g[k]).item() == 0, k


# ------------------------------------------------------------------------ determinism

@pytest.mark.parametrize("layer", LAYERS)
def test_backward_is_bitwise_reproducible(layer):
    """Two runs on the same inputs, each into fresh NaN-poisoned outputs and workspace, give the
    same bits everywhere (parameter gradients included)."""
    for (M, N, xdt) in [(401408, 24, "f32"), (8192, 128, "bf16"), (4099, 2048, "bf16"), (2049, 1025, "bf16")]:
        wl = workloads.small(layer, M, N, xdt, "f32", seed=1)
        _banner(wl, "determinism")
        inp = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, DEV).items()}
        a = gc.gpu_run(layer, inp, wl.eps, poison=True)
        b = gc.gpu_run(layer, inp, wl.eps, poison=True)
        for k in a:
            if a[k] is not None:
                assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                                   b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k]), (wl.name, k)


# ------------------------------------------------------------------------ DyT alpha edges

@pytest.mark.parametrize("alpha", [math.inf, 0.0])
@pytest.mark.parametrize("N", [32, 128, 256])
def test_dyt_alpha_edges_full_rows(alpha, N):
    """alpha = +inf and 0 at M = 1,048,573 (prime, above 65,535): finite gradients, matching
    the oracle.  Padded rows of the last tile must not poison the sums."""
    wl = workloads.WORKLOADS[f"dyt_bf16_1048573x{N}"].with_(alpha=alpha)
    _banner(wl.name, "alpha", alpha)
    inp = workloads.make_inputs(wl, DEV)
    if alpha == math.inf:
        assert torch.count_nonzero(inp["x"] == 0).item() == 0
    rows = gc.sample_rows(wl.M)
    reps = gc.check_workload(wl, DEV, rows=rows, inputs=inp)
    g = gc.gpu_run("dyt", inp, wl.eps)
    for k in ("dalpha", "dgamma", "dbeta"):
        assert torch.isfinite(g[k]).all(), k
    if alpha == math.inf:
        assert g["dalpha"].item() == 0.0
    tol.assert_reports(reps)


@pytest.mark.parametrize("alpha", [-0.5, -3.0, -0.0, -math.inf, 2.0 ** -40, -(2.0 ** 40), 1e-20, 1e20, 3e38])
def test_dyt_alpha_values(alpha):
    """Alphas on both sides of the DyT kernels' per-launch constants and backward fast path:
    negative (its sign applied to gamma and to the dgamma sums), -0, -inf, the fast path's
    bounds 2^-40 and 2^40, and magnitudes past them (formed element by element from alpha x).
    Narrow (general kernels, ALIGNED and SHIFTED chunks) and wide (split) shapes, every output against the
    oracle."""
    reps = []
    for (M, N, xdt, pdt) in ((4099, 24, "f32", "f32"), (1031, 32, "bf16", "f32"), (515, 17, "f16", "f32"),
                             (257, 1025, "bf16", "bf16"), (67, 4096, "f32", "f32")):
        wl = workloads.small("dyt", M, N, xdt, pdt, seed=M + N, alpha=alpha)
        _banner(wl, "alpha", alpha)
        reps += gc.check_workload(wl, DEV)
    tol.assert_reports(reps)


# ----------------------------------------------------------------- full-size workloads

FULL = [n for n in workloads.WORKLOADS]


@pytest.mark.parametrize("layer", LAYERS)
def test_dx_only_backward_matches_full_backward(layer):
    """With every gradient pointer NULL (and no workspace) the backward computes dx alone; that
    dx is bitwise the full backward's, at narrow, wide, shifted and scalar shapes and at the
    headline size."""
    shapes = [(4099, 24, "f32", "f32"), (1031, 128, "bf16", "f32"), (263, 1024, "bf16", "bf16"),
              (257, 1025, "bf16", "f32"), (65, 17, "f16", "f16"), (67, 4096, "f32", "f32")]
    if layer == "layernorm":
        shapes.append((401408, 24, "f32", "f32"))
    for (M, N, xdt, pdt) in shapes:
        wl = workloads.small(layer, M, N, xdt, pdt, seed=M + N)
        _banner(wl, "dx only")
        inp = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, DEV).items()}
        x, dy = inp["x"], inp["dy"]
        if layer == "dyt":
            full = rwn.dyt_bwd(x, dy, inp["alpha"], inp["gamma"])
            only = rwn.dyt_bwd(x, dy, inp["alpha"], inp["gamma"], need_param_grads=False)
        elif layer == "layernorm":
            _, mean, rstd = rwn.layernorm_fwd(x, inp["gamma"], inp["beta"], wl.eps)
            full = rwn.layernorm_bwd(x, dy, mean, rstd, inp["gamma"], wl.eps)
            only = rwn.layernorm_bwd(x, dy, mean, rstd, inp["gamma"], wl.eps, need_param_grads=False)
        else:
            _, rstd = rwn.rmsnorm_fwd(x, inp["weight"], wl.eps)
            full = rwn.rmsnorm_bwd(x, dy, rstd, inp["weight"], wl.eps)
            only = rwn.rmsnorm_bwd(x, dy, rstd, inp["weight"], wl.eps, need_param_grads=False)
        torch.cuda.synchronize()
        assert all(t is None for t in only[1:])
        assert torch.equal(only[0].view(torch.uint8), full[0].view(torch.uint8)), wl.name


LN_GRAD_SHAPES = [(4099, 24, "f32", "f32"), (1031, 128, "bf16", "f32"), (263, 1024, "bf16", "bf16"),
                  (257, 1025, "bf16", "f32"), (65, 17, "f16", "f16"), (67, 4096, "f32", "f32"),
                  (129, 3001, "f16", "f32"), (401408, 24, "f32", "f32"), (1031, 48, "bf16", "f32")]


@pytest.mark.parametrize("which", ["dgamma", "dbeta"])
def test_layernorm_single_gradient_matches_full_backward(which):
    """One LayerNorm parameter gradient alone (flat, general, split, scalar and wide shapes, and
    the 401408 x 24 float32 size): dx and that gradient are bitwise the full backward's, the
    other is not returned, and stage 1 writes half the partial slots of a NaN-poisoned
    workspace (only the requested gradient's columns)."""
    for (M, N, xdt, pdt) in LN_GRAD_SHAPES:
        wl = workloads.small("layernorm", M, N, xdt, pdt, seed=M + 3 * N)
        _banner(wl, which, "only")
        inp = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, DEV).items()}
        x, dy, g = inp["x"], inp["dy"], inp["gamma"]
        _, mean, rstd = rwn.layernorm_fwd(x, g, inp["beta"], wl.eps)
        ws_full, ws_one = gc._poisoned_ws("layernorm", x), gc._poisoned_ws("layernorm", x)
        full = rwn.layernorm_bwd(x, dy, mean, rstd, g, wl.eps, workspace=ws_full)
        one = rwn.layernorm_bwd(x, dy, mean, rstd, g, wl.eps, need_dgamma=which == "dgamma",
                                need_dbeta=which == "dbeta", workspace=ws_one)
        torch.cuda.synchronize()
        k = 1 if which == "dgamma" else 2
        assert one[3 - k] is None, wl.name
        assert torch.equal(one[0].view(torch.uint8), full[0].view(torch.uint8)), wl.name
        assert torch.equal(one[k].view(torch.uint8), full[k].view(torch.uint8)), wl.name
        n = ws_full.numel() // 4 * 4
        written_full = int(torch.isfinite(ws_full[:n].view(torch.float32)).sum())
        written_one = int(torch.isfinite(ws_one[:n].view(torch.float32)).sum())
        assert written_one * 2 == written_full, (wl.name, written_one, written_full)


@pytest.mark.parametrize("trainable", ["weight", "bias"])
def test_layernorm_autograd_one_trainable_parameter(trainable):
    """nn.LayerNorm-style use with one parameter frozen, and with gamma but no bias: the autograd
    function asks only for the trainable parameter's gradient; y, dx and that gradient match
    the oracle (a missing bias is zero, its gradient is not formed)."""
    for (M, N, xdt, pdt), no_bias in [((1001, 24, "f32", "f32"), False), ((257, 1025, "bf16", "f32"), False),
                                      ((999, 48, "f32", "f32"), True), ((131, 4096, "bf16", "bf16"), True)]:
        if no_bias and trainable == "bias":
            continue
        wl = workloads.small("layernorm", M, N, xdt, pdt, seed=M + N)
        _banner(wl, "trainable", trainable, "no bias" if no_bias else "")
        inp = workloads.make_inputs(wl)
        if no_bias:
            inp["beta"] = torch.zeros_like(inp["beta"])
        x = inp["x"].to(DEV).requires_grad_(True)
        w = inp["gamma"].to(DEV).requires_grad_(trainable == "weight")
        b = None if no_bias else inp["beta"].to(DEV).requires_grad_(trainable == "bias")
        y = ag.layer_norm(x, w, b, wl.eps)
        y.backward(inp["dy"].to(DEV))
        torch.cuda.synchronize()
        assert (w.grad is None) == (trainable != "weight")
        assert b is None or (b.grad is None) == (trainable != "bias")
        gpu = {"y": y.detach(), "dx": x.grad, "dgamma": w.grad, "dbeta": None if b is None else b.grad}
        ora = gc.oracle_run("layernorm", inp, wl.eps)
        tol.assert_reports(gc.compare("layernorm", gpu, ora, gc.DT[xdt], gc.DT[pdt]))


# Workloads compared on every element of y, dx and the statistics (the oracle streams row
# chunks); the others (the 134M- to 1G-element ones) are compared on whole launch tiles.
FULL_ROWS = {n for n, w in workloads.WORKLOADS.items() if w.M * w.N <= (40 << 20)}


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """Every workload at its real size, in the launch configuration the benchmark times, with
    NaN-poisoned outputs and workspace: y/dx/stats on every row (workloads up to 40M elements)
    or on whole tiles of 16 workgroups spread over the forward and backward grids (first, middle
    and last tile of each, and the grid's last tile); parameter gradients over all M rows."""
    wl = workloads.WORKLOADS[name]
    if name in FULL_ROWS:
        _banner(name, "all rows")
        reps = gc.check_full_rows(wl, DEV)
    else:
        rows = gc.tile_rows(wl)
        _banner(name, "whole tiles", len(rows), "rows")
        reps = gc.check_workload(wl, DEV, rows=rows, on_gpu_inputs=True)
    for r in reps:
        print("  ", r, flush=True)
    tol.assert_reports(reps)


@pytest.mark.parametrize("layer,M,N,xdt,pdt", [("dyt", 300000, 24, "bf16", "f32"), ("dyt", 300000, 128, "bf16", "f32"),
                                               ("rmsnorm", 40000, 2048, "bf16", "bf16"),
                                               ("layernorm", 300000, 24, "f32", "f32"),
                                               ("layernorm", 40000, 1025, "bf16", "f32")])
def test_multi_tile_workgroups_all_rows(layer, M, N, xdt, pdt):
    """Shapes where every workgroup of the persistent grids walks several tiles, so the
    pipelined tile loops rotate through all of their buffers; every element compared.  The
    grids follow the kernels' residency on the device, so M grows (up to 4x) until one of the
    two grids has at least four tiles per workgroup."""
    for _ in range(3):
        pf = rwn.plan(layer, False, M, N, gc.DT[xdt], param_dtype=gc.DT[pdt])
        pb = rwn.plan(layer, True, M, N, gc.DT[xdt])
        if pf["ntiles"] >= 4 * pf["grid"] // pf["ncb"] or pb["ntiles"] >= 4 * pb["grid"] // pb["ncb"]:
            break
        M = 2 * M + 37
    assert pf["ntiles"] >= 4 * pf["grid"] // pf["ncb"] or pb["ntiles"] >= 4 * pb["grid"] // pb["ncb"], (M, pf, pb)
    wl = workloads.small(layer, M, N, xdt, pdt, seed=M + N)
    _banner(wl, "multi-tile", pf["ntiles"] * pf["ncb"] / pf["grid"], pb["ntiles"] * pb["ncb"] / pb["grid"])
    reps = gc.check_full_rows(wl, DEV)
    tol.assert_reports(reps)


# ------------------------------------------------------------- tuning overrides keep parity

_OVERRIDE_SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import workloads
from tests import gpu_cases as gc
bad = []
for layer in ("dyt", "layernorm", "rmsnorm"):
    for (M, N, xdt, pdt) in [(4099, 24, "f32", "f32"), (1031, 128, "bf16", "f32"), (130, 2048, "bf16", "bf16"),
                             (67, 1025, "bf16", "f32"), (33, 4096, "f32", "f32"), (515, 1025, "f32", "f32"),
                             (129, 3001, "f16", "f16")]:
        wl = workloads.small(layer, M, N, xdt, pdt, seed=11)
        print("case:", wl.name, flush=True)
        bad += [str(r) for r in gc.check_workload(wl, "cuda") if not r.ok()]
print("BAD", bad, flush=True)
"""


@pytest.mark.parametrize("env", ["RWN_PREFETCH=0", "RWN_PREFETCH=1", "RWN_PREFETCH=2", "RWN_FWD_RT=4 RWN_BWD_RT=2",
                                 "RWN_WIDE_CPT=4", "RWN_BLOCKED_K=3", "RWN_XCD_REMAP=0 RWN_WG_PER_CU=2",
                                 "RWN_FLAT=0", "RWN_XCD_REMAP=1 RWN_BLOCKED_K=2", "RWN_SPLIT=0", "RWN_SPLIT=2",
                                 "RWN_SPLIT_CPT=1", "RWN_SPLIT_CPT=4", "RWN_FLAT12=0", "RWN_SPLIT_PF=0",
                                 "RWN_SPLIT_PF=1", "RWN_MIN_WAVES=32", "RWN_WIDE_BLOCK=1024", "RWN_PACKED_ROWS=0"])
def test_tuning_overrides_keep_parity(env):
    """The tuning knobs change the launch plan (pipelining depth, rows per thread, chunks per
    thread, tile assignment, grid); every plan they reach must still match the oracle.  The
    knobs are read once per process, so each setting runs in a child process."""
    import os, subprocess, sys
    _banner("overrides", env)
    child_env = dict(os.environ)
    child_env.update(kv.split("=") for kv in env.split())
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-u", "-c", _OVERRIDE_SCRIPT.format(root=root)], env=child_env,
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "BAD []" in r.stdout, r.stdout[-3000:]
