"""GPU parity of the flat LayerNorm (and DyT) kernels with 12-byte lane chunks (plans with flat = 2): rows
of 12 * 2^k bytes (float32 N = 3 * 2^k, 16-bit N = 6 * 2^k, 2^k <= 64 lanes per row) on 4-byte
aligned operands.  Every group size and dtype pair, ragged row counts, row counts that give every
workgroup several tiles, operands 4 bytes (not 16) past an aligned address, a forward without
statistics outputs, and the backward's gradient subsets, against the oracle under the bars of
tests/tolerance.py, with every output and the workspace NaN-poisoned before the call."""
import pytest
import torch

import row_wise_normalization_dyt_amd as rwn
import workloads
from tests import gpu_cases as gc
from tests import tolerance as tol

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = (("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16"))


def _banner(*a):
    print("case:", *a, flush=True)


def _widths(xdt):
    esz = 4 if xdt == "f32" else 2
    return [12 * lanes // esz for lanes in (1, 2, 4, 8, 16, 32, 64)]


def _plan(M, N, xdt, pdt, backward=False, mis=0):
    return rwn.plan("layernorm", backward, M, N, gc.DT[xdt], misalign_bytes=mis,
                    param_dtype=None if backward else gc.DT[pdt])


@pytest.mark.parametrize("xdt,pdt", PAIRS)
def test_every_group_size_and_ragged_rows(xdt, pdt):
    """Group sizes 1..64 lanes at 1, 63 and 1031 rows (a wave's tile is 64 / group-size rows,
    twice that in the forward), with the forward's statistics passed to the backward and
    recomputed by it."""
    reps = []
    for N in _widths(xdt):
        for M in (1, 63, 1031):
            wl = workloads.small("layernorm", M, N, xdt, pdt, seed=N + 7 * M)
            assert _plan(M, N, xdt, pdt)["flat"] == 2 and _plan(M, N, xdt, pdt, True)["flat"] == 2, wl.name
            _banner(wl)
            reps += gc.check_workload(wl, DEV)
            reps += gc.check_workload(wl, DEV, use_stats=False)
    tol.assert_reports(reps)


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_several_tiles_per_workgroup(xdt):
    """Row counts at which every workgroup of the persistent grid runs at least two tiles of
    the forward and of the backward (1, 8 and 64 lanes per row); whole tensors compared."""
    reps = []
    esz = 4 if xdt == "f32" else 2
    for lanes in (1, 8, 64):
        N = 12 * lanes // esz
        rows_per_tile = 4 * (64 // lanes) * (1 if lanes == 1 else 2)   # full workgroups, forward
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        M = 2 * 8 * cus * rows_per_tile + 37   # the persistent grid holds at most 8 workgroups per CU
        p, pb = _plan(M, N, xdt, "f32"), _plan(M, N, xdt, "f32", True)
        assert p["flat"] == 2 and pb["flat"] == 2, (p, pb)
        assert p["ntiles"] >= 2 * p["grid"] and pb["ntiles"] >= 2 * pb["grid"], (p, pb)
        wl = workloads.small("layernorm", M, N, xdt, "f32", seed=lanes)
        _banner(wl, "tiles per workgroup", p["ntiles"] / p["grid"], pb["ntiles"] / pb["grid"])
        reps += gc.check_workload(wl, DEV)
    tol.assert_reports(reps)


@pytest.mark.parametrize("xdt,pdt", PAIRS)
def test_dyt_every_group_size_and_ragged_rows(xdt, pdt):
    """DyT rows of 12 * 2^k bytes take the 12-byte kernels too (backwards always, forwards where
    the rows are not whole 16-byte chunks): group sizes 1..64 lanes at 1, 63
    and 1031 rows, then row counts that give every workgroup of both grids several tiles, and
    alpha = +inf, 0 and negative values (the general kernels' edge handling), against the
    oracle."""
    reps = []
    for N in _widths(xdt):
        for M in (1, 63, 1031):
            wl = workloads.small("dyt", M, N, xdt, pdt, seed=N + 11 * M)
            p, pb = rwn.plan("dyt", False, M, N, gc.DT[xdt], param_dtype=gc.DT[pdt]), rwn.plan("dyt", True, M, N, gc.DT[xdt])
            esz = 4 if xdt == "f32" else 2
            assert pb["flat"] == 2 and p["flat"] == (2 if (N * esz) % 16 else 0), (wl.name, p, pb)
            _banner(wl)
            reps += gc.check_workload(wl, DEV)
    esz = 4 if xdt == "f32" else 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for lanes, alpha in ((2, 0.5), (8, float("inf")), (16, 0.0), (64, -1.5)):
        N = 12 * lanes // esz
        M = 2 * 8 * cus * 4 * (64 // lanes) * 2 + 29
        wl = workloads.small("dyt", M, N, xdt, pdt, seed=lanes, alpha=alpha)
        pb = rwn.plan("dyt", True, M, N, gc.DT[xdt])
        assert pb["flat"] == 2 and pb["ntiles"] >= 2 * pb["grid"], pb
        _banner(wl, "alpha", alpha, "tiles per workgroup", pb["ntiles"] / pb["grid"])
        reps += gc.check_workload(wl, DEV)
    tol.assert_reports(reps)


def _abi_layernorm(x, dy, gamma, beta, eps, use_stats=True):
    """Forward then backward through the C ABI on the given [M, N] views as they are (the
    binding would copy a misaligned view whose rows are whole 16-byte chunks), into NaN-poisoned
    outputs at x's address modulo 16 and a poisoned workspace."""
    lib = rwn._lib.load()
    M, N = x.shape
    nan = float("nan")
    stream = torch.cuda.current_stream().cuda_stream
    y, dx = rwn._like(x).fill_(nan), rwn._like(x).fill_(nan)
    assert y.data_ptr() % 16 == x.data_ptr() % 16 == dx.data_ptr() % 16 == dy.data_ptr() % 16
    mean = torch.full((M,), nan, device=x.device)
    rstd = torch.full((M,), nan, device=x.device)
    dg = torch.full((N,), nan, dtype=gamma.dtype, device=x.device)
    db = torch.full((N,), nan, dtype=gamma.dtype, device=x.device)
    ws = gc._poisoned_ws("layernorm", x)
    xt, pt = rwn._DT[x.dtype], rwn._DT[gamma.dtype]
    rwn._lib.check(lib, "layernorm_fwd", lib.layernorm_fwd(M, N, x.data_ptr(), xt, gamma.data_ptr(), beta.data_ptr(), pt,
                                                         eps, y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), stream))
    st = (mean.data_ptr(), rstd.data_ptr()) if use_stats else (None, None)
    rwn._lib.check(lib, "layernorm_bwd", lib.layernorm_bwd(M, N, x.data_ptr(), dy.data_ptr(), xt, *st, gamma.data_ptr(),
                                                         pt, eps, dx.data_ptr(), dg.data_ptr(), db.data_ptr(),
                                                         ws.data_ptr(), ws.numel(), stream))
    torch.cuda.synchronize()
    return {"y": y, "mean": mean, "rstd": rstd, "dx": dx, "dgamma": dg, "dbeta": db}


@pytest.mark.parametrize("xdt,offset_bytes", [("f32", 4), ("f32", 12), ("bf16", 4), ("bf16", 8), ("f16", 12)])
def test_four_byte_aligned_operands(xdt, offset_bytes):
    """Every [M, N] operand starts offset_bytes past a 16-byte boundary (called through the C
    ABI): the 12-byte kernels take them, with the backward given the statistics and
    recomputing them."""
    esz = 4 if xdt == "f32" else 2
    off = offset_bytes // esz
    reps = []
    for lanes, M in ((2, 999), (8, 1031), (32, 77), (64, 300)):
        N = 12 * lanes // esz
        wl = workloads.small("layernorm", M, N, xdt, "f32", seed=M + offset_bytes)
        assert _plan(M, N, xdt, "f32", mis=offset_bytes)["flat"] == 2
        assert _plan(M, N, xdt, "f32", True, mis=offset_bytes)["flat"] == 2
        _banner(wl, "offset bytes", offset_bytes)
        inp = workloads.make_inputs(wl)
        dev = {}
        for k, v in inp.items():
            if k in ("x", "dy"):
                buf = torch.empty(v.numel() + 16, dtype=v.dtype, device=DEV)
                view = buf[off:off + v.numel()].view(v.shape)
                view.copy_(v.to(DEV))
                assert view.data_ptr() % 16 == offset_bytes
                dev[k] = view
            else:
                dev[k] = v.to(DEV)
        o = gc.oracle_run("layernorm", inp, wl.eps)
        for use_stats in (True, False):
            g = _abi_layernorm(dev["x"], dev["dy"], dev["gamma"], dev["beta"], wl.eps, use_stats)
            reps += gc.compare("layernorm", g, o, gc.DT[xdt], torch.float32)
    tol.assert_reports(reps)


def test_forward_without_statistics_outputs():
    """mean and rstd NULL (the forward's statistics stores skipped): y is bitwise the y of the
    call that writes them."""
    for (M, N, xdt) in ((1031, 24, "f32"), (515, 48, "bf16"), (70, 3, "f32")):
        wl = workloads.small("layernorm", M, N, xdt, "f32", seed=M)
        _banner(wl, "no statistics")
        inp = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, DEV).items()}
        y_ref, _, _ = rwn.layernorm_fwd(inp["x"], inp["gamma"], inp["beta"], wl.eps)
        lib = rwn._lib.load()
        x = inp["x"]
        y = torch.full_like(x, float("nan"))
        st = lib.layernorm_fwd(M, N, x.data_ptr(), rwn._DT[x.dtype], inp["gamma"].data_ptr(), inp["beta"].data_ptr(),
                               rwn._DT[torch.float32], wl.eps, y.data_ptr(), None, None,
                               torch.cuda.current_stream().cuda_stream)
        rwn._lib.check(lib, "layernorm_fwd", st)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), y_ref.view(torch.uint8)), wl.name


@pytest.mark.parametrize("which", ["dgamma", "dbeta", "none"])
def test_gradient_subsets(which):
    """One gradient or none: dx and the requested gradient bitwise those of the full backward."""
    for (M, N, xdt, pdt) in ((4099, 24, "f32", "f32"), (1031, 48, "bf16", "f32"), (257, 384, "f16", "f16"),
                             (999, 6, "bf16", "bf16")):
        wl = workloads.small("layernorm", M, N, xdt, pdt, seed=M + N)
        assert _plan(M, N, xdt, pdt, True)["flat"] == 2
        _banner(wl, which)
        inp = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, DEV).items()}
        x, dy, g = inp["x"], inp["dy"], inp["gamma"]
        _, mean, rstd = rwn.layernorm_fwd(x, g, inp["beta"], wl.eps)
        full = rwn.layernorm_bwd(x, dy, mean, rstd, g, wl.eps, workspace=gc._poisoned_ws("layernorm", x))
        if which == "none":
            one = rwn.layernorm_bwd(x, dy, mean, rstd, g, wl.eps, need_param_grads=False)
        else:
            one = rwn.layernorm_bwd(x, dy, mean, rstd, g, wl.eps, need_dgamma=which == "dgamma",
                                    need_dbeta=which == "dbeta", workspace=gc._poisoned_ws("layernorm", x))
        torch.cuda.synchronize()
        assert torch.equal(one[0].view(torch.uint8), full[0].view(torch.uint8)), wl.name
        for k, name in ((1, "dgamma"), (2, "dbeta")):
            if which == name:
                assert torch.equal(one[k].view(torch.uint8), full[k].view(torch.uint8)), (wl.name, name)
            else:
                assert one[k] is None, (wl.name, name)


@pytest.mark.parametrize("xdt,offset_bytes", [("f32", 4), ("bf16", 12)])
def test_binding_keeps_four_byte_aligned_views(xdt, offset_bytes):
    """Through the Python binding: x and dy views offset_bytes past a 16-byte boundary are
    passed as they are (no aligned copy), y and dx come back at the same offset, and every
    result matches the oracle."""
    esz = 4 if xdt == "f32" else 2
    off = offset_bytes // esz
    reps = []
    for lanes, M in ((8, 1031), (64, 77)):
        N = 12 * lanes // esz
        wl = workloads.small("layernorm", M, N, xdt, "f32", seed=M + N)
        _banner(wl, "binding, offset bytes", offset_bytes)
        inp = workloads.make_inputs(wl)
        dev = {}
        for k, v in inp.items():
            if k in ("x", "dy"):
                buf = torch.empty(v.numel() + 16, dtype=v.dtype, device=DEV)
                view = buf[off:off + v.numel()].view(v.shape)
                view.copy_(v.to(DEV))
                assert view.data_ptr() % 16 == offset_bytes
                dev[k] = view
            else:
                dev[k] = v.to(DEV)
        g = gc.gpu_run("layernorm", dev, wl.eps, poison=False)
        assert g["y"].data_ptr() % 16 == offset_bytes and g["dx"].data_ptr() % 16 == offset_bytes
        o = gc.oracle_run("layernorm", inp, wl.eps)
        reps += gc.compare("layernorm", g, o, gc.DT[xdt], torch.float32)
    tol.assert_reports(reps)
