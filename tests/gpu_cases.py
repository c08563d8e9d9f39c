"""Runs one workload through the HIP path and through the oracle, and compares the two.

Shared by the GPU parity tests, the smoke check and the benchmark's parity spot check.  The
HIP side is the package's C-ABI binding; the oracle side is oracle/ (CPU, fp64).  The two share
nothing but the inputs, which come from workloads.make_inputs.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
import row_wise_normalization_dyt_amd as rwn
from tests import tolerance as tol
import workloads

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
GRAD_NAMES = {"dyt": ["dgamma", "dbeta", "dalpha"], "layernorm": ["dgamma", "dbeta"], "rmsnorm": ["dweight"]}


NAN = float("nan")


def _poisoned_rows(x: torch.Tensor) -> torch.Tensor:
    """A NaN-filled [M, N] output laid out like x (same address modulo 16 bytes)."""
    x2 = rwn._as_2d(x, "x")
    return rwn._like(x2).fill_(NAN)


def _poisoned_vec(n: int, dtype, dev) -> torch.Tensor:
    return torch.full((n,), NAN, dtype=dtype, device=dev)


def _poisoned_ws(layer: str, x: torch.Tensor) -> torch.Tensor:
    """A workspace whose every byte is 0xFF (each float32 partial slot reads as NaN until the
    kernel writes it)."""
    N = x.shape[-1]
    M = x.numel() // N
    n = rwn.workspace_size(layer, M, N, x.dtype, x.device)
    return torch.full((max(n, 16),), 255, dtype=torch.uint8, device=x.device)


def gpu_run(layer: str, inp: Dict[str, torch.Tensor], eps: float, use_stats: bool = True,
            form: str = "cast_then_weight", poison: bool = True, grads: bool = True) -> Dict[str, torch.Tensor]:
    """Forward then backward on the tensors' device (dy is the upstream gradient of y).

    With poison (the default) every output, statistic, gradient and the backward workspace is a
    fresh buffer filled with NaN before the call, so an element or partial the kernels fail to
    write shows up as NaN instead of inheriting a plausible stale value.  grads=False asks the
    backward for dx only (no parameter gradient, no workspace)."""
    x, dy = inp["x"], inp["dy"]
    N = x.shape[-1]
    M = x.numel() // N
    dev = x.device
    P = (lambda f: f()) if poison else (lambda f: None)
    Q = (lambda f: f()) if (poison and grads) else (lambda f: None)
    if layer == "dyt":
        pt = inp["gamma"].dtype
        y = rwn.dyt_fwd(x, inp["alpha"], inp["gamma"], inp["beta"], y=P(lambda: _poisoned_rows(x)))
        dx, da, dg, db = rwn.dyt_bwd(x, dy, inp["alpha"], inp["gamma"], grads, dx=P(lambda: _poisoned_rows(x)),
                                     dalpha=Q(lambda: _poisoned_vec(1, pt, dev)),
                                     dgamma=Q(lambda: _poisoned_vec(N, pt, dev)),
                                     dbeta=Q(lambda: _poisoned_vec(N, pt, dev)),
                                     workspace=Q(lambda: _poisoned_ws("dyt", x)))
        return {"y": y, "dx": dx, "dalpha": da, "dgamma": dg, "dbeta": db}
    if layer == "layernorm":
        g = inp.get("gamma")
        pt = g.dtype if g is not None else torch.float32
        y, mean, rstd = rwn.layernorm_fwd(x, g, inp.get("beta"), eps, y=P(lambda: _poisoned_rows(x)),
                                          mean=P(lambda: _poisoned_vec(M, torch.float32, dev)),
                                          rstd=P(lambda: _poisoned_vec(M, torch.float32, dev)))
        if not use_stats:
            mean = rstd = None
        dx, dg, db = rwn.layernorm_bwd(x, dy, mean, rstd, g, eps, need_param_grads=grads,
                                       dx=P(lambda: _poisoned_rows(x)),
                                       dgamma=Q(lambda: _poisoned_vec(N, pt, dev)),
                                       dbeta=Q(lambda: _poisoned_vec(N, pt, dev)),
                                       workspace=Q(lambda: _poisoned_ws("layernorm", x)))
        out = {"y": y, "dx": dx, "dgamma": dg, "dbeta": db}
        if use_stats:
            out.update(mean=mean, rstd=rstd)
        return out
    w = inp["weight"]
    y, rstd = rwn.rmsnorm_fwd(x, w, eps, form=form, y=P(lambda: _poisoned_rows(x)),
                              rstd=P(lambda: _poisoned_vec(M, torch.float32, dev)))
    dx, dw = rwn.rmsnorm_bwd(x, dy, rstd if use_stats else None, w, eps, need_param_grads=grads, form=form,
                             dx=P(lambda: _poisoned_rows(x)), dweight=Q(lambda: _poisoned_vec(N, w.dtype, dev)),
                             workspace=Q(lambda: _poisoned_ws("rmsnorm", x)))
    out = {"y": y, "dx": dx, "dweight": dw}
    if use_stats:
        out["rstd"] = rstd
    return out


def oracle_run(layer: str, inp: Dict[str, torch.Tensor], eps: float, rows: Optional[Sequence[int]] = None,
               grads: bool = True, form: str = "cast_then_weight") -> Dict[str, np.ndarray]:
    """Oracle on host copies.  rows: compute y/dx (and stats) only for these rows; the
    parameter gradients always use every row."""
    h = {k: v.detach().cpu() for k, v in inp.items()}
    x, dy = h["x"], h["dy"]
    xs, dys = (x, dy) if rows is None else (x[list(rows)], dy[list(rows)])
    e = workloads.eps_f32(eps)
    out: Dict[str, np.ndarray] = {}
    if layer == "dyt":
        out.update(oracle.dyt_fwd(xs, h["alpha"], h["gamma"], h["beta"]))
        b = oracle.dyt_bwd(xs, dys, h["alpha"], h["gamma"])
        out.update(dx=b["dx"], dx_scale=b["dx_scale"])
        if grads:
            out.update({k: v for k, v in (b if rows is None else oracle.dyt_bwd(x, dy, h["alpha"], h["gamma"], want_dx=False)).items()
                        if k.startswith(("dgamma", "dbeta", "dalpha"))})
    elif layer == "layernorm":
        f = oracle.layernorm_fwd(xs, h.get("gamma", torch.ones(x.shape[1])), h.get("beta", torch.zeros(x.shape[1])), e)
        out.update(f)
        g = h.get("gamma", torch.ones(x.shape[1]))
        b = oracle.layernorm_bwd(xs, dys, g, e)
        out.update(dx=b["dx"], dx_scale=b["dx_scale"])
        if grads:
            out.update({k: v for k, v in (b if rows is None else oracle.layernorm_bwd(x, dy, g, e, want_dx=False)).items()
                        if k.startswith(("dgamma", "dbeta"))})
    else:
        out.update(oracle.rmsnorm_fwd(xs, h["weight"], e, form=form))
        b = oracle.rmsnorm_bwd(xs, dys, h["weight"], e, form=form)
        out.update(dx=b["dx"], dx_scale=b["dx_scale"])
        if grads:
            out.update({k: v for k, v in (b if rows is None else oracle.rmsnorm_bwd(x, dy, h["weight"], e, want_dx=False, form=form)).items()
                        if k.startswith("dweight")})
    return out


def compare(layer: str, gpu: Dict[str, torch.Tensor], ora: Dict[str, np.ndarray], xdt: torch.dtype,
            pdt: torch.dtype, rows: Optional[Sequence[int]] = None, grads: bool = True) -> List[tol.Report]:
    def pick(t):
        t = t.reshape(-1, t.shape[-1]) if t.dim() > 1 else t
        return t if rows is None else t[torch.as_tensor(list(rows), device=t.device)]

    reps = [tol.compare(f"{layer}.y", pick(gpu["y"]), ora["y"], ora["y_scale"], xdt,
                        alt=ora.get("y_alt")),
            tol.compare(f"{layer}.dx", pick(gpu["dx"]), ora["dx"], ora["dx_scale"], xdt)]
    if "mean" in gpu:
        reps.append(tol.compare(f"{layer}.mean", pick(gpu["mean"]), ora["mean"], ora["mean_scale"], torch.float32))
    if "rstd" in gpu:
        # LayerNorm: the oracle's magnitude-based scale; RMSNorm: mean(x^2) has no cancellation,
        # so the scale is rstd itself (a plain relative bound)
        reps.append(tol.compare(f"{layer}.rstd", pick(gpu["rstd"]), ora["rstd"], ora.get("rstd_scale", ora["rstd"]),
                                torch.float32))
    if grads:
        for n in GRAD_NAMES[layer]:
            if gpu.get(n) is not None:
                reps.append(tol.compare_param(f"{layer}.{n}", gpu[n], ora[n], ora[n + "_scale"], pdt,
                                              slack=ora.get(n + "_slack")))
    return reps


def check_workload(wl: workloads.Workload, device="cuda", rows: Optional[Sequence[int]] = None,
                   use_stats: bool = True, inputs=None, on_gpu_inputs: bool = False) -> List[tol.Report]:
    """Full round trip of one workload: inputs -> HIP path and oracle -> reports."""
    if inputs is None:
        inputs = workloads.make_inputs(wl, device if on_gpu_inputs else "cpu")
    dev_in = {k: v.to(device) for k, v in inputs.items()}
    g = gpu_run(wl.layer, dev_in, wl.eps, use_stats, form=wl.form)
    torch.cuda.synchronize()
    o = oracle_run(wl.layer, inputs, wl.eps, rows=rows, form=wl.form)
    return compare(wl.layer, g, o, DT[wl.xdt], DT[wl.pdt], rows=rows)


def sample_rows(M: int, k: int = 48, seed: int = 0) -> List[int]:
    """First, last and tile-boundary rows plus a seeded random sample."""
    fixed = {0, 1, 2, M - 1, M - 2, M // 2}
    for b in (64, 128, 256, 1024, 4096):
        if M > b:
            fixed.update({b - 1, b})
    rng = np.random.default_rng(seed)
    fixed.update(int(r) for r in rng.integers(0, M, size=k))
    return sorted(r for r in fixed if 0 <= r < M)


def tile_rows(wl: workloads.Workload, n_wg: int = 16) -> List[int]:
    """Rows of whole launch tiles: for n_wg workgroups spread over the grid of the forward and of
    the backward plan, the first, a middle and the last tile each visits, plus the grid's last
    tile.  Every row of those tiles is returned, so each sampled tile is compared whole."""
    rows = set()
    for bwd in (False, True):
        p = rwn.plan(wl.layer, bwd, wl.M, wl.N, DT[wl.xdt], param_dtype=None if bwd else DT[wl.pdt])
        rpt = p["rpp"] * p["rt"]
        ntiles = p["ntiles"]
        stride = p["grid"] // p["ncb"]          # tile stride of a strided (persistent) grid
        tiles = {ntiles - 1}
        for i in range(min(n_wg, stride)):
            w = (i * stride) // min(n_wg, stride)
            if p["strided"]:
                cnt = (ntiles - w + stride - 1) // stride
                if cnt <= 0:
                    continue
                tiles.update({w, w + (cnt // 2) * stride, w + (cnt - 1) * stride})
            else:
                kt = p["kt"]
                t0, t1 = w * kt, min(ntiles, (w + 1) * kt)
                if t0 < t1:
                    tiles.update({t0, (t0 + t1 - 1) // 2, t1 - 1})
        for t in tiles:
            rows.update(range(t * rpt, min(wl.M, (t + 1) * rpt)))
    return sorted(rows)


def check_full_rows(wl: workloads.Workload, device="cuda", chunk_elems: int = 1 << 22,
                    use_stats: bool = True) -> List[tol.Report]:
    """Every element of y, dx and the statistics against the oracle, and the parameter
    gradients over all rows; the oracle runs on row chunks of about chunk_elems elements so
    host memory stays bounded.  Inputs are drawn on the device (one host copy for the oracle);
    outputs and workspace are NaN-poisoned before the GPU calls."""
    dev_in = workloads.make_inputs(wl, device)
    g = gpu_run(wl.layer, dev_in, wl.eps, use_stats, form=wl.form, grads=wl.param_grads)
    torch.cuda.synchronize()
    h = {k: v.detach().cpu() for k, v in dev_in.items()}
    del dev_in
    xdt, pdt = DT[wl.xdt], DT[wl.pdt]
    # parameter gradients: all rows at once (rows=[0] keeps the oracle's y/dx to one row)
    o = oracle_run(wl.layer, h, wl.eps, rows=[0], form=wl.form)
    reps = [tol.compare_param(f"{wl.layer}.{n}", g[n], o[n], o[n + "_scale"], pdt, slack=o.get(n + "_slack"))
            for n in GRAD_NAMES[wl.layer] if g.get(n) is not None]
    step = max(1, chunk_elems // wl.N)
    parts: Dict[str, List[tol.Report]] = {}
    for r0 in range(0, wl.M, step):
        r1 = min(wl.M, r0 + step)
        sub = {k: (v[r0:r1] if k in ("x", "dy") else v) for k, v in h.items()}
        oc = oracle_run(wl.layer, sub, wl.eps, grads=False, form=wl.form)
        gc_ = {k: g[k].reshape(-1, wl.N)[r0:r1] for k in ("y", "dx")}
        for k in ("mean", "rstd"):
            if k in g:
                gc_[k] = g[k][r0:r1]
        for r in compare(wl.layer, gc_, oc, xdt, pdt, grads=False):
            parts.setdefault(r.name, []).append(r)
    reps += [tol.merge(v) for v in parts.values()]
    return reps
