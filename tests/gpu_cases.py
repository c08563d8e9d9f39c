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


def gpu_run(layer: str, inp: Dict[str, torch.Tensor], eps: float, use_stats: bool = True,
            form: str = "cast_then_weight") -> Dict[str, torch.Tensor]:
    """Forward then backward on the tensors' device (dy is the upstream gradient of y)."""
    x, dy = inp["x"], inp["dy"]
    if layer == "dyt":
        y = rwn.dyt_fwd(x, inp["alpha"], inp["gamma"], inp["beta"])
        dx, da, dg, db = rwn.dyt_bwd(x, dy, inp["alpha"], inp["gamma"])
        return {"y": y, "dx": dx, "dalpha": da, "dgamma": dg, "dbeta": db}
    if layer == "layernorm":
        y, mean, rstd = rwn.layernorm_fwd(x, inp.get("gamma"), inp.get("beta"), eps)
        if not use_stats:
            mean = rstd = None
        dx, dg, db = rwn.layernorm_bwd(x, dy, mean, rstd, inp.get("gamma"), eps)
        out = {"y": y, "dx": dx, "dgamma": dg, "dbeta": db}
        if use_stats:
            out.update(mean=mean, rstd=rstd)
        return out
    y, rstd = rwn.rmsnorm_fwd(x, inp["weight"], eps, form=form)
    dx, dw = rwn.rmsnorm_bwd(x, dy, rstd if use_stats else None, inp["weight"], eps, form=form)
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
        mean = pick(gpu["mean"])
        reps.append(tol.compare(f"{layer}.mean", mean, ora["mean"], np.abs(ora["mean"]) + 1.0 / ora["rstd"],
                                torch.float32))
    if "rstd" in gpu:
        reps.append(tol.compare(f"{layer}.rstd", pick(gpu["rstd"]), ora["rstd"], ora["rstd"], torch.float32))
    if grads:
        names = {"dyt": ["dgamma", "dbeta", "dalpha"], "layernorm": ["dgamma", "dbeta"], "rmsnorm": ["dweight"]}[layer]
        for n in names:
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
