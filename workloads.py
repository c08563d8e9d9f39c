"""Seeded synthetic inputs for the row-wise normalization layers (DyT, LayerNorm, RMSNorm).

This module only draws random tensors.  It holds none of the layers' arithmetic, so the
GPU path and the CPU oracle can both consume what it produces without sharing code.

Each workload is named by what it is (layer, dtype, shape).  The shapes and value
distributions follow the pages' workloads:

* DyT with a scalar alpha (Liger-Kernel PR #1617, "fix(dyt): use a 1D grid and tile
  small-width rows", Summary): narrow rows, M far above 65,535, alpha = +inf / 0 edge runs.
* LayerNorm over a normalized dim of 24 at M = 25088*16 (intel/torch-xpu-ops PR #1880,
  "Layernorm bwd OPT", the tnt_s_patch16_224 shape [25088,16,24] in the description).
* Llama-style RMSNorm at hidden sizes 2048 and 4096 with bf16 weight (DeepSpeed PR #8664 /
  #8645, Summary and "Which modules are replaced").

Readings used where the pages are silent: N(mu, s) means standard deviation s; "1%
outliers x10" is an i.i.d. per-element Bernoulli(0.01) scaling by 10; unstated dy is
N(0,1); unstated DyT params follow the first DyT workload.

Every tensor is drawn in float32 from its own seeded ``torch.Generator`` on the requested
device, then rounded (round-to-nearest-even, torch's ``.to``) to its storage dtype, so both
consumers see identical bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

BASE_SEED = 20261202

LAYERS = ("dyt", "layernorm", "rmsnorm")
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration: layer, shape, dtypes and value distributions."""

    name: str
    layer: str
    M: int
    N: int
    xdt: str                      # "f32" | "bf16" | "f16"
    pdt: str                      # dtype of alpha/gamma/beta or of the RMSNorm weight
    seed: int
    x_std: float = 1.0
    outlier_frac: float = 0.0     # Bernoulli probability of scaling an element of x by 10
    dy_std: float = 1.0
    gamma_mean: float = 1.0
    gamma_std: float = 0.1
    beta_mean: float = 0.0
    beta_std: float = 0.1
    alpha: float = 0.5            # DyT only
    form: str = "cast_then_weight"  # RMSNorm form: cast_then_weight | weight_then_cast | one_plus_weight
    param_grads: bool = True        # False: the backward is asked for dx only (frozen parameters)
    eps: float = 1e-5             # LayerNorm / RMSNorm only

    def with_shape(self, M: int, N: Optional[int] = None) -> "Workload":
        return dataclasses.replace(self, M=M, N=self.N if N is None else N,
                                   name=f"{self.name}@{M}x{self.N if N is None else N}")

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def elems(self) -> int:
        return self.M * self.N

    def algorithmic_bytes(self) -> Dict[str, int]:
        """HBM bytes one forward and one backward must move at minimum.

        fwd: read x, write y (+ write the per-row float32 stats: 8 B/row LayerNorm,
        4 B/row RMSNorm).  bwd: read x, dy and the stats, write dx.  The O(N) parameters and
        their gradients are included.
        """
        sx = 4 if self.xdt == "f32" else 2
        sp = 4 if self.pdt == "f32" else 2
        stats = {"dyt": 0, "layernorm": 8, "rmsnorm": 4}[self.layer] * self.M
        nparam_vec = {"dyt": 2, "layernorm": 2, "rmsnorm": 1}[self.layer]
        scalar = sp if self.layer == "dyt" else 0
        params = nparam_vec * self.N * sp + scalar
        fwd = 2 * self.elems * sx + stats + params
        # bwd reads x, dy, stats and the params it needs; writes dx and the param grads.
        # gamma (+alpha) read; grads written (none when only dx is asked for)
        bwd_params = (self.N * sp + scalar) + (params if self.param_grads else 0)
        bwd = 3 * self.elems * sx + stats + bwd_params
        return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}


def _cfg_seed(k: int) -> int:
    return BASE_SEED + k


# The five synthetic configurations, in order.  Index 0 is the small case the oracle finishes
# in seconds; index 1 is the headline throughput workload.
def standard_workloads() -> Dict[str, Workload]:
    w: Dict[str, Workload] = {}
    w["dyt_f32_4096x64"] = Workload("dyt_f32_4096x64", "dyt", 4096, 64, "f32", "f32",
                                    _cfg_seed(1), alpha=0.5)
    w["layernorm_f32_401408x24"] = Workload("layernorm_f32_401408x24", "layernorm", 25088 * 16, 24,
                                            "f32", "f32", _cfg_seed(2), x_std=2.0, eps=1e-5)
    for n in (32, 128, 256):
        w[f"dyt_bf16_1048573x{n}"] = Workload(f"dyt_bf16_1048573x{n}", "dyt", 1048573, n, "bf16", "f32",
                                              _cfg_seed(3), alpha=0.5)
    for (m, n) in ((16384, 2048), (8192, 4096)):
        w[f"rmsnorm_bf16_{m}x{n}"] = Workload(f"rmsnorm_bf16_{m}x{n}", "rmsnorm", m, n, "bf16", "bf16",
                                              _cfg_seed(4), outlier_frac=0.01, gamma_mean=1.0,
                                              gamma_std=0.02, eps=1e-6)
    for layer in LAYERS:
        for n in (1025, 4096, 8192, 16384):
            eps = {"dyt": 0.0, "layernorm": 1e-5, "rmsnorm": 1e-6}[layer]
            w[f"wide_{layer}_bf16_65536x{n}"] = Workload(
                f"wide_{layer}_bf16_65536x{n}", layer, 65536, n, "bf16", "f32", _cfg_seed(5),
                gamma_mean=1.0, gamma_std=0.1, beta_mean=1.0, beta_std=0.1, alpha=0.5, eps=eps)
    # float16 counterparts of one shape from each of configurations 3, 4 and 5 (same seeds and
    # value distributions; float16 activations, parameters as in the bfloat16 originals but in
    # float16 where those were bfloat16).
    for base, pdt in (("dyt_bf16_1048573x128", "f32"), ("rmsnorm_bf16_16384x2048", "f16"),
                      ("wide_layernorm_bf16_65536x4096", "f32")):
        name = base.replace("bf16", "f16")
        w[name] = dataclasses.replace(w[base], name=name, xdt="f16", pdt=pdt)
    # Backwards asked for dx only (frozen parameters): no column partials and no second pass.
    for base in ("layernorm_f32_401408x24", "dyt_bf16_1048573x128", "wide_rmsnorm_bf16_65536x4096"):
        name = base + "_dx_only"
        w[name] = dataclasses.replace(w[base], name=name, param_grads=False)
    # The two float32 RMSNorm forms at configuration 4's first shape.
    for form in ("weight_then_cast", "one_plus_weight"):
        name = f"rmsnorm_{form}_bf16_16384x2048"
        w[name] = dataclasses.replace(w["rmsnorm_bf16_16384x2048"], name=name, form=form)
    return w


WORKLOADS = standard_workloads()
HEADLINE = "layernorm_f32_401408x24"


def _gen(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, mean: float, std: float, seed: int, device) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def make_inputs(wl: Workload, device="cpu", seed_offset: int = 0) -> Dict[str, torch.Tensor]:
    """Draw every input of ``wl`` on ``device``.

    Returns x, dy (storage dtype = wl.xdt) and the parameters (dtype = wl.pdt):
    DyT: alpha [1], gamma [N], beta [N]; LayerNorm: gamma, beta; RMSNorm: weight.
    Tensor k uses seed ``wl.seed * 16 + k + seed_offset``.
    """
    device = torch.device(device)
    s = wl.seed * 16 + seed_offset
    xdt, pdt = DTYPES[wl.xdt], DTYPES[wl.pdt]
    x = _normal((wl.M, wl.N), 0.0, wl.x_std, s + 0, device)
    if wl.outlier_frac > 0.0:
        u = torch.rand((wl.M, wl.N), generator=_gen(device, s + 1), device=device)
        x = torch.where(u < wl.outlier_frac, x * 10.0, x)
        del u
    x = x.to(xdt)
    if wl.layer == "dyt" and math.isinf(wl.alpha):
        # With alpha = +inf an exact zero is a true NaN (tanh(inf * 0)); the generators can emit
        # 0.0 (about once per 2^24 draws), so such elements are moved to the smallest normal.
        tiny = torch.finfo(xdt).tiny
        x = torch.where(x == 0, torch.full_like(x, tiny), x)
    out = {"x": x}
    del x
    out["dy"] = _normal((wl.M, wl.N), 0.0, wl.dy_std, s + 2, device).to(xdt)
    if wl.layer == "dyt":
        out["alpha"] = torch.full((1,), wl.alpha, device=device, dtype=torch.float32).to(pdt)
        out["gamma"] = _normal((wl.N,), wl.gamma_mean, wl.gamma_std, s + 3, device).to(pdt)
        out["beta"] = _normal((wl.N,), wl.beta_mean, wl.beta_std, s + 4, device).to(pdt)
    elif wl.layer == "layernorm":
        out["gamma"] = _normal((wl.N,), wl.gamma_mean, wl.gamma_std, s + 3, device).to(pdt)
        out["beta"] = _normal((wl.N,), wl.beta_mean, wl.beta_std, s + 4, device).to(pdt)
    elif wl.layer == "rmsnorm":
        out["weight"] = _normal((wl.N,), wl.gamma_mean, wl.gamma_std, s + 3, device).to(pdt)
    else:
        raise ValueError(wl.layer)
    return out


def small(layer: str, M: int, N: int, xdt: str = "f32", pdt: str = "f32", seed: int = 7,
          **kw) -> Workload:
    """A small ad-hoc workload (edge shapes, parity sweeps)."""
    defaults = {"dyt": dict(alpha=0.5), "layernorm": dict(eps=1e-5), "rmsnorm": dict(eps=1e-6)}[layer]
    defaults.update(kw)
    return Workload(f"{layer}_{xdt}_{pdt}_{M}x{N}", layer, M, N, xdt, pdt, seed, **defaults)


def eps_f32(eps: float) -> float:
    """The epsilon both sides use: the float32 value nearest to ``eps`` (eager adds a Python
    float to a float32 tensor, so the effective epsilon is float32)."""
    import struct
    return struct.unpack("f", struct.pack("f", eps))[0] if math.isfinite(eps) else eps
