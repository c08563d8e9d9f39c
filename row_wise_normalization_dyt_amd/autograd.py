"""torch.autograd integration: Functions and modules over the binding (first-order only).

The forward of each Function is the binding's forward entry point and its backward the
binding's backward entry point, so every step still runs in the library's HIP kernels; the
Functions only decide what to save and which gradients to ask for.  Backward is
once-differentiable: a double backward raises, as the library's gradients are first-order.
There is no fallback: a CPU tensor or an unsupported dtype raises, as the binding does.

Layers (each forward cites the passage that defines it in include/rwnorm.h):
  DyT        y = weight * tanh(alpha * x) + bias, scalar alpha
  LayerNorm  torch.nn.LayerNorm over the last dimension (affine and bias optional)
  RMSNorm    weight * (x.float() * rsqrt(mean(x.float()^2) + eps)).to(x.dtype)
"""
from __future__ import annotations

from typing import Optional

import torch
from torch import nn
from torch.autograd.function import once_differentiable

from . import dyt_bwd, dyt_fwd, layernorm_bwd, layernorm_fwd, rmsnorm_bwd, rmsnorm_fwd

__all__ = ["DyTFunction", "LayerNormFunction", "RMSNormFunction", "DyT", "LayerNorm", "RMSNorm",
           "dyt", "layer_norm", "rms_norm", "swap_norms"]


class DyTFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, alpha, weight, bias):
        ctx.save_for_backward(x, alpha, weight)
        return dyt_fwd(x, alpha, weight, bias)

    @staticmethod
    @once_differentiable
    def backward(ctx, dy):
        x, alpha, weight = ctx.saved_tensors
        need = any(ctx.needs_input_grad[1:])
        dx, da, dg, db = dyt_bwd(x, dy, alpha, weight, need_param_grads=need)
        if not need:
            return dx, None, None, None
        n = ctx.needs_input_grad
        return (dx, da.reshape(alpha.shape) if n[1] else None, dg.reshape(weight.shape) if n[2] else None,
                db.reshape(weight.shape) if n[3] else None)


class LayerNormFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, eps):
        y, mean, rstd = layernorm_fwd(x, weight, bias, eps)
        ctx.save_for_backward(x, mean, rstd, weight)
        ctx.eps = eps
        ctx.param_dtype = weight.dtype if weight is not None else (bias.dtype if bias is not None else None)
        ctx.shapes = (None if weight is None else weight.shape, None if bias is None else bias.shape)
        return y

    @staticmethod
    @once_differentiable
    def backward(ctx, dy):
        x, mean, rstd, weight = ctx.saved_tensors
        n = ctx.needs_input_grad
        need = bool(n[1] or n[2])
        dx, dg, db = layernorm_bwd(x, dy, mean, rstd, weight, ctx.eps, param_dtype=ctx.param_dtype,
                                   need_param_grads=need)
        gw = dg.reshape(ctx.shapes[0]) if need and n[1] else None
        gb = db.reshape(ctx.shapes[1]) if need and n[2] else None
        return dx, gw, gb, None


class RMSNormFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, eps):
        y, rstd = rmsnorm_fwd(x, weight, eps)
        ctx.save_for_backward(x, rstd, weight)
        ctx.eps = eps
        return y

    @staticmethod
    @once_differentiable
    def backward(ctx, dy):
        x, rstd, weight = ctx.saved_tensors
        need = bool(ctx.needs_input_grad[1])
        dx, dw = rmsnorm_bwd(x, dy, rstd, weight, ctx.eps, need_param_grads=need)
        return dx, (dw.reshape(weight.shape) if need else None), None


def dyt(x: torch.Tensor, alpha: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    return DyTFunction.apply(x, alpha, weight, bias)


def layer_norm(x: torch.Tensor, weight: Optional[torch.Tensor], bias: Optional[torch.Tensor],
               eps: float = 1e-5) -> torch.Tensor:
    return LayerNormFunction.apply(x, weight, bias, float(eps))


def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    return RMSNormFunction.apply(x, weight, float(eps))


class DyT(nn.Module):
    """Dynamic Tanh over the last dimension: a learnable scalar alpha (initial value
    ``alpha_init``) and per-channel weight (ones) and bias (zeros)."""

    def __init__(self, num_features: int, alpha_init: float = 0.5, device=None, dtype=None):
        super().__init__()
        kw = dict(device=device, dtype=dtype)
        self.num_features = num_features
        self.alpha = nn.Parameter(torch.full((1,), float(alpha_init), **kw))
        self.weight = nn.Parameter(torch.ones(num_features, **kw))
        self.bias = nn.Parameter(torch.zeros(num_features, **kw))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return dyt(x, self.alpha, self.weight, self.bias)

    def extra_repr(self) -> str:
        return f"{self.num_features}"


class LayerNorm(nn.Module):
    """torch.nn.LayerNorm over the last dimension (normalized_shape is one integer)."""

    def __init__(self, normalized_shape: int, eps: float = 1e-5, elementwise_affine: bool = True,
                 bias: bool = True, device=None, dtype=None):
        super().__init__()
        kw = dict(device=device, dtype=dtype)
        self.normalized_shape = (int(normalized_shape),)
        self.eps = eps
        self.weight = nn.Parameter(torch.ones(self.normalized_shape, **kw)) if elementwise_affine else None
        self.bias = nn.Parameter(torch.zeros(self.normalized_shape, **kw)) if elementwise_affine and bias else None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return layer_norm(x, self.weight, self.bias, self.eps)

    def extra_repr(self) -> str:
        return f"{self.normalized_shape}, eps={self.eps}, elementwise_affine={self.weight is not None}"


class RMSNorm(nn.Module):
    """Llama-style RMSNorm: float32 statistics, the normalized value rounded to x's dtype,
    then the weight multiply."""

    def __init__(self, hidden_size: int, eps: float = 1e-6, device=None, dtype=None):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(hidden_size, device=device, dtype=dtype))
        self.variance_epsilon = eps

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return rms_norm(x, self.weight, self.variance_epsilon)

    def extra_repr(self) -> str:
        return f"{tuple(self.weight.shape)}, eps={self.variance_epsilon}"


def _is_llama_rmsnorm(m: nn.Module) -> bool:
    """A module of the Llama RMSNorm form: a 1-D ``weight`` parameter and a float
    ``variance_epsilon``, nothing else learnable."""
    w = getattr(m, "weight", None)
    return (isinstance(w, nn.Parameter) and w.dim() == 1 and isinstance(getattr(m, "variance_epsilon", None), float)
            and sum(1 for _ in m.parameters(recurse=False)) == 1 and not isinstance(m, RMSNorm))


def swap_norms(model: nn.Module) -> int:
    """Opt-in module swap: replaces, in place, every torch.nn.LayerNorm over one dimension and
    every module of the Llama RMSNorm form with this package's module, sharing the original
    Parameter objects.  Returns the number of modules replaced.  Inputs the library does not
    support raise at call time; nothing falls back to another implementation."""
    count = 0
    for name, child in list(model.named_children()):
        new = None
        if isinstance(child, nn.LayerNorm) and len(child.normalized_shape) == 1:
            new = LayerNorm.__new__(LayerNorm)
            nn.Module.__init__(new)
            new.normalized_shape = tuple(child.normalized_shape)
            new.eps = child.eps
            new.weight = child.weight
            new.bias = child.bias
        elif _is_llama_rmsnorm(child):
            new = RMSNorm.__new__(RMSNorm)
            nn.Module.__init__(new)
            new.weight = child.weight
            new.variance_epsilon = child.variance_epsilon
        if new is not None:
            setattr(model, name, new)
            count += 1
        else:
            count += swap_norms(child)
    return count
