"""torch.autograd integration: Functions and modules over the binding (first-order only).

The forward of each Function is the binding's forward entry point and its backward the
binding's backward entry point, so every step still runs in the library's HIP kernels; the
Functions only decide what to save and which gradients to ask for.  Backward is
once-differentiable: a double backward raises, as the library's gradients are first-order.
The Functions and this package's own modules have no fallback: a CPU tensor or an unsupported
dtype raises, as the binding does.  Only modules installed by ``swap_norms`` in place of a
model's own norms run that model's original eager forward, for inputs the kernels do not take
(DeepSpeed PR #8645, "Where the kernels run").

Layers (each forward cites the passage that defines it in include/rwnorm.h):
  DyT        y = weight * tanh(alpha * x) + bias, scalar alpha
  LayerNorm  torch.nn.LayerNorm over the last dimension (affine and bias optional)
  RMSNorm    weight * (x.float() * rsqrt(mean(x.float()^2) + eps)).to(x.dtype)
"""
from __future__ import annotations

import importlib
import warnings
from typing import Optional

import torch
from torch import nn
from torch.autograd.function import once_differentiable

from . import _lib, dyt_bwd, dyt_fwd, layernorm_bwd, layernorm_fwd, rmsnorm_bwd, rmsnorm_fwd

__all__ = ["DyTFunction", "LayerNormFunction", "RMSNormFunction", "DyT", "LayerNorm", "RMSNorm",
           "dyt", "layer_norm", "rms_norm", "swap_norms", "RMS_NORM_CLASSES"]


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
        dx, dg, db = layernorm_bwd(x, dy, mean, rstd, weight, ctx.eps, param_dtype=ctx.param_dtype,
                                   need_dgamma=bool(n[1]), need_dbeta=bool(n[2]))
        gw = dg.reshape(ctx.shapes[0]) if n[1] else None
        gb = db.reshape(ctx.shapes[1]) if n[2] else None
        return dx, gw, gb, None


class RMSNormFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, eps, form="cast_then_weight"):
        y, rstd = rmsnorm_fwd(x, weight, eps, form=form)
        ctx.save_for_backward(x, rstd, weight)
        ctx.eps = eps
        ctx.form = form
        return y

    @staticmethod
    @once_differentiable
    def backward(ctx, dy):
        x, rstd, weight = ctx.saved_tensors
        need = bool(ctx.needs_input_grad[1])
        dx, dw = rmsnorm_bwd(x, dy, rstd, weight, ctx.eps, need_param_grads=need, form=ctx.form)
        return dx, (dw.reshape(weight.shape) if need else None), None, None


def dyt(x: torch.Tensor, alpha: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    return DyTFunction.apply(x, alpha, weight, bias)


def layer_norm(x: torch.Tensor, weight: Optional[torch.Tensor], bias: Optional[torch.Tensor],
               eps: float = 1e-5) -> torch.Tensor:
    return LayerNormFunction.apply(x, weight, bias, float(eps))


def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, form: str = "cast_then_weight") -> torch.Tensor:
    """RMSNorm of one of the library's forms: "cast_then_weight" (Llama), "weight_then_cast",
    "one_plus_weight" (Gemma)."""
    return RMSNormFunction.apply(x, weight, float(eps), form)


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
    """RMSNorm with float32 statistics in one of the library's forms: "cast_then_weight" (the
    Llama form: the normalized value rounded to x's dtype, then the weight multiply),
    "weight_then_cast" or "one_plus_weight" (multiply in float32 by weight or 1 + weight, one
    rounding)."""

    def __init__(self, hidden_size: int, eps: float = 1e-6, form: str = "cast_then_weight", device=None, dtype=None):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(hidden_size, device=device, dtype=dtype))
        self.variance_epsilon = eps
        self.form = form

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return rms_norm(x, self.weight, self.variance_epsilon, self.form)

    def extra_repr(self) -> str:
        return f"{tuple(self.weight.shape)}, eps={self.variance_epsilon}, form={self.form}"


# ------------------------------------------------------------------------------- swap_norms
#
# Which RMSNorm classes take which form is decided by an explicit list of exact classes, not by
# their attributes: a 1-D weight and a float epsilon do not fix where the weight meets the
# rounding to x's dtype (DeepSpeed PR #8645, "Which modules are replaced").  Each listed class's
# forward is checked against its form's eager expression by tests/test_autograd.py on the
# installed transformers, so a class that changes its cast order upstream fails there.
RMS_NORM_CLASSES = {
    "cast_then_weight": ["llama.LlamaRMSNorm", "mistral.MistralRMSNorm", "mixtral.MixtralRMSNorm",
                         "phi3.Phi3RMSNorm", "qwen2.Qwen2RMSNorm", "qwen2_moe.Qwen2MoeRMSNorm",
                         "qwen3.Qwen3RMSNorm", "qwen3_moe.Qwen3MoeRMSNorm", "deepseek_v2.DeepseekV2RMSNorm",
                         "deepseek_v3.DeepseekV3RMSNorm"],
    "weight_then_cast": ["olmo2.Olmo2RMSNorm", "olmo3.Olmo3RMSNorm", "flex_olmo.FlexOlmoRMSNorm",
                         "gpt_oss.GptOssRMSNorm", "helium.HeliumRMSNorm"],
    "one_plus_weight": ["gemma.GemmaRMSNorm", "gemma2.Gemma2RMSNorm", "gemma3.Gemma3RMSNorm"],
}


def rms_norm_classes():
    """{class: form} for the listed classes the installed transformers defines."""
    out = {}
    for form, names in RMS_NORM_CLASSES.items():
        for qual in names:
            mod, cls = qual.split(".")
            try:
                m = importlib.import_module(f"transformers.models.{mod}.modeling_{mod}")
            except Exception:   # transformers absent, or a model it does not have
                continue
            c = getattr(m, cls, None)
            if isinstance(c, type):
                out[c] = form
    return out


_WARNED = set()


def _eager_once(kind: str, why: str) -> None:
    if kind not in _WARNED:
        _WARNED.add(kind)
        warnings.warn(f"{kind}: {why}; running the module's own eager forward (warned once)", stacklevel=3)


_KERNEL_DTYPES = (torch.float32, torch.bfloat16, torch.float16)


def _rows_supported(x: torch.Tensor, params) -> Optional[str]:
    """None if the kernels take x with these parameters, else why not."""
    if not x.is_cuda:
        return "input on the host"
    if x.dtype not in _KERNEL_DTYPES:
        return f"input dtype {x.dtype}"
    ps = [p for p in params if p is not None]
    if any(p.device != x.device for p in ps):
        return "parameters on another device"
    pdts = {p.dtype for p in ps}
    if len(pdts) > 1 or (pdts and next(iter(pdts)) not in (torch.float32, x.dtype)) or \
            (x.dtype == torch.float32 and pdts and next(iter(pdts)) != torch.float32):
        return f"parameter dtype {sorted(map(str, pdts))} with input {x.dtype}"
    n = x.shape[-1] if x.dim() else 0
    if n < 1 or n > (16377 if x.element_size() == 2 else 16381):
        return f"width {n}"
    return None


class _SwappedLayerNorm(LayerNorm):
    """LayerNorm installed by swap_norms; the original module (sharing its Parameters) runs
    inputs the kernels do not take."""

    def forward(self, x):
        why = _rows_supported(x, (self.weight, self.bias))
        if why is None:
            return layer_norm(x, self.weight, self.bias, self.eps)
        _eager_once("LayerNorm", why)
        return self._eager(x)


class _SwappedRMSNorm(RMSNorm):
    """RMSNorm installed by swap_norms in place of a listed class (see RMS_NORM_CLASSES)."""

    def forward(self, x):
        why = _rows_supported(x, (self.weight,))
        if why is None and self.form == "cast_then_weight" and self.weight.dtype != x.dtype:
            # the eager Llama form returns the promoted dtype (float32 for a float32 weight)
            why = f"weight dtype {self.weight.dtype} with input {x.dtype}"
        if why is None:
            return rms_norm(x, self.weight, self.variance_epsilon, self.form)
        _eager_once(type(self._eager).__name__, why)
        return self._eager(x)


def _unpatched(m: nn.Module) -> bool:
    """The module runs its own class's forward: not patched on the instance, not wrapped."""
    return "forward" not in vars(m) and not hasattr(type(m).forward, "__wrapped__")


def swap_norms(model: nn.Module) -> int:
    """Opt-in module swap: replaces, in place, every exact torch.nn.LayerNorm over one dimension
    and every exact instance of a listed RMSNorm class (RMS_NORM_CLASSES, in its own form) with
    this package's module, sharing the original Parameter objects.  Subclasses, look-alikes and
    modules whose forward was patched or wrapped are left alone.  A swapped module runs the
    kernels on every input they take; for any other input (host tensors, float64, mixed
    parameter dtypes, a Llama-form float32 weight under a 16-bit input) it runs the original
    module's eager forward, with one warning.  Returns the number of modules replaced; raises if
    the HIP library is not built."""
    _lib.load()
    classes = rms_norm_classes()
    count = 0
    for name, child in list(model.named_children()):
        new = None
        if type(child) is nn.LayerNorm and len(child.normalized_shape) == 1 and _unpatched(child):
            new = _SwappedLayerNorm.__new__(_SwappedLayerNorm)
            nn.Module.__init__(new)
            new.normalized_shape = tuple(child.normalized_shape)
            new.eps = child.eps
            new.weight = child.weight
            new.bias = child.bias
        elif type(child) in classes and _unpatched(child) and getattr(child, "weight", None) is not None:
            eps = getattr(child, "variance_epsilon", getattr(child, "eps", None))
            if isinstance(eps, float):
                new = _SwappedRMSNorm.__new__(_SwappedRMSNorm)
                nn.Module.__init__(new)
                new.weight = child.weight
                new.variance_epsilon = eps
                new.form = classes[type(child)]
        if new is not None:
            object.__setattr__(new, "_eager", child)    # not a submodule: no second state-dict entry
            setattr(model, name, new)
            count += 1
        else:
            count += swap_norms(child)
    return count
