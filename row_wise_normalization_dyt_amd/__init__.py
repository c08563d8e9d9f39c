"""Row-wise normalization for MI355X (gfx950): DyT, LayerNorm and RMSNorm, forward and backward.

Thin binding over librwnorm's C ABI (include/rwnorm.h), with the same entry-point names.  It
only marshals arguments: shapes and dtypes are checked, leading dimensions flattened to [M, N],
non-contiguous inputs copied, outputs and the backward workspace allocated with torch, and the
call enqueued on the current stream of the tensors' device.  Every step of the computation
runs in the library's HIP kernels; there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

__all__ = ["dyt_fwd", "dyt_bwd", "layernorm_fwd", "layernorm_bwd", "rmsnorm_fwd", "rmsnorm_bwd",
           "workspace_size", "version", "trace_begin", "trace_end", "stream_probe", "plan", "RwnError"]

RwnError = _lib.RwnError
_DT = {torch.float32: _lib.RWN_F32, torch.bfloat16: _lib.RWN_BF16, torch.float16: _lib.RWN_F16}


def _L():
    return _lib.load()


def _dt(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{name}: dtype {t.dtype} is not supported (float32, bfloat16 or float16)")
    return _DT[t.dtype]


def _as_2d(x: torch.Tensor, name: str) -> torch.Tensor:
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if x.dim() < 1:
        raise ValueError(f"{name} must have at least one dimension")
    x = x.contiguous()
    x = x.reshape(-1, x.shape[-1]) if x.dim() != 2 else x
    if x.data_ptr() % 16 and x.shape[-1] % (16 // x.element_size()) == 0:
        # Rows of a misaligned view would straddle chunk boundaries; an aligned copy takes the
        # faster aligned kernels.
        x = x.clone()
    return x


def _like(x2: torch.Tensor) -> torch.Tensor:
    """An empty [M, N] tensor whose address has x2's offset modulo 16 bytes (the library needs
    all [M, N] operands of a call to share it)."""
    esz = x2.element_size()
    off = (x2.data_ptr() % 16) // esz
    if off == 0:
        return torch.empty_like(x2)
    buf = torch.empty(x2.numel() + 16 // esz, dtype=x2.dtype, device=x2.device)
    shift = ((x2.data_ptr() - buf.data_ptr()) % 16) // esz
    return buf[shift:shift + x2.numel()].view(x2.shape)


def _pair(x2: torch.Tensor, dy2: torch.Tensor):
    """x and dy with a common address modulo 16 (copies both if they differ)."""
    if x2.data_ptr() % 16 != dy2.data_ptr() % 16:
        return x2.clone(), dy2.clone()
    return x2, dy2


def _vec(p: Optional[torch.Tensor], n: int, name: str, dev) -> Optional[torch.Tensor]:
    if p is None:
        return None
    if p.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    p = p.contiguous().reshape(-1)
    if p.numel() != n:
        raise ValueError(f"{name} must have {n} elements (got {p.numel()})")
    return p


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _param_dtype(*ps) -> int:
    dts = {p.dtype for p in ps if p is not None}
    if len(dts) != 1:
        raise TypeError(f"parameters must share one dtype (got {sorted(map(str, dts))})")
    return _dt(next(p for p in ps if p is not None), "parameters")


def workspace_size(layer: str, M: int, N: int, dtype: torch.dtype, device=None) -> int:
    """Backward workspace bytes for layer in {"dyt", "layernorm", "rmsnorm"}."""
    lib = _L()
    fn = {"dyt": "dyt_bwd_workspace_size", "layernorm": "layernorm_bwd_workspace_size",
          "rmsnorm": "rmsnorm_bwd_workspace_size"}[layer]
    out = ctypes.c_size_t(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _lib.check(lib, fn, getattr(lib, fn)(M, N, _DT[dtype], ctypes.byref(out)))
    return int(out.value)


def _workspace(layer: str, M: int, N: int, dtype, dev, given: Optional[torch.Tensor] = None) -> torch.Tensor:
    n = workspace_size(layer, M, N, dtype, dev)
    if given is None:
        return torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    if given.device != dev or not given.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    if given.numel() * given.element_size() < n:
        raise ValueError(f"workspace has {given.numel() * given.element_size()} bytes, {n} needed")
    return given


def _ws_bytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def _out_rows(given: Optional[torch.Tensor], x2: torch.Tensor, name: str) -> torch.Tensor:
    """An [M, N] output: a fresh tensor laid out like x2, or the caller's buffer (contiguous, x's
    dtype and device, M * N elements, the same address as x2 modulo 16 bytes)."""
    if given is None:
        return _like(x2)
    if given.device != x2.device or given.dtype != x2.dtype:
        raise ValueError(f"{name} must be a {x2.dtype} tensor on {x2.device}")
    if not given.is_contiguous() or given.numel() != x2.numel():
        raise ValueError(f"{name} must be contiguous with {x2.numel()} elements")
    if given.data_ptr() % 16 != x2.data_ptr() % 16:
        raise ValueError(f"{name} must share x's address modulo 16 bytes")
    return given.view(x2.shape)


def _out_vec(given: Optional[torch.Tensor], n: int, dtype, dev, name: str) -> torch.Tensor:
    """A length-n output vector: fresh, or the caller's contiguous buffer of that dtype."""
    if given is None:
        return torch.empty(n, dtype=dtype, device=dev)
    if given.device != dev or given.dtype != dtype or not given.is_contiguous() or given.numel() != n:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {n} elements on {dev}")
    return given.view(n)


# ------------------------------------------------------------------------------------ DyT

def dyt_fwd(x: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, *,
            y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = gamma * tanh(alpha * x) + beta over the last dimension; y has x's shape and dtype.
    y=: an output buffer to write instead of a fresh tensor."""
    lib = _L()
    x2 = _as_2d(x, "x")
    M, N = x2.shape
    alpha, gamma, beta = _vec(alpha, 1, "alpha", x2.device), _vec(gamma, N, "gamma", x2.device), _vec(beta, N, "beta", x2.device)
    y = _out_rows(y, x2, "y")
    with torch.cuda.device(x2.device):
        _lib.check(lib, "dyt_fwd", lib.dyt_fwd(M, N, _ptr(x2), _dt(x2, "x"), _ptr(alpha), _ptr(gamma), _ptr(beta),
                                               _param_dtype(alpha, gamma, beta), _ptr(y), _stream(x2.device)))
    return y.reshape(x.shape)


def dyt_bwd(x: torch.Tensor, dy: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor,
            need_param_grads: bool = True, *, dx: Optional[torch.Tensor] = None,
            dalpha: Optional[torch.Tensor] = None, dgamma: Optional[torch.Tensor] = None,
            dbeta: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, ...]:
    """Returns (dx, dalpha [1], dgamma [N], dbeta [N]); gradients in the parameters' dtype.
    dx=, dalpha=, dgamma=, dbeta=, workspace=: buffers to use instead of fresh tensors."""
    lib = _L()
    x2, dy2 = _as_2d(x, "x"), _as_2d(dy, "dy")
    if dy2.shape != x2.shape or dy2.dtype != x2.dtype:
        raise ValueError("dy must match x in shape and dtype")
    x2, dy2 = _pair(x2, dy2)
    M, N = x2.shape
    alpha, gamma = _vec(alpha, 1, "alpha", x2.device), _vec(gamma, N, "gamma", x2.device)
    pdt = _param_dtype(alpha, gamma)
    dx = _out_rows(dx, x2, "dx")
    da = _out_vec(dalpha, 1, gamma.dtype, x2.device, "dalpha") if need_param_grads else None
    dg = _out_vec(dgamma, N, gamma.dtype, x2.device, "dgamma") if need_param_grads else None
    db = _out_vec(dbeta, N, gamma.dtype, x2.device, "dbeta") if need_param_grads else None
    with torch.cuda.device(x2.device):
        ws = _workspace("dyt", M, N, x2.dtype, x2.device, workspace) if need_param_grads else None
        _lib.check(lib, "dyt_bwd", lib.dyt_bwd(M, N, _ptr(x2), _ptr(dy2), _dt(x2, "x"), _ptr(alpha), _ptr(gamma), pdt,
                                               _ptr(dx), _ptr(da), _ptr(dg), _ptr(db), _ptr(ws), _ws_bytes(ws),
                                               _stream(x2.device)))
    return dx.reshape(x.shape), da, dg, db


# ------------------------------------------------------------------------------ LayerNorm

def layernorm_fwd(x: torch.Tensor, gamma: Optional[torch.Tensor], beta: Optional[torch.Tensor], eps: float,
                  want_stats: bool = True, *, y: Optional[torch.Tensor] = None,
                  mean: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None):
    """Returns (y, mean [M] float32, rstd [M] float32); mean/rstd are None if not wanted.
    y=, mean=, rstd=: buffers to write instead of fresh tensors."""
    lib = _L()
    x2 = _as_2d(x, "x")
    M, N = x2.shape
    gamma, beta = _vec(gamma, N, "gamma", x2.device), _vec(beta, N, "beta", x2.device)
    pdt = _param_dtype(gamma, beta) if (gamma is not None or beta is not None) else _lib.RWN_F32
    y = _out_rows(y, x2, "y")
    mean = _out_vec(mean, M, torch.float32, x2.device, "mean") if want_stats else None
    rstd = _out_vec(rstd, M, torch.float32, x2.device, "rstd") if want_stats else None
    with torch.cuda.device(x2.device):
        _lib.check(lib, "layernorm_fwd", lib.layernorm_fwd(M, N, _ptr(x2), _dt(x2, "x"), _ptr(gamma), _ptr(beta), pdt,
                                                           float(eps), _ptr(y), _ptr(mean), _ptr(rstd),
                                                           _stream(x2.device)))
    return y.reshape(x.shape), mean, rstd


def layernorm_bwd(x: torch.Tensor, dy: torch.Tensor, mean: Optional[torch.Tensor], rstd: Optional[torch.Tensor],
                  gamma: Optional[torch.Tensor], eps: float, param_dtype: Optional[torch.dtype] = None,
                  need_param_grads: bool = True, *, dx: Optional[torch.Tensor] = None,
                  dgamma: Optional[torch.Tensor] = None, dbeta: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, need_dgamma: Optional[bool] = None,
                  need_dbeta: Optional[bool] = None):
    """Returns (dx, dgamma, dbeta).  mean/rstd None: recomputed from x.
    need_dgamma / need_dbeta (default: need_param_grads) select the parameter gradients; one
    not wanted is returned as None and its column partials are never formed.
    dx=, dgamma=, dbeta=, workspace=: buffers to use instead of fresh tensors."""
    lib = _L()
    x2, dy2 = _as_2d(x, "x"), _as_2d(dy, "dy")
    if dy2.shape != x2.shape or dy2.dtype != x2.dtype:
        raise ValueError("dy must match x in shape and dtype")
    x2, dy2 = _pair(x2, dy2)
    M, N = x2.shape
    gamma = _vec(gamma, N, "gamma", x2.device)
    pdtype = gamma.dtype if gamma is not None else (param_dtype or torch.float32)
    mean = _vec(mean, M, "mean", x2.device) if mean is not None else None
    rstd = _vec(rstd, M, "rstd", x2.device) if rstd is not None else None
    for t, nm in ((mean, "mean"), (rstd, "rstd")):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    dx = _out_rows(dx, x2, "dx")
    want_g = need_param_grads if need_dgamma is None else need_dgamma
    want_b = need_param_grads if need_dbeta is None else need_dbeta
    dg = _out_vec(dgamma, N, pdtype, x2.device, "dgamma") if want_g else None
    db = _out_vec(dbeta, N, pdtype, x2.device, "dbeta") if want_b else None
    with torch.cuda.device(x2.device):
        ws = _workspace("layernorm", M, N, x2.dtype, x2.device, workspace) if (want_g or want_b) else None
        _lib.check(lib, "layernorm_bwd", lib.layernorm_bwd(M, N, _ptr(x2), _ptr(dy2), _dt(x2, "x"), _ptr(mean),
                                                           _ptr(rstd), _ptr(gamma), _DT[pdtype], float(eps),
                                                           _ptr(dx), _ptr(dg), _ptr(db), _ptr(ws), _ws_bytes(ws),
                                                           _stream(x2.device)))
    return dx.reshape(x.shape), dg, db


# -------------------------------------------------------------------------------- RMSNorm

RMS_FORMS = {"cast_then_weight": 0, "weight_then_cast": 1, "one_plus_weight": 2}


def _form(form: str) -> int:
    if form not in RMS_FORMS:
        raise ValueError(f"unknown RMSNorm form {form!r} (one of {sorted(RMS_FORMS)})")
    return RMS_FORMS[form]


def rmsnorm_fwd(x: torch.Tensor, weight: torch.Tensor, eps: float, want_stats: bool = True,
                form: str = "cast_then_weight", *, y: Optional[torch.Tensor] = None,
                rstd: Optional[torch.Tensor] = None):
    """Returns (y, rstd [M] float32 or None); y keeps x's dtype.  form: "cast_then_weight"
    (Llama), "weight_then_cast" or "one_plus_weight" (Gemma).  y=, rstd=: buffers to write."""
    lib = _L()
    x2 = _as_2d(x, "x")
    M, N = x2.shape
    weight = _vec(weight, N, "weight", x2.device)
    y = _out_rows(y, x2, "y")
    rstd = _out_vec(rstd, M, torch.float32, x2.device, "rstd") if want_stats else None
    with torch.cuda.device(x2.device):
        _lib.check(lib, "rmsnorm_fwd_form", lib.rmsnorm_fwd_form(M, N, _ptr(x2), _dt(x2, "x"), _ptr(weight),
                                                                 _dt(weight, "weight"), float(eps), _form(form),
                                                                 _ptr(y), _ptr(rstd), _stream(x2.device)))
    return y.reshape(x.shape), rstd


def rmsnorm_bwd(x: torch.Tensor, dy: torch.Tensor, rstd: Optional[torch.Tensor], weight: torch.Tensor, eps: float,
                need_param_grads: bool = True, form: str = "cast_then_weight", *,
                dx: Optional[torch.Tensor] = None, dweight: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None):
    """Returns (dx, dweight).  rstd None: recomputed from x.  dx=, dweight=, workspace=: buffers
    to use instead of fresh tensors."""
    lib = _L()
    x2, dy2 = _as_2d(x, "x"), _as_2d(dy, "dy")
    if dy2.shape != x2.shape or dy2.dtype != x2.dtype:
        raise ValueError("dy must match x in shape and dtype")
    x2, dy2 = _pair(x2, dy2)
    M, N = x2.shape
    weight = _vec(weight, N, "weight", x2.device)
    rstd = _vec(rstd, M, "rstd", x2.device) if rstd is not None else None
    if rstd is not None and rstd.dtype != torch.float32:
        raise TypeError("rstd must be float32")
    dx = _out_rows(dx, x2, "dx")
    dw = _out_vec(dweight, N, weight.dtype, x2.device, "dweight") if need_param_grads else None
    with torch.cuda.device(x2.device):
        ws = _workspace("rmsnorm", M, N, x2.dtype, x2.device, workspace) if need_param_grads else None
        _lib.check(lib, "rmsnorm_bwd_form", lib.rmsnorm_bwd_form(M, N, _ptr(x2), _ptr(dy2), _dt(x2, "x"), _ptr(rstd),
                                                                 _ptr(weight), _dt(weight, "weight"), float(eps),
                                                                 _form(form), _ptr(dx), _ptr(dw), _ptr(ws),
                                                                 _ws_bytes(ws), _stream(x2.device)))
    return dx.reshape(x.shape), dw


# -------------------------------------------------------------------------------- support

def version() -> str:
    return _L().rwn_version().decode()


def trace_begin(capacity: int = 4096) -> None:
    """Start bracketing every kernel the entry points launch (on this thread) with HIP events."""
    lib = _L()
    _lib.check(lib, "rwn_trace_begin", lib.rwn_trace_begin(int(capacity)))


def trace_end(capacity: int = 4096):
    """Wait for the traced kernels; returns [(kernel name, milliseconds), ...] in launch order."""
    lib = _L()
    ms = (ctypes.c_float * capacity)()
    tags = (ctypes.c_int * capacity)()
    n = lib.rwn_trace_end(ms, tags, capacity)
    if n < 0:
        raise RwnError("rwn_trace_end", 4, (lib.rwn_last_error() or b"").decode())
    return [(_lib.KERNEL_TAGS.get(tags[i], str(tags[i])), float(ms[i])) for i in range(n)]


def stream_probe(src: torch.Tensor, dst: torch.Tensor, src2: Optional[torch.Tensor] = None, unroll: int = 4,
                 nontemporal: bool = True, wg_per_cu: int = 8) -> None:
    """dst[:] = src (or src XOR src2) with the library's streaming probe kernel (a bandwidth
    measurement aid; every tensor's bytes are copied as opaque 16-byte chunks)."""
    lib = _L()
    n = src.numel() * src.element_size()
    for t in (dst, src2):
        if t is not None and t.numel() * t.element_size() != n:
            raise ValueError("stream_probe: sizes differ")
    with torch.cuda.device(src.device):
        _lib.check(lib, "rwn_stream_probe", lib.rwn_stream_probe(src.data_ptr(), _ptr(src2), dst.data_ptr(), n,
                                                                 int(unroll), int(bool(nontemporal)), int(wg_per_cu),
                                                                 _stream(src.device)))


def plan(layer: str, backward: bool, M: int, N: int, dtype: torch.dtype, misalign_bytes: int = 0,
         cus: int = 0, param_dtype: Optional[torch.dtype] = None):
    """The launch plan the library picks.  cus = 0 plans for the current device, as the entry
    points do; any other value plans for that many compute units without touching a device."""
    lib = _L()
    out = (ctypes.c_int64 * 16)()
    li = {"dyt": 0, "layernorm": 1, "rmsnorm": 2}[layer]
    pd = -1 if param_dtype is None else _DT[param_dtype]
    _lib.check(lib, "rwn_plan", lib.rwn_plan(li, int(backward), M, N, _DT[dtype], pd, misalign_bytes, cus, out))
    keys = ("mode", "cpt", "rt", "tpr", "rpp", "block", "grid", "ntiles", "vec", "kt", "strided", "ncb", "xcd_remap",
            "prefetch", "flat", "split")
    return dict(zip(keys, [int(v) for v in out]))
