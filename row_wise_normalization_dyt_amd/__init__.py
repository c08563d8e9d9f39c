"""Row-wise normalization for MI355X (gfx950): DyT, LayerNorm and RMSNorm, forward and backward.

Thin binding over librwnorm's C ABI (include/rwnorm.h), with the same entry-point names.  It
only marshals arguments: shapes and dtypes are checked, contiguous inputs flattened to [M, N],
non-contiguous ones handed to the strided entry points with their strides, outputs and the
backward workspace allocated with torch, and the call enqueued on the current stream of the
tensors' device.  Every step of the computation
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


def _rows12(N: int, esz: int) -> bool:
    """LayerNorm rows of 12 * 2^k bytes (2^k <= 64 lanes): the library moves them in 12-byte
    chunks, which need only 4-byte alignment."""
    b = N * esz
    lanes = b // 12
    return b % 12 == 0 and 1 <= lanes <= 64 and lanes & (lanes - 1) == 0


def _as_2d(x: torch.Tensor, name: str, rows12: bool = False) -> torch.Tensor:
    """x as a contiguous [M, N] matrix.  rows12: the caller's rows are LayerNorm rows the
    library takes in 12-byte chunks, so a view 4, 8 or 12 bytes past a 16-byte boundary is kept."""
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if x.dim() < 1:
        raise ValueError(f"{name} must have at least one dimension")
    x = x.contiguous()
    x = x.reshape(-1, x.shape[-1]) if x.dim() != 2 else x
    keep = rows12 and x.data_ptr() % 4 == 0 and _rows12(x.shape[-1], x.element_size())
    if x.data_ptr() % 16 and x.shape[-1] % (16 // x.element_size()) == 0 and not keep:
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


# ------------------------------------------------------------------------- strided operands
#
# A non-contiguous x or dy (a slice of a wider matrix, a head-major view, a transposed incoming
# gradient) or a non-contiguous parameter vector goes to the *_strided entry points as it is:
# the leading dimensions are handed over with each tensor's own strides (size-1 dimensions
# dropped, neighbours merged where every tensor allows), and nothing is copied.  Only a last
# dimension that is not contiguous, more than three leading dimensions that do not merge, or
# a shape the strided kernels do not take (rows of different alignment wider than the
# element-wise kernels' limit) fall back to contiguous copies.  Fresh outputs are contiguous.

def _rows_view(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() < 1:
        raise ValueError(f"{name} must have at least one dimension")
    return t if (t.shape[-1] == 1 or t.stride(-1) == 1) else t.contiguous()


def _use_strided(rows, params) -> bool:
    if any(not t.is_cuda or t.dim() < 1 or t.numel() == 0 for t in rows):
        return False
    if any(t.shape[-1] > 1 and t.stride(-1) != 1 for t in rows):
        return False
    return any(not t.is_contiguous() for t in rows) or \
        any(p is not None and p.numel() > 1 and not p.is_contiguous() for p in params)


def _fresh_rows(x: torch.Tensor) -> torch.Tensor:
    """A contiguous tensor of x's shape and dtype at x's address modulo 16 bytes."""
    esz = x.element_size()
    if x.data_ptr() % 16 == 0:
        return torch.empty(x.shape, dtype=x.dtype, device=x.device)
    buf = torch.empty(x.numel() + 16 // esz, dtype=x.dtype, device=x.device)
    shift = ((x.data_ptr() - buf.data_ptr()) % 16) // esz
    return buf[shift:shift + x.numel()].view(x.shape)


def _out_strided(given: Optional[torch.Tensor], x: torch.Tensor, name: str) -> torch.Tensor:
    if given is None:
        return _fresh_rows(x)
    if given.device != x.device or given.dtype != x.dtype or given.shape != x.shape:
        raise ValueError(f"{name} must be a {x.dtype} tensor of shape {tuple(x.shape)} on {x.device}")
    if x.shape[-1] > 1 and given.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return given


def _svec(p: Optional[torch.Tensor], n: int, name: str, dev):
    """(1-D view of a parameter vector, its element stride); no copy where a view exists."""
    if p is None:
        return None, 1
    if p.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if p.numel() != n:
        raise ValueError(f"{name} must have {n} elements (got {p.numel()})")
    v = p.reshape(-1)
    return v, (v.stride(0) if n > 1 else 1)


def _row_layout(ts):
    """(nlead, lead sizes, [strides of each tensor]) as ctypes arrays for tensors of one shape
    [..., N], or None when more than three leading dimensions remain after merging."""
    dims = []
    for i, size in enumerate(ts[0].shape[:-1]):
        if size == 1:
            continue
        st = [t.stride(i) for t in ts]
        if dims and all(ps == s * size for ps, s in zip(dims[-1][1], st)):
            dims[-1] = (dims[-1][0] * size, st)
        else:
            dims.append((size, st))
    if not dims:
        dims = [(1, [0] * len(ts))]
    if len(dims) > 3:
        return None
    n = len(dims)
    lead = (ctypes.c_int64 * n)(*[d[0] for d in dims])
    strides = [(ctypes.c_int64 * n)(*[d[1][k] for d in dims]) for k in range(len(ts))]
    return n, lead, strides


def _try_strided(lib, fn: str, call) -> bool:
    """Runs call(); False (nothing launched) when the strided kernels do not take the shape."""
    code = call()
    if code == 2:   # RWN_ERR_UNSUPPORTED: validated before any launch
        return False
    _lib.check(lib, fn, code)
    return True


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
    if _use_strided([x], [gamma, beta]):
        xs = _rows_view(x, "x")
        N = xs.shape[-1]
        a = _vec(alpha, 1, "alpha", xs.device)
        (g, gs), (b, bs) = _svec(gamma, N, "gamma", xs.device), _svec(beta, N, "beta", xs.device)
        ys = _out_strided(y, xs, "y")
        lay = _row_layout([xs, ys])
        if lay is not None:
            n, lead, (sx, sy) = lay
            with torch.cuda.device(xs.device):
                if _try_strided(lib, "dyt_fwd_strided", lambda: lib.dyt_fwd_strided(
                        n, lead, N, _ptr(xs), sx, _dt(xs, "x"), _ptr(a), _ptr(g), gs, _ptr(b), bs,
                        _param_dtype(a, g, b), _ptr(ys), sy, _stream(xs.device))):
                    return ys
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
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    if _use_strided([x, dy], [gamma]):
        xs, dys = _rows_view(x, "x"), _rows_view(dy, "dy")
        N = xs.shape[-1]
        a = _vec(alpha, 1, "alpha", xs.device)
        g, gs = _svec(gamma, N, "gamma", xs.device)
        dxs = _out_strided(dx, xs, "dx")
        lay = _row_layout([xs, dys, dxs])
        if lay is not None:
            n, lead, (sx, sdy, sdx) = lay
            M = xs.numel() // N
            da = _out_vec(dalpha, 1, g.dtype, xs.device, "dalpha") if need_param_grads else None
            dg = _out_vec(dgamma, N, g.dtype, xs.device, "dgamma") if need_param_grads else None
            db = _out_vec(dbeta, N, g.dtype, xs.device, "dbeta") if need_param_grads else None
            with torch.cuda.device(xs.device):
                ws = _workspace("dyt", M, N, xs.dtype, xs.device, workspace) if need_param_grads else None
                if _try_strided(lib, "dyt_bwd_strided", lambda: lib.dyt_bwd_strided(
                        n, lead, N, _ptr(xs), sx, _ptr(dys), sdy, _dt(xs, "x"), _ptr(a), _ptr(g), gs,
                        _param_dtype(a, g), _ptr(dxs), sdx, _ptr(da), _ptr(dg), _ptr(db), _ptr(ws), _ws_bytes(ws),
                        _stream(xs.device))):
                    return dxs, da, dg, db
    x2, dy2 = _as_2d(x, "x"), _as_2d(dy, "dy")
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
    if _use_strided([x], [gamma, beta]):
        xs = _rows_view(x, "x")
        N = xs.shape[-1]
        M = xs.numel() // N
        (g, gs), (b, bs) = _svec(gamma, N, "gamma", xs.device), _svec(beta, N, "beta", xs.device)
        pd = _param_dtype(g, b) if (g is not None or b is not None) else _lib.RWN_F32
        ys = _out_strided(y, xs, "y")
        lay = _row_layout([xs, ys])
        if lay is not None:
            n, lead, (sx, sy) = lay
            mu = _out_vec(mean, M, torch.float32, xs.device, "mean") if want_stats else None
            rs = _out_vec(rstd, M, torch.float32, xs.device, "rstd") if want_stats else None
            with torch.cuda.device(xs.device):
                if _try_strided(lib, "layernorm_fwd_strided", lambda: lib.layernorm_fwd_strided(
                        n, lead, N, _ptr(xs), sx, _dt(xs, "x"), _ptr(g), gs, _ptr(b), bs, pd, float(eps), _ptr(ys),
                        sy, _ptr(mu), _ptr(rs), _stream(xs.device))):
                    return ys, mu, rs
    x2 = _as_2d(x, "x", rows12=True)
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
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    want_g = need_param_grads if need_dgamma is None else need_dgamma
    want_b = need_param_grads if need_dbeta is None else need_dbeta
    for t, nm in ((mean, "mean"), (rstd, "rstd")):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    if _use_strided([x, dy], [gamma]):
        xs, dys = _rows_view(x, "x"), _rows_view(dy, "dy")
        N = xs.shape[-1]
        M = xs.numel() // N
        g, gs = _svec(gamma, N, "gamma", xs.device)
        pdtype = g.dtype if g is not None else (param_dtype or torch.float32)
        dxs = _out_strided(dx, xs, "dx")
        lay = _row_layout([xs, dys, dxs])
        if lay is not None:
            n, lead, (sx, sdy, sdx) = lay
            mu = _vec(mean, M, "mean", xs.device) if mean is not None else None
            rs = _vec(rstd, M, "rstd", xs.device) if rstd is not None else None
            dg = _out_vec(dgamma, N, pdtype, xs.device, "dgamma") if want_g else None
            db = _out_vec(dbeta, N, pdtype, xs.device, "dbeta") if want_b else None
            with torch.cuda.device(xs.device):
                ws = _workspace("layernorm", M, N, xs.dtype, xs.device, workspace) if (want_g or want_b) else None
                if _try_strided(lib, "layernorm_bwd_strided", lambda: lib.layernorm_bwd_strided(
                        n, lead, N, _ptr(xs), sx, _ptr(dys), sdy, _dt(xs, "x"), _ptr(mu), _ptr(rs), _ptr(g), gs,
                        _DT[pdtype], float(eps), _ptr(dxs), sdx, _ptr(dg), _ptr(db), _ptr(ws), _ws_bytes(ws),
                        _stream(xs.device))):
                    return dxs, dg, db
    x2, dy2 = _as_2d(x, "x", rows12=True), _as_2d(dy, "dy", rows12=True)
    x2, dy2 = _pair(x2, dy2)
    M, N = x2.shape
    gamma = _vec(gamma, N, "gamma", x2.device)
    pdtype = gamma.dtype if gamma is not None else (param_dtype or torch.float32)
    mean = _vec(mean, M, "mean", x2.device) if mean is not None else None
    rstd = _vec(rstd, M, "rstd", x2.device) if rstd is not None else None
    dx = _out_rows(dx, x2, "dx")
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
    if _use_strided([x], [weight]):
        xs = _rows_view(x, "x")
        N = xs.shape[-1]
        M = xs.numel() // N
        w, ws_ = _svec(weight, N, "weight", xs.device)
        ys = _out_strided(y, xs, "y")
        lay = _row_layout([xs, ys])
        if lay is not None:
            n, lead, (sx, sy) = lay
            rs = _out_vec(rstd, M, torch.float32, xs.device, "rstd") if want_stats else None
            with torch.cuda.device(xs.device):
                if _try_strided(lib, "rmsnorm_fwd_strided", lambda: lib.rmsnorm_fwd_strided(
                        n, lead, N, _ptr(xs), sx, _dt(xs, "x"), _ptr(w), ws_, _dt(w, "weight"), float(eps),
                        _form(form), _ptr(ys), sy, _ptr(rs), _stream(xs.device))):
                    return ys, rs
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
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    if rstd is not None and rstd.dtype != torch.float32:
        raise TypeError("rstd must be float32")
    if _use_strided([x, dy], [weight]):
        xs, dys = _rows_view(x, "x"), _rows_view(dy, "dy")
        N = xs.shape[-1]
        M = xs.numel() // N
        w, ws_ = _svec(weight, N, "weight", xs.device)
        dxs = _out_strided(dx, xs, "dx")
        lay = _row_layout([xs, dys, dxs])
        if lay is not None:
            n, lead, (sx, sdy, sdx) = lay
            rs = _vec(rstd, M, "rstd", xs.device) if rstd is not None else None
            dw = _out_vec(dweight, N, w.dtype, xs.device, "dweight") if need_param_grads else None
            with torch.cuda.device(xs.device):
                wsp = _workspace("rmsnorm", M, N, xs.dtype, xs.device, workspace) if need_param_grads else None
                if _try_strided(lib, "rmsnorm_bwd_strided", lambda: lib.rmsnorm_bwd_strided(
                        n, lead, N, _ptr(xs), sx, _ptr(dys), sdy, _dt(xs, "x"), _ptr(rs), _ptr(w), ws_,
                        _dt(w, "weight"), float(eps), _form(form), _ptr(dxs), sdx, _ptr(dw), _ptr(wsp),
                        _ws_bytes(wsp), _stream(xs.device))):
                    return dxs, dw
    x2, dy2 = _as_2d(x, "x"), _as_2d(dy, "dy")
    x2, dy2 = _pair(x2, dy2)
    M, N = x2.shape
    weight = _vec(weight, N, "weight", x2.device)
    rstd = _vec(rstd, M, "rstd", x2.device) if rstd is not None else None
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
         cus: int = 0, param_dtype: Optional[torch.dtype] = None, layout: int = 0):
    """The launch plan the library picks.  cus = 0 plans for the current device, as the entry
    points do; any other value plans for that many compute units without touching a device."""
    lib = _L()
    out = (ctypes.c_int64 * 16)()
    li = {"dyt": 0, "layernorm": 1, "rmsnorm": 2}[layer]
    pd = -1 if param_dtype is None else _DT[param_dtype]
    _lib.check(lib, "rwn_plan", lib.rwn_plan(li, int(backward), M, N, _DT[dtype], pd, misalign_bytes, cus,
                                             int(layout), out))
    keys = ("mode", "cpt", "rt", "tpr", "rpp", "block", "grid", "ntiles", "vec", "kt", "strided", "ncb", "xcd_remap",
            "prefetch", "flat", "split")
    return dict(zip(keys, [int(v) for v in out]))
