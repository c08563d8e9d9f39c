"""CPU oracle for DyT, LayerNorm and RMSNorm forward/backward (fp64, plain C, OpenMP).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg are the only code that may import this package.  The GPU library never
calls it and shares no code with it.

Every function takes host tensors (torch CPU tensors of dtype float32, bfloat16 or float16, row-major
[M, N]) and returns a dict of float64 numpy arrays holding the exact values before the final
cast to the output dtype, plus the per-element or per-column magnitude sums ("*_scale") that
bound fp32 rounding error.  See ``oracle.c`` for the definition of each quantity and the
passages of the pages it follows.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64, F16 = 0, 1, 2, 3
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float64: F64, torch.float16: F16}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE double arithmetic: no fast-math,
    no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_variant(src_text: str, out_path: str) -> str:
    """Compile another version of oracle.c (the tests that plant a mistake in the oracle use
    this to check that the pins catch it)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-shared", "-fPIC", src, "-o", out_path, "-lm"], check=True)
    return out_path


@contextlib.contextmanager
def using_library(path: str):
    """Within the block, every oracle function calls the library at ``path``."""
    global _lib
    saved = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # ORACLE_LIBRARY points the pins at another build of oracle.c (the mutation tests).
    path = os.environ.get("ORACLE_LIBRARY") or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build()
    _lib = _bind(ctypes.CDLL(path))
    return _lib


def _bind(lib):
    i64, vp, ci, cd = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    dp = ctypes.c_void_p
    lib.oracle_dyt_fwd.argtypes = [i64, i64, vp, ci, cd, vp, vp, ci, dp, dp]
    lib.oracle_dyt_bwd.argtypes = [i64, i64, vp, vp, ci, cd, vp, ci, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_layernorm_fwd.argtypes = [i64, i64, vp, ci, vp, vp, ci, cd, dp, dp, dp, dp, dp, dp]
    lib.oracle_layernorm_bwd.argtypes = [i64, i64, vp, vp, ci, vp, ci, cd, dp, dp, dp, dp, dp, dp]
    lib.oracle_rmsnorm_fwd.argtypes = [i64, i64, vp, ci, vp, ci, cd, dp, dp, dp, dp]
    lib.oracle_rmsnorm_bwd.argtypes = [i64, i64, vp, vp, ci, vp, ci, cd, dp, dp, dp, dp, dp]
    lib.oracle_rmsnorm_fwd_form.argtypes = [i64, i64, vp, ci, vp, ci, cd, ci, dp, dp, dp, dp]
    lib.oracle_rmsnorm_bwd_form.argtypes = [i64, i64, vp, vp, ci, vp, ci, cd, ci, dp, dp, dp, dp, dp]
    for f in ("oracle_dyt_fwd", "oracle_dyt_bwd", "oracle_layernorm_fwd", "oracle_layernorm_bwd",
              "oracle_rmsnorm_fwd", "oracle_rmsnorm_bwd", "oracle_rmsnorm_fwd_form", "oracle_rmsnorm_bwd_form"):
        getattr(lib, f).restype = ci
    lib.oracle_round_bf16.argtypes = [cd]
    lib.oracle_round_bf16.restype = cd
    lib.oracle_round_f32.argtypes = [cd]
    lib.oracle_round_f32.restype = cd
    lib.oracle_round_f16.argtypes = [cd]
    lib.oracle_round_f16.restype = cd
    lib.oracle_round_array.argtypes = [dp, dp, i64, ci]
    lib.oracle_round_array.restype = None
    lib.oracle_load_array.argtypes = [vp, ci, i64, dp]
    lib.oracle_load_array.restype = None
    return lib


def set_threads(n: Optional[int]) -> None:
    """Set the OpenMP thread count the oracle uses (None: leave the runtime default)."""
    if n is None:
        return
    gomp = ctypes.CDLL("libgomp.so.1")
    gomp.omp_set_num_threads(ctypes.c_int(int(n)))


def max_threads() -> int:
    gomp = ctypes.CDLL("libgomp.so.1")
    gomp.omp_get_max_threads.restype = ctypes.c_int
    return int(gomp.omp_get_max_threads())


def _host(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError(f"oracle: {name} must be a host tensor")
    if t.dtype not in _DT:
        raise ValueError(f"oracle: {name} has unsupported dtype {t.dtype}")
    return t.contiguous()


def _out(shape) -> np.ndarray:
    return np.empty(shape, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _scalar(t) -> float:
    if isinstance(t, torch.Tensor):
        return float(t.detach().to(torch.float64).cpu().reshape(-1)[0])
    return float(t)


def _check(rc: int, fn: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{fn} failed with code {rc}")


def dyt_fwd(x, alpha, gamma, beta) -> Dict[str, np.ndarray]:
    lib = _load()
    x, gamma, beta = _host(x, "x"), _host(gamma, "gamma"), _host(beta, "beta")
    M, N = x.shape
    y, ys = _out((M, N)), _out((M, N))
    _check(lib.oracle_dyt_fwd(M, N, x.data_ptr(), _DT[x.dtype], _scalar(alpha), gamma.data_ptr(),
                              beta.data_ptr(), _DT[gamma.dtype], _p(y), _p(ys)), "oracle_dyt_fwd")
    return {"y": y, "y_scale": ys}


def dyt_bwd(x, dy, alpha, gamma, want_dx: bool = True) -> Dict[str, np.ndarray]:
    """Backward.  ``want_dx=False`` skips dx (the parameter gradients still use all rows)."""
    lib = _load()
    x, dy, gamma = _host(x, "x"), _host(dy, "dy"), _host(gamma, "gamma")
    M, N = x.shape
    dx = _out((M, N)) if want_dx else None
    dxs = _out((M, N)) if want_dx else None
    dg, db, dgs, dbs = _out(N), _out(N), _out(N), _out(N)
    da, das = _out(1), _out(1)
    _check(lib.oracle_dyt_bwd(M, N, x.data_ptr(), dy.data_ptr(), _DT[x.dtype], _scalar(alpha),
                              gamma.data_ptr(), _DT[gamma.dtype], _p(dx), _p(dxs), _p(dg), _p(db),
                              _p(da), _p(dgs), _p(dbs), _p(das)), "oracle_dyt_bwd")
    out = {"dgamma": dg, "dbeta": db, "dalpha": da, "dgamma_scale": dgs, "dbeta_scale": dbs,
           "dalpha_scale": das}
    if want_dx:
        out.update(dx=dx, dx_scale=dxs)
    return out


def layernorm_fwd(x, gamma, beta, eps: float) -> Dict[str, np.ndarray]:
    lib = _load()
    x, gamma, beta = _host(x, "x"), _host(gamma, "gamma"), _host(beta, "beta")
    M, N = x.shape
    y, ys, mu, rs, ms, vs = _out((M, N)), _out((M, N)), _out(M), _out(M), _out(M), _out(M)
    _check(lib.oracle_layernorm_fwd(M, N, x.data_ptr(), _DT[x.dtype], gamma.data_ptr(),
                                    beta.data_ptr(), _DT[gamma.dtype], float(eps), _p(y), _p(ys),
                                    _p(mu), _p(rs), _p(ms), _p(vs)), "oracle_layernorm_fwd")
    return {"y": y, "y_scale": ys, "mean": mu, "rstd": rs, "mean_scale": ms, "rstd_scale": vs}


def layernorm_bwd(x, dy, gamma, eps: float, want_dx: bool = True) -> Dict[str, np.ndarray]:
    lib = _load()
    x, dy, gamma = _host(x, "x"), _host(dy, "dy"), _host(gamma, "gamma")
    M, N = x.shape
    dx = _out((M, N)) if want_dx else None
    dxs = _out((M, N)) if want_dx else None
    dg, db, dgs, dbs = _out(N), _out(N), _out(N), _out(N)
    _check(lib.oracle_layernorm_bwd(M, N, x.data_ptr(), dy.data_ptr(), _DT[x.dtype],
                                    gamma.data_ptr(), _DT[gamma.dtype], float(eps), _p(dx),
                                    _p(dxs), _p(dg), _p(db), _p(dgs), _p(dbs)),
           "oracle_layernorm_bwd")
    out = {"dgamma": dg, "dbeta": db, "dgamma_scale": dgs, "dbeta_scale": dbs}
    if want_dx:
        out.update(dx=dx, dx_scale=dxs)
    return out


RMS_FORMS = {"cast_then_weight": 0, "weight_then_cast": 1, "one_plus_weight": 2}


def rmsnorm_fwd(x, weight, eps: float, form: str = "cast_then_weight") -> Dict[str, np.ndarray]:
    lib = _load()
    x, weight = _host(x, "x"), _host(weight, "weight")
    M, N = x.shape
    y, ys, ya, rs = _out((M, N)), _out((M, N)), _out((M, N)), _out(M)
    _check(lib.oracle_rmsnorm_fwd_form(M, N, x.data_ptr(), _DT[x.dtype], weight.data_ptr(),
                                       _DT[weight.dtype], float(eps), RMS_FORMS[form], _p(y), _p(ys),
                                       _p(ya), _p(rs)), "oracle_rmsnorm_fwd_form")
    return {"y": y, "y_scale": ys, "y_alt": ya, "rstd": rs}


def rmsnorm_bwd(x, dy, weight, eps: float, want_dx: bool = True,
                form: str = "cast_then_weight") -> Dict[str, np.ndarray]:
    lib = _load()
    x, dy, weight = _host(x, "x"), _host(dy, "dy"), _host(weight, "weight")
    M, N = x.shape
    dx = _out((M, N)) if want_dx else None
    dxs = _out((M, N)) if want_dx else None
    dw, dws, dwl = _out(N), _out(N), _out(N)
    _check(lib.oracle_rmsnorm_bwd_form(M, N, x.data_ptr(), dy.data_ptr(), _DT[x.dtype],
                                       weight.data_ptr(), _DT[weight.dtype], float(eps), RMS_FORMS[form],
                                       _p(dx), _p(dxs), _p(dw), _p(dws), _p(dwl)), "oracle_rmsnorm_bwd_form")
    out = {"dweight": dw, "dweight_scale": dws, "dweight_slack": dwl}
    if want_dx:
        out.update(dx=dx, dx_scale=dxs)
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    lib.oracle_round_array(v.ctypes.data, out.ctypes.data, v.size, BF16)
    return out


def round_f16(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    lib.oracle_round_array(v.ctypes.data, out.ctypes.data, v.size, F16)
    return out


def load_values(t: torch.Tensor) -> np.ndarray:
    """The float64 values the oracle reads from a host tensor's elements."""
    t = _host(t, "t")
    out = np.empty(t.numel(), dtype=np.float64)
    _load().oracle_load_array(t.data_ptr(), _DT[t.dtype], t.numel(), out.ctypes.data)
    return out.reshape(tuple(t.shape))


def round_f32(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    lib.oracle_round_array(v.ctypes.data, out.ctypes.data, v.size, F32)
    return out
