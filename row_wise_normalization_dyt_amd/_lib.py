"""ctypes declarations of librwnorm's C ABI (include/rwnorm.h).

Loading never falls back to anything: if the shared library is missing or a symbol is absent
the import of the binding raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "librwnorm.so")
HEADER = os.path.join(ROOT, "include", "rwnorm.h")

RWN_F32, RWN_BF16, RWN_F16 = 0, 1, 2
STATUS = {0: "RWN_OK", 1: "RWN_ERR_INVALID_ARG", 2: "RWN_ERR_UNSUPPORTED", 3: "RWN_ERR_WORKSPACE",
          4: "RWN_ERR_LAUNCH"}
KERNEL_TAGS = {1: "dyt_fwd", 2: "dyt_bwd", 3: "layernorm_fwd", 4: "layernorm_bwd", 5: "rmsnorm_fwd",
               6: "rmsnorm_bwd", 7: "colreduce", 8: "stream_probe"}

_i64, _vp, _ci, _cf, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_fp = ctypes.c_void_p   # float* (device)
_ip = ctypes.POINTER(ctypes.c_int64)   # const int64_t* (host array)

SIGNATURES = {
    "dyt_fwd": (_ci, [_i64, _i64, _vp, _ci, _vp, _vp, _vp, _ci, _vp, _vp]),
    "dyt_bwd": (_ci, [_i64, _i64, _vp, _vp, _ci, _vp, _vp, _ci, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dyt_bwd_workspace_size": (_ci, [_i64, _i64, _ci, ctypes.POINTER(_sz)]),
    "layernorm_fwd": (_ci, [_i64, _i64, _vp, _ci, _vp, _vp, _ci, _cf, _vp, _fp, _fp, _vp]),
    "layernorm_bwd": (_ci, [_i64, _i64, _vp, _vp, _ci, _fp, _fp, _vp, _ci, _cf, _vp, _vp, _vp, _vp, _sz, _vp]),
    "layernorm_bwd_workspace_size": (_ci, [_i64, _i64, _ci, ctypes.POINTER(_sz)]),
    "layernorm_bwd_noalloc": (_ci, [_i64, _i64, _vp, _vp, _ci, _fp, _fp, _vp, _ci, _cf, _vp, _vp, _vp, _vp]),
    "rmsnorm_fwd": (_ci, [_i64, _i64, _vp, _ci, _vp, _ci, _cf, _vp, _fp, _vp]),
    "rmsnorm_bwd": (_ci, [_i64, _i64, _vp, _vp, _ci, _fp, _vp, _ci, _cf, _vp, _vp, _vp, _sz, _vp]),
    "rmsnorm_bwd_workspace_size": (_ci, [_i64, _i64, _ci, ctypes.POINTER(_sz)]),
    "rmsnorm_fwd_form": (_ci, [_i64, _i64, _vp, _ci, _vp, _ci, _cf, _ci, _vp, _fp, _vp]),
    "rmsnorm_bwd_form": (_ci, [_i64, _i64, _vp, _vp, _ci, _fp, _vp, _ci, _cf, _ci, _vp, _vp, _vp, _sz, _vp]),
    "dyt_fwd_strided": (_ci, [_ci, _ip, _i64, _vp, _ip, _ci, _vp, _vp, _i64, _vp, _i64, _ci, _vp, _ip, _vp]),
    "dyt_bwd_strided": (_ci, [_ci, _ip, _i64, _vp, _ip, _vp, _ip, _ci, _vp, _vp, _i64, _ci, _vp, _ip, _vp, _vp, _vp,
                              _vp, _sz, _vp]),
    "layernorm_fwd_strided": (_ci, [_ci, _ip, _i64, _vp, _ip, _ci, _vp, _i64, _vp, _i64, _ci, _cf, _vp, _ip, _fp, _fp,
                                    _vp]),
    "layernorm_bwd_strided": (_ci, [_ci, _ip, _i64, _vp, _ip, _vp, _ip, _ci, _fp, _fp, _vp, _i64, _ci, _cf, _vp, _ip,
                                    _vp, _vp, _vp, _sz, _vp]),
    "rmsnorm_fwd_strided": (_ci, [_ci, _ip, _i64, _vp, _ip, _ci, _vp, _i64, _ci, _cf, _ci, _vp, _ip, _fp, _vp]),
    "rmsnorm_bwd_strided": (_ci, [_ci, _ip, _i64, _vp, _ip, _vp, _ip, _ci, _fp, _vp, _i64, _ci, _cf, _ci, _vp, _ip,
                                  _vp, _vp, _sz, _vp]),
    "rwn_last_error": (ctypes.c_char_p, []),
    "rwn_version": (ctypes.c_char_p, []),
    "rwn_trace_begin": (_ci, [_ci]),
    "rwn_trace_end": (_ci, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int), _ci]),
    "rwn_stream_probe": (_ci, [_vp, _vp, _vp, _sz, _ci, _ci, _ci, _vp]),
    "rwn_plan": (_ci, [_ci, _ci, _i64, _i64, _ci, _ci, _ci, _ci, _ci, ctypes.POINTER(_i64)]),
}


def declared_functions(header: str = HEADER) -> List[str]:
    """Names of the functions include/rwnorm.h declares."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:rwn_status|const char\s*\*|int|size_t)\s+(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


class RwnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS.get(code, code)}: {msg}")
        self.code = code


_LIB = None


def load(path: str = LIB_PATH):
    """Load librwnorm.so and bind every declared function (raises if anything is missing)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)   # AttributeError if the symbol is missing
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _LIB = lib
    return lib


def check(lib, fn: str, code: int) -> None:
    if code != 0:
        raise RwnError(fn, code, (lib.rwn_last_error() or b"").decode())
