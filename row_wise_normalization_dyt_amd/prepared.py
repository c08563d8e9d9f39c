"""A forward + backward of one layer on fixed tensors, with every output, statistic and the
workspace allocated once, so repeated steps are just two C-ABI calls (no per-call torch
allocation or Python-side checks).  Used to time steps; results match the plain entry points.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _lib, _like, _DT, _form, workspace_size


class PreparedStep:
    def __init__(self, layer: str, inputs: Dict[str, torch.Tensor], eps: float = 0.0,
                 stream: Optional[torch.cuda.Stream] = None, form: str = "cast_then_weight",
                 param_grads: bool = True):
        self.layer = layer
        self.lib = lib = _lib.load()
        x, dy = inputs["x"], inputs["dy"]
        assert x.is_cuda and x.dim() == 2 and x.is_contiguous() and dy.shape == x.shape
        M, N = x.shape
        dev = x.device
        self.stream = (stream or torch.cuda.current_stream(dev)).cuda_stream
        xdt = _DT[x.dtype]
        self.y, self.dx = _like(x), _like(x)
        # Without parameter gradients the backward computes dx only and takes no workspace.
        ws_bytes = workspace_size(layer, M, N, x.dtype, dev) if param_grads else 0
        self.ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if param_grads else None
        self.inputs = inputs
        p = lambda t: None if t is None else t.data_ptr()
        wsn = self.ws.numel() if param_grads else 0
        gp = lambda name: p(self.grads[name]) if param_grads else None   # NULL: gradient not wanted
        s = self.stream
        if layer == "dyt":
            a, g, b = inputs["alpha"], inputs["gamma"], inputs["beta"]
            pdt = _DT[g.dtype]
            self.grads = {"dalpha": torch.empty(1, dtype=g.dtype, device=dev),
                          "dgamma": torch.empty(N, dtype=g.dtype, device=dev),
                          "dbeta": torch.empty(N, dtype=g.dtype, device=dev)}
            self._f, self._fa = lib.dyt_fwd, (M, N, p(x), xdt, p(a), p(g), p(b), pdt, p(self.y), s)
            self._b, self._ba = lib.dyt_bwd, (M, N, p(x), p(dy), xdt, p(a), p(g), pdt, p(self.dx),
                                              gp("dalpha"), gp("dgamma"),
                                              gp("dbeta"), p(self.ws), wsn, s)
        elif layer == "layernorm":
            g, b = inputs.get("gamma"), inputs.get("beta")
            pdt = _DT[g.dtype] if g is not None else _lib.RWN_F32
            pt = g.dtype if g is not None else torch.float32
            self.mean = torch.empty(M, dtype=torch.float32, device=dev)
            self.rstd = torch.empty(M, dtype=torch.float32, device=dev)
            self.grads = {"dgamma": torch.empty(N, dtype=pt, device=dev),
                          "dbeta": torch.empty(N, dtype=pt, device=dev)}
            self._f, self._fa = lib.layernorm_fwd, (M, N, p(x), xdt, p(g), p(b), pdt, float(eps), p(self.y),
                                                    p(self.mean), p(self.rstd), s)
            self._b, self._ba = lib.layernorm_bwd, (M, N, p(x), p(dy), xdt, p(self.mean), p(self.rstd), p(g), pdt,
                                                    float(eps), p(self.dx), gp("dgamma"),
                                                    gp("dbeta"), p(self.ws), wsn, s)
        elif layer == "rmsnorm":
            w = inputs["weight"]
            wdt = _DT[w.dtype]
            self.rstd = torch.empty(M, dtype=torch.float32, device=dev)
            self.grads = {"dweight": torch.empty(N, dtype=w.dtype, device=dev)}
            f = _form(form)
            self._f, self._fa = lib.rmsnorm_fwd_form, (M, N, p(x), xdt, p(w), wdt, float(eps), f, p(self.y),
                                                       p(self.rstd), s)
            self._b, self._ba = lib.rmsnorm_bwd_form, (M, N, p(x), p(dy), xdt, p(self.rstd), p(w), wdt, float(eps), f,
                                                       p(self.dx), gp("dweight"), p(self.ws),
                                                       wsn, s)
        else:
            raise ValueError(layer)
        if not param_grads:
            self.grads = {}

    def fwd(self) -> None:
        rc = self._f(*self._fa)
        if rc:
            _lib.check(self.lib, f"{self.layer}_fwd", rc)

    def bwd(self) -> None:
        rc = self._b(*self._ba)
        if rc:
            _lib.check(self.lib, f"{self.layer}_bwd", rc)

    def step(self) -> None:
        self.fwd()
        self.bwd()

    def outputs(self) -> Dict[str, torch.Tensor]:
        out = {"y": self.y, "dx": self.dx, **self.grads}
        if self.layer == "layernorm":
            out.update(mean=self.mean, rstd=self.rstd)
        if self.layer == "rmsnorm":
            out["rstd"] = self.rstd
        return out
