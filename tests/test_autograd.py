"""torch.autograd integration (row_wise_normalization_dyt_amd.autograd).

CPU: the opt-in module swap and the absence of any fallback.  GPU: gradients through the
autograd Functions are bitwise those of the binding's backward entry points, and match the
oracle to the parity bars of tests/tolerance.py.
"""
import pytest
import torch
from torch import nn

import row_wise_normalization_dyt_amd as rwn
from row_wise_normalization_dyt_amd import autograd as ag
import workloads
from tests import gpu_cases as gc
from tests import tolerance as tol


class _LlamaStyleRMSNorm(nn.Module):
    def __init__(self, n, eps=1e-6):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(n))
        self.variance_epsilon = eps


def _model():
    return nn.Sequential(nn.Linear(8, 8), nn.LayerNorm(8),
                         nn.Sequential(_LlamaStyleRMSNorm(8), nn.LayerNorm(8, elementwise_affine=False)),
                         nn.LayerNorm((2, 4)))


def test_swap_norms_replaces_and_shares_parameters():
    m = _model()
    ln_w = m[1].weight
    rms_w = m[2][0].weight
    assert ag.swap_norms(m) == 3
    assert isinstance(m[1], ag.LayerNorm) and m[1].weight is ln_w and m[1].eps == 1e-5
    assert isinstance(m[2][0], ag.RMSNorm) and m[2][0].weight is rms_w and m[2][0].variance_epsilon == 1e-6
    assert isinstance(m[2][1], ag.LayerNorm) and m[2][1].weight is None and m[2][1].bias is None
    assert isinstance(m[3], nn.LayerNorm)            # two normalized dimensions: left alone
    assert isinstance(m[0], nn.Linear)
    assert ag.swap_norms(m) == 0                      # idempotent


def test_no_fallback_for_host_tensors():
    with pytest.raises(ValueError, match="GPU tensor"):
        ag.DyT(8)(torch.randn(4, 8))
    with pytest.raises(ValueError, match="GPU tensor"):
        ag.LayerNorm(8)(torch.randn(4, 8))
    with pytest.raises(ValueError, match="GPU tensor"):
        ag.RMSNorm(8)(torch.randn(4, 8))


def _params(layer, wl, inp, dev):
    if layer == "dyt":
        return [inp["alpha"], inp["gamma"], inp["beta"]]
    if layer == "layernorm":
        return [inp["gamma"], inp["beta"]]
    return [inp["weight"]]


@pytest.mark.gpu
@pytest.mark.parametrize("xdt,pdt", [("f32", "f32"), ("bf16", "f32"), ("f16", "f16")])
@pytest.mark.parametrize("layer", ["dyt", "layernorm", "rmsnorm"])
def test_autograd_matches_entry_points_and_oracle(layer, xdt, pdt):
    M, N = 2 * 515, 1025 if layer == "layernorm" else 256
    wl = workloads.small(layer, M, N, xdt, pdt, seed=17)
    print("case:", wl, flush=True)
    inp = workloads.make_inputs(wl)
    dev = {k: v.to("cuda") for k, v in inp.items()}
    x = dev["x"].reshape(2, M // 2, N).clone().requires_grad_(True)
    ps = [p.clone().requires_grad_(True) for p in _params(layer, wl, dev, "cuda")]
    if layer == "dyt":
        y = ag.dyt(x, *ps)
    elif layer == "layernorm":
        y = ag.layer_norm(x, *ps, eps=wl.eps)
    else:
        y = ag.rms_norm(x, *ps, eps=wl.eps)
    y.backward(dev["dy"].reshape(2, M // 2, N))
    torch.cuda.synchronize()
    ref = gc.gpu_run(layer, dev, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(y.detach().reshape(M, N), ref["y"])
    assert torch.equal(x.grad.reshape(M, N), ref["dx"])
    names = {"dyt": ["dalpha", "dgamma", "dbeta"], "layernorm": ["dgamma", "dbeta"], "rmsnorm": ["dweight"]}[layer]
    for p, nm in zip(ps, names):
        assert p.grad.dtype == p.dtype and torch.equal(p.grad.reshape(-1), ref[nm].reshape(-1)), nm
    got = {"y": y.detach().reshape(M, N), "dx": x.grad.reshape(M, N)}
    got.update({nm: p.grad for p, nm in zip(ps, names)})
    o = gc.oracle_run(layer, inp, wl.eps)
    tol.assert_reports(gc.compare(layer, got, o, gc.DT[xdt], gc.DT[pdt]))


@pytest.mark.gpu
def test_autograd_skips_parameter_gradients_not_asked_for():
    wl = workloads.small("layernorm", 300, 512, "bf16", "f32", seed=3)
    inp = {k: v.to("cuda") for k, v in workloads.make_inputs(wl).items()}
    x = inp["x"].clone().requires_grad_(True)
    y = ag.layer_norm(x, inp["gamma"], inp["beta"], wl.eps)     # parameters without grad
    (g,) = torch.autograd.grad(y, x, inp["dy"])
    ref = gc.gpu_run("layernorm", inp, wl.eps)
    assert torch.equal(g, ref["dx"])
    with pytest.raises(RuntimeError):
        # first-order only: a double backward raises
        x2 = inp["x"].clone().requires_grad_(True)
        y2 = ag.layer_norm(x2, inp["gamma"], inp["beta"], wl.eps)
        (g2,) = torch.autograd.grad(y2, x2, inp["dy"], create_graph=True)
        g2.sum().backward()
