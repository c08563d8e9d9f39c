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


transformers = pytest.importorskip("transformers")
from transformers.models.llama.modeling_llama import LlamaRMSNorm  # noqa: E402


class _WeightBeforeCastRMSNorm(nn.Module):
    """Looks like the Llama RMSNorm (a 1-D weight, a float variance_epsilon) but multiplies the
    float32 normalized value by the weight before rounding: not a listed class, never swapped."""

    def __init__(self, n, eps=1e-6):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(n))
        self.variance_epsilon = eps

    def forward(self, x):
        h = x.float() * torch.rsqrt(x.float().pow(2).mean(-1, keepdim=True) + self.variance_epsilon)
        return (self.weight * h).to(x.dtype)


class _LlamaSubclass(LlamaRMSNorm):
    pass


class _LayerNormSubclass(nn.LayerNorm):
    pass


def _model():
    return nn.Sequential(nn.Linear(8, 8), nn.LayerNorm(8),
                         nn.Sequential(LlamaRMSNorm(8), nn.LayerNorm(8, elementwise_affine=False)),
                         nn.LayerNorm((2, 4)))


def test_swap_norms_replaces_and_shares_parameters():
    m = _model()
    ln_w = m[1].weight
    rms_w = m[2][0].weight
    orig_rms = m[2][0]
    assert ag.swap_norms(m) == 3
    assert isinstance(m[1], ag.LayerNorm) and m[1].weight is ln_w and m[1].eps == 1e-5
    assert isinstance(m[2][0], ag.RMSNorm) and m[2][0].weight is rms_w and m[2][0].variance_epsilon == 1e-6
    assert m[2][0].form == "cast_then_weight" and m[2][0]._eager is orig_rms
    assert isinstance(m[2][1], ag.LayerNorm) and m[2][1].weight is None and m[2][1].bias is None
    assert isinstance(m[3], nn.LayerNorm)            # two normalized dimensions: left alone
    assert isinstance(m[0], nn.Linear)
    # the original module is kept for the eager fallback but is not a submodule
    assert sorted(k for k, _ in m.named_parameters()) == ["0.bias", "0.weight", "1.bias", "1.weight", "2.0.weight",
                                                          "3.bias", "3.weight"]
    assert ag.swap_norms(m) == 0                      # idempotent


def test_swap_norms_leaves_look_alikes_subclasses_and_patched_modules():
    patched = LlamaRMSNorm(8)
    patched.forward = lambda x: x                     # an instance-level override
    wrapped_ln = nn.LayerNorm(8)
    wrapped_ln.forward = wrapped_ln.forward           # bound method stored on the instance
    m = nn.Sequential(_WeightBeforeCastRMSNorm(8), _LlamaSubclass(8), _LayerNormSubclass(8), patched, wrapped_ln)
    kinds = [type(c) for c in m]
    assert ag.swap_norms(m) == 0
    assert [type(c) for c in m] == kinds


def _form_expression(form, x, w, eps):
    """The three RMSNorm forms written out in eager torch (float32 statistics)."""
    h = x.float() * torch.rsqrt(x.float().pow(2).mean(-1, keepdim=True) + eps)
    if form == "cast_then_weight":
        return w * h.to(x.dtype)
    if form == "weight_then_cast":
        return (w.float() * h).to(x.dtype)
    return (h * (1.0 + w.float())).to(x.dtype)


@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16, torch.float32])
def test_listed_rmsnorm_classes_compute_their_form(xdt):
    """Every listed class the installed transformers defines computes exactly its form's
    expression (the kernels' variant is chosen from this list), and all three forms are
    represented."""
    classes = ag.rms_norm_classes()
    assert set(classes.values()) == set(ag.RMS_NORM_CLASSES)
    gen = torch.Generator().manual_seed(5)
    x = (torch.randn(33, 40, generator=gen) * 3).to(xdt)
    for cls, form in classes.items():
        mod = cls(40, eps=1e-6).to(xdt)
        with torch.no_grad():
            mod.weight.copy_(torch.randn(40, generator=gen).to(xdt))
        got = mod(x)
        want = _form_expression(form, x, mod.weight.detach(), 1e-6)
        assert got.dtype == want.dtype == xdt, cls.__name__
        assert torch.equal(got, want), cls.__name__
        # and not the other forms (the data tells them apart)
        for other in ag.RMS_NORM_CLASSES:
            if other != form and xdt != torch.float32:
                assert not torch.equal(got, _form_expression(other, x, mod.weight.detach(), 1e-6)), (cls, other)


def test_swapped_modules_fall_back_on_host_input_with_one_warning():
    m = nn.Sequential(nn.LayerNorm(16), LlamaRMSNorm(16))
    x = torch.randn(5, 16)
    ref = m(x)
    assert ag.swap_norms(m) == 2
    ag._WARNED.clear()
    with pytest.warns(UserWarning, match="eager forward") as rec:
        out = m(x)
        out2 = m(x)
    assert len([w for w in rec if "LayerNorm" in str(w.message)]) == 1
    assert len([w for w in rec if "LlamaRMSNorm" in str(w.message)]) == 1
    assert torch.equal(out, ref) and torch.equal(out2, ref)


def test_swap_norms_needs_the_library(monkeypatch):
    from row_wise_normalization_dyt_amd import _lib

    def missing():
        raise RuntimeError("librwnorm.so not built")
    monkeypatch.setattr(_lib, "load", missing)
    m = nn.Sequential(nn.LayerNorm(8))
    with pytest.raises(RuntimeError, match="not built"):
        ag.swap_norms(m)
    assert type(m[0]) is nn.LayerNorm


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


@pytest.mark.gpu
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16])
def test_swapped_modules_keep_the_originals_dtype_and_values(xdt):
    """On the GPU a swapped module returns the original module's dtype and values (to a few
    ulps of that dtype: the kernels reduce in another order), for a listed class of each form
    with a weight in x's dtype and in float32; the Llama form with a float32 weight under a
    16-bit input (the eager class returns float32 there) stays on the original's forward.
    (A LayerNorm with float32 parameters under a 16-bit input, which eager torch refuses, runs
    on the kernels and is compared with the float32 computation.)"""
    classes = ag.rms_norm_classes()
    picks = {}
    for cls, form in classes.items():
        picks.setdefault(form, cls)
    gen = torch.Generator().manual_seed(11)
    x = (torch.randn(257, 1024, generator=gen) * 2).to(xdt).cuda()
    mods = [(nn.LayerNorm(1024), "layernorm")] + [(cls(1024), form) for form, cls in picks.items()]
    for orig, form in mods:
        for wdt in (xdt, torch.float32):
            o = orig.to("cuda", wdt)
            with torch.no_grad():
                for p in o.parameters():
                    p.copy_(torch.randn(p.shape, generator=gen).to(wdt))
            print("case:", type(o).__name__, form, xdt, wdt, flush=True)
            try:
                ref = o(x)
            except RuntimeError:
                # eager nn.LayerNorm takes no float32 parameters under a 16-bit input; the
                # kernels do: compare with the float32 computation rounded once to x's dtype
                assert form == "layernorm" and wdt != xdt
                ref = nn.functional.layer_norm(x.float(), o.normalized_shape, o.weight.float(), o.bias.float(),
                                               o.eps).to(xdt)
            m = nn.Sequential(o)
            assert ag.swap_norms(m) == 1
            fallback = form == "cast_then_weight" and wdt != xdt
            out = m(x)
            torch.cuda.synchronize()
            assert out.dtype == ref.dtype, (type(o).__name__, wdt)
            if fallback:
                assert torch.equal(out, ref)
            else:
                ulp = 2.0 ** (-7 if xdt == torch.bfloat16 else -10)
                err = ((out.float() - ref.float()).abs() / ref.float().abs().clamp_min(1e-3)).max().item()
                assert err <= 4 * ulp, (type(o).__name__, wdt, err)


@pytest.mark.gpu
@pytest.mark.parametrize("layer", ["layernorm", "rmsnorm", "dyt"])
def test_autograd_head_major_upstream_gradient(layer, monkeypatch):
    """A q/k norm as attention uses it: x is [B, S, H, D] contiguous, the output is read transposed to
    [B, H, S, D], so the gradient reaching the norm is a head-major view.  The backward takes it in
    place through the strided entry point (no copy), and x's and the parameters' gradients match
    the oracle on the logical rows."""
    B, S, H, D = 2, 300, 32, 128
    pdt = "bf16" if layer == "rmsnorm" else "f32"
    wl = workloads.small(layer, B * S * H, D, "bf16", pdt, seed=9)
    print("case:", wl, flush=True)
    inp = workloads.make_inputs(wl)
    calls = []
    real = rwn._try_strided
    monkeypatch.setattr(rwn, "_try_strided", lambda lib, fn, call: calls.append(fn) or real(lib, fn, call))
    x = inp["x"].reshape(B, S, H, D).cuda().requires_grad_(True)
    ps = [inp[k].cuda().requires_grad_(True) for k in {"dyt": ["alpha", "gamma", "beta"],
                                                        "layernorm": ["gamma", "beta"], "rmsnorm": ["weight"]}[layer]]
    if layer == "dyt":
        y = ag.dyt(x, *ps)
    elif layer == "layernorm":
        y = ag.layer_norm(x, *ps, eps=wl.eps)
    else:
        y = ag.rms_norm(x, *ps, eps=wl.eps)
    g = inp["dy"].reshape(B, S, H, D).transpose(1, 2).contiguous().cuda()   # upstream gradient of y.transpose(1, 2)
    y.transpose(1, 2).backward(g)
    torch.cuda.synchronize()
    assert calls == [f"{'dyt' if layer == 'dyt' else layer}_bwd_strided"], calls
    names = {"dyt": ["dalpha", "dgamma", "dbeta"], "layernorm": ["dgamma", "dbeta"], "rmsnorm": ["dweight"]}[layer]
    got = {"y": y.detach().reshape(-1, D), "dx": x.grad.reshape(-1, D)}
    got.update({nm: p.grad for p, nm in zip(ps, names)})
    tol.assert_reports(gc.compare(layer, got, gc.oracle_run(layer, inp, wl.eps), gc.DT["bf16"], gc.DT[pdt]))
