"""GPU parity over seeded random shapes: random layer, dtype pair, width (narrow, medium, wide and
12 * 2^k-byte rows), row count (including multi-tile ones) and 16-bit base offset, each forward +
backward against the oracle under the bars of tests/tolerance.py.  The draws are fixed by the seed,
so a failure names a reproducible case; they reach plan combinations (flat, split, SHIFTED,
SCALAR, column blocks, several tiles per workgroup) that the hand-picked shapes may not.  A second
test does the same for random strided views (shuffled leading dimensions, column slices)."""
import random

import pytest
import torch

import workloads
from tests import gpu_cases as gc
from tests import tolerance as tol

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")]


def _cases(seed: int, n: int):
    rng = random.Random(seed)
    for i in range(n):
        layer = rng.choice(["dyt", "layernorm", "rmsnorm"])
        xdt, pdt = rng.choice(PAIRS)
        esz = 4 if xdt == "f32" else 2
        N = rng.choice([rng.randint(1, 64), rng.randint(1, 600), rng.randint(600, 4200),
                        max(1, 12 * 2 ** rng.randint(0, 6) // esz)])
        M = rng.choice([rng.randint(1, 70), rng.randint(1, 5000),
                        rng.randint(5000, 70000) if N <= 256 else rng.randint(1, 3000)])
        off = rng.choice([0, 0, 1, 3]) if xdt == "f32" else rng.choice([0, 0, 1, 2, 3])
        yield i, layer, xdt, pdt, M, N, off


@pytest.mark.parametrize("seed", [20261203])
def test_random_shapes(seed):
    reps = []
    for i, layer, xdt, pdt, M, N, off in _cases(seed, 200):
        wl = workloads.small(layer, M, N, xdt, pdt, seed=seed + i)
        print("case:", i, wl.name, "offset", off, flush=True)
        inp = workloads.make_inputs(wl)
        dev = {}
        for k, v in inp.items():
            if k in ("x", "dy") and off:
                buf = torch.empty(v.numel() + 16, dtype=v.dtype, device=DEV)
                view = buf[off:off + v.numel()].view(v.shape)
                view.copy_(v.to(DEV))
                dev[k] = view
            else:
                dev[k] = v.to(DEV)
        # offset views come back through the binding's same-offset outputs; NaN poisoning is
        # applied to aligned calls (its buffers are allocated at the aligned phase)
        g = gc.gpu_run(layer, dev, wl.eps, poison=off == 0)
        torch.cuda.synchronize()
        o = gc.oracle_run(layer, inp, wl.eps)
        reps += gc.compare(layer, g, o, gc.DT[xdt], gc.DT[pdt])
    tol.assert_reports(reps)


def _strided_cases(seed: int, n: int):
    rng = random.Random(seed)
    for i in range(n):
        layer = rng.choice(["dyt", "layernorm", "rmsnorm"])
        xdt, pdt = rng.choice([p for p in PAIRS if p != ("f16", "f32")])
        N = rng.choice([rng.randint(1, 64), rng.randint(64, 700), rng.choice([24, 64, 128, 256, 1024, 1025])])
        nd = rng.choice([3, 4])
        lead = [rng.randint(1, 24 if rng.random() < 0.3 else 9) for _ in range(nd - 1)]
        perm = list(range(nd - 1))
        rng.shuffle(perm)
        extra = rng.choice([0, 0, 8, 3])
        x_strided, dy_strided = rng.random() < 0.8, rng.random() < 0.6
        yield i, layer, xdt, pdt, N, lead, perm, extra, x_strided, dy_strided


@pytest.mark.parametrize("seed", [20261204])
def test_random_strided_views(seed):
    """x and dy as random views: leading dimensions stored in a shuffled order, rows padded so the
    view is a column slice, either operand dense instead.  The binding passes such views to the
    strided entry points (or the dense ones when they are dense after all); results must match the
    oracle on the same logical [M, N] values."""
    reps = []
    for i, layer, xdt, pdt, N, lead, perm, extra, xs_, dys_ in _strided_cases(seed, 150):
        nd = len(lead) + 1
        M = 1
        for v in lead:
            M *= v
        wl = workloads.small(layer, M, N, xdt, pdt, seed=seed + i)
        print("case:", i, wl.name, lead, perm, extra, flush=True)
        inp = workloads.make_inputs(wl)

        def strided(v):
            store = torch.zeros([lead[p] for p in perm] + [N + extra], dtype=v.dtype, device=DEV)
            inv = [perm.index(k) for k in range(nd - 1)]
            view = store.permute(*inv, nd - 1)[..., :N]
            view.copy_(v.reshape(*lead, N).to(DEV))
            return view

        dev = {k: v.to(DEV) for k, v in inp.items() if k not in ("x", "dy")}
        dev["x"] = strided(inp["x"]) if xs_ else inp["x"].reshape(*lead, N).to(DEV)
        dev["dy"] = strided(inp["dy"]) if dys_ else inp["dy"].reshape(*lead, N).to(DEV)
        g = gc.gpu_run(layer, dev, wl.eps, poison=False)
        torch.cuda.synchronize()
        o = gc.oracle_run(layer, inp, wl.eps)
        reps += gc.compare(layer, g, o, gc.DT[xdt], gc.DT[pdt])
    tol.assert_reports(reps)
