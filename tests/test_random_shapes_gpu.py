"""GPU parity over seeded random shapes: random layer, dtype pair, width (narrow, medium, wide and
12 * 2^k-byte rows), row count (including multi-tile ones) and 16-bit base offset, each forward +
backward against the oracle under the bars of tests/tolerance.py.  The draws are fixed by the seed,
so a failure names a reproducible case; they reach plan combinations (flat, split, SHIFTED,
SCALAR, column blocks, several tiles per workgroup) that the hand-picked shapes may not."""
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
