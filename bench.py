#!/usr/bin/env python3
"""Benchmark: forward + backward of row-wise normalization layers on one MI355X.

A step is one forward and one backward (stage 1 + stage 2) of a layer over one batch of
synthetic input already resident in HBM.  Several copies of the inputs rotate through the
timed steps so that every step reads data last touched more than ~768 MB earlier, past the
256 MB Infinity Cache: the rate is HBM bandwidth, not cache bandwidth.

Prints ONE JSON line:
  value        algorithmic fwd+bwd bytes per step / step time (GB/s) of the headline workload
               (LayerNorm float32 [401408, 24]), timed over K steps between HIP events;
  config       the headline's details, and per_config: the same measurement for one workload of
               each shape the metric names (DyT 4096x64 f32; DyT 1048573x{32,128,256} bf16;
               RMSNorm 16384x2048 and 8192x4096 bf16; DyT, LayerNorm, RMSNorm 65536x{1025,
               4096,8192,16384} bf16), each with a parity spot check of its timed outputs
               against the CPU oracle; stream_probe: streaming ceilings at the headline's size;
  roofline     the headline's dominant kernel: its algorithmic bytes / its average duration;
  cpu_baseline the oracle timed on the host cores on a bounded sample of the headline.

Per-step kernel durations come from two kinds of timing: untraced back-to-back loops of the
forward call alone and the backward call alone (which add up to the step), and in-packet
dispatch timestamps in a separate traced region (what rocprofv3 reports; the timestamps
lengthen each kernel by about a microsecond, so their sum can exceed the untraced step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "achieved HBM GB/s (fwd+bwd) and % of peak, M>>N and wide-row norm configs"
# One workload of every shape the metric names (configurations 1 to 5), in that order.
CONFIG_WORKLOADS = (["dyt_f32_4096x64", "layernorm_f32_401408x24"] +
                    [f"dyt_bf16_1048573x{n}" for n in (32, 128, 256)] +
                    ["rmsnorm_bf16_16384x2048", "rmsnorm_bf16_8192x4096"] +
                    [f"wide_{l}_bf16_65536x{n}" for l in ("dyt", "layernorm", "rmsnorm")
                     for n in (1025, 4096, 8192, 16384)])


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline workload)")
    ap.add_argument("--configs", default=None,
                    help="comma-separated workload names for per_config (default: every configuration; 'none': skip)")
    ap.add_argument("--sweep", default=None, help="also time every workload and write JSON lines here")
    ap.add_argument("--only", default=None, help="comma-separated substrings: sweep only matching workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the per-config parity spot checks")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming probes")
    ap.add_argument("--probe-only", type=int, default=0, metavar="BYTES",
                    help="run 3 launches of the one-in-one-out streaming probe over BYTES and exit (a "
                         "known-size dispatch for calibrating HBM byte counters)")
    return ap.parse_args()


def kernel_source_sha() -> str:
    d = os.path.join(ROOT, "row_wise_normalization_dyt_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def kernel_bytes(wl, kernel: str) -> int:
    """Algorithmic HBM bytes of one launch of `kernel` on workload wl."""
    sx = 4 if wl.xdt == "f32" else 2
    sp = 4 if wl.pdt == "f32" else 2
    e = wl.M * wl.N
    stats = {"dyt": 0, "layernorm": 8, "rmsnorm": 4}[wl.layer] * wl.M
    nvec = {"dyt": 2, "layernorm": 2, "rmsnorm": 1}[wl.layer]
    if kernel.endswith("_fwd"):
        return 2 * e * sx + stats + nvec * wl.N * sp + (sp if wl.layer == "dyt" else 0)
    if kernel.endswith("_bwd"):
        return 3 * e * sx + stats + wl.N * sp + (sp if wl.layer == "dyt" else 0)
    if kernel == "colreduce":
        return nvec * wl.N * sp + (sp if wl.layer == "dyt" else 0)
    return 0


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def time_workload(wl, steps: int, warmup: int, chunk: int = 10):
    """Times `steps` steps of wl (untraced), the forward and backward calls alone, per-chunk step
    times and the traced per-kernel durations.  Returns the measurements and the first input
    set's inputs and outputs (the outputs of the last timed step on that set)."""
    import torch
    import workloads
    import row_wise_normalization_dyt_amd as rwn
    from row_wise_normalization_dyt_amd.prepared import PreparedStep

    base = workloads.make_inputs(wl, "cuda")
    sx = 4 if wl.xdt == "f32" else 2
    set_bytes = 4 * wl.M * wl.N * sx + 16 * wl.M
    nsets = max(1, min(256, math.ceil(3 * MALL_BYTES / max(set_bytes, 1))))
    sets = [PreparedStep(wl.layer, base if i == 0 else {k: v.clone() for k, v in base.items()}, wl.eps,
                         form=wl.form, param_grads=wl.param_grads) for i in range(nsets)]
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def region(fn, n):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    step = lambda i: sets[i % nsets].step()
    ms_step = region(step, steps)
    ms_fwd = region(lambda i: sets[i % nsets].fwd(), steps)
    ms_bwd = region(lambda i: sets[i % nsets].bwd(), steps)
    # distribution: events every `chunk` steps in a region of its own
    nch = max(2, steps // chunk)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    es = [ev() for _ in range(nch + 1)]
    es[0].record()
    for c in range(nch):
        for i in range(chunk):
            step(c * chunk + i)
        es[c + 1].record()
    torch.cuda.synchronize()
    per_chunk = [es[c].elapsed_time(es[c + 1]) / chunk for c in range(nch)]
    # traced region: in-packet timestamps on every kernel
    n_tr = max(steps, 10)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    rwn.trace_begin(3 * n_tr + 8)
    a, b = ev(), ev()
    a.record()
    for i in range(n_tr):
        step(i)
    b.record()
    torch.cuda.synchronize()
    events = rwn.trace_end(3 * n_tr + 8)
    per = {}
    for name, ms in events:
        tot, cnt = per.get(name, (0.0, 0))
        per[name] = (tot + ms, cnt + 1)
    kernels = {k: {"avg_ms": t / c, "launches": c, "total_ms": t} for k, (t, c) in per.items()}
    # the outputs of set 0 were last written by a timed step on set 0 (sets rotate in order)
    return {"ms_per_step": ms_step, "fwd_ms": ms_fwd, "bwd_ms": ms_bwd, "kernels": kernels, "nsets": nsets,
            "chunk_ms": per_chunk, "ms_per_step_traced": a.elapsed_time(b) / n_tr,
            "outputs": sets[0].outputs(), "inputs": base}


def roofline(wl, kernels, r=None):
    """The dominant kernel (most total traced time): its algorithmic bytes per launch / its
    average traced duration.  With r (untraced call timings), also that bytes count over the
    untraced back-to-back time of the call that launches it (forward, or backward stage 1 +
    stage 2), a lower bound on the kernel's own rate."""
    dom = max(kernels, key=lambda k: kernels[k]["total_ms"])
    b = kernel_bytes(wl, dom)
    achieved = b / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
    out = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
           "algorithmic_bytes_per_launch": b, "avg_launch_ms": round(kernels[dom]["avg_ms"], 5)}
    if r is not None:
        call = r["fwd_ms"] if dom.endswith("_fwd") else r["bwd_ms"]
        out["untraced_call_ms"] = round(call, 5)
        out["frac_untraced_call"] = round(b / (call * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    return out


def traffic_for(wl, dom):
    tdb_path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(tdb_path)) if os.path.exists(tdb_path) else {}
    rec = db.get(f"{wl.name}/{dom}")
    if rec and rec.get("kernel_source_sha") == kernel_source_sha():
        return rec.get("hbm_bytes_per_launch")
    return None


# ------------------------------------------------------------------------------------------
# CPU leg: the oracle on the host cores.  It times the oracle for the baseline and checks the
# outputs of the timed GPU steps against it.  (The only use of the oracle in this file.)

def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, inputs, target_s: float):
    """The oracle (as it stands) on rows [0, S) of the workload, S sized for ~target_s of CPU
    work (repeated if the whole workload takes less), on every host core."""
    import oracle
    import workloads
    cores = host_cores()
    oracle.set_threads(cores)
    h = {k: v.detach().cpu() for k, v in inputs.items()}

    def run(S):
        sub = {k: (v[:S] if k in ("x", "dy") else v) for k, v in h.items()}
        e = workloads.eps_f32(wl.eps)
        t = time.perf_counter()
        if wl.layer == "dyt":
            oracle.dyt_fwd(sub["x"], sub["alpha"], sub["gamma"], sub["beta"])
            oracle.dyt_bwd(sub["x"], sub["dy"], sub["alpha"], sub["gamma"])
        elif wl.layer == "layernorm":
            oracle.layernorm_fwd(sub["x"], sub["gamma"], sub["beta"], e)
            oracle.layernorm_bwd(sub["x"], sub["dy"], sub["gamma"], e)
        else:
            oracle.rmsnorm_fwd(sub["x"], sub["weight"], e, form=wl.form)
            oracle.rmsnorm_bwd(sub["x"], sub["dy"], sub["weight"], e, form=wl.form)
        return time.perf_counter() - t

    S0 = max(1, min(wl.M, 2_000_000 // wl.N))
    t0 = run(S0)
    S = max(1, min(wl.M, int(S0 * target_s / max(t0, 1e-3))))
    t = run(S) if S != S0 else t0
    passes = 1
    while t < target_s and passes < 1000:      # a sample smaller than the target: repeat it
        t += run(S)
        passes += 1
    sub_wl = wl.with_(M=S)
    gbps = passes * sub_wl.algorithmic_bytes()["total"] / t / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"rows [0, {S}) of {wl.M} x {wl.N} ({S * wl.N} elements), fwd+bwd, "
                      f"{passes} pass(es), {t:.1f} s"}


def parity_spot_check(wl, inputs, outputs):
    """The timed outputs against the oracle: y, dx (and the statistics) on sampled rows -- the
    first, last and tile-boundary rows and a seeded random sample -- and every parameter
    gradient over all rows.  Returns ok and, per output, the bound usage and the pages'
    accuracy diagnostics (max ULP, share within one ULP, elements outside the BF16 policy)."""
    import oracle  # noqa: F401  (through tests.gpu_cases)
    from tests import gpu_cases as gc
    oracle.set_threads(host_cores())
    rows = gc.sample_rows(wl.M, k=24)
    h = {k: v.detach().cpu() for k, v in inputs.items()}
    o = gc.oracle_run(wl.layer, h, wl.eps, rows=rows, grads=wl.param_grads, form=wl.form)
    g = {k: v for k, v in outputs.items()}
    reps = gc.compare(wl.layer, g, o, gc.DT[wl.xdt], gc.DT[wl.pdt], rows=rows, grads=wl.param_grads)
    out = {"ok": all(r.ok() for r in reps), "rows": len(rows)}
    for r in reps:
        out[r.name.split(".", 1)[1]] = {"bad": r.bad, "max_err_over_bound": round(r.max_ratio, 4),
                                        "max_ulp": round(r.max_ulp, 3), "within_1ulp": round(r.within_1ulp, 5),
                                        "outside_bf16_policy": r.outside_policy}
    return out


# ------------------------------------------------------------------------------------------

def stream_probes(sizes):
    """Streaming ceilings: the best rate of the probe kernel over its variants (loads in flight
    per lane, nontemporal hint, workgroups per CU) for one-in-one-out and two-in-one-out at
    each size, over rotating buffers (every launch streams from HBM)."""
    import torch
    import row_wise_normalization_dyt_amd as rwn
    res = {}
    for nbytes in sizes:
        nb = (nbytes + 15) // 16 * 16
        nrot = max(2, math.ceil(3 * MALL_BYTES / (3 * nb)))
        bufs = [[torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(3)] for _ in range(nrot)]
        for bb in bufs:
            for t in bb:
                t.fill_(1)
        for two in (False, True):
            best = None
            table = {}
            for unroll in (1, 4, 8):
                for nt in (0, 1):
                    for wpc in (4, 8, 16):
                        def launch(i):
                            a, b, c = bufs[i % nrot]
                            rwn.stream_probe(a, c, b if two else None, unroll=unroll, nontemporal=nt, wg_per_cu=wpc)
                        for i in range(5):
                            launch(i)
                        torch.cuda.synchronize()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        n = 40
                        e0.record()
                        for i in range(n):
                            launch(i)
                        e1.record()
                        torch.cuda.synchronize()
                        ms = e0.elapsed_time(e1) / n
                        gbps = (3 if two else 2) * nb / (ms * 1e-3) / 1e9
                        table[f"u{unroll}_nt{nt}_w{wpc}"] = round(gbps, 1)
                        if best is None or gbps > best[0]:
                            best = (gbps, ms, f"u{unroll}_nt{nt}_w{wpc}")
            res[f"{'two_in_one_out' if two else 'one_in_one_out'}_{nb}B"] = {
                "GBps": round(best[0], 1), "us_per_launch": round(best[1] * 1e3, 2), "variant": best[2],
                "variants": table}
        del bufs
        torch.cuda.empty_cache()
    return res


def steps_for(wl, target_ms: float = 60.0) -> int:
    """Steps whose timed region takes about target_ms (10..200), from the algorithmic bytes at
    ~5 TB/s plus ~15 us of launches per step."""
    est_ms = wl.algorithmic_bytes()["total"] / 5e12 * 1e3 + 0.015
    return int(max(10, min(200, target_ms / est_ms)))


def config_entry(wl, r, parity):
    byts = wl.algorithmic_bytes()["total"]
    v = byts / (r["ms_per_step"] * 1e-3) / 1e9
    rl = roofline(wl, r["kernels"], r)
    e = {"workload": wl.name, "layer": wl.layer, "M": wl.M, "N": wl.N, "x_dtype": wl.xdt, "param_dtype": wl.pdt,
         "GBps": round(v, 1), "pct_of_peak": round(100 * v / HBM_PEAK_GBPS, 2),
         "ms_per_step": round(r["ms_per_step"], 5),
         "ms_per_step_p10_p50_p90": [round(_pct(r["chunk_ms"], q), 5) for q in (0.1, 0.5, 0.9)],
         "fwd_ms": round(r["fwd_ms"], 5), "bwd_ms": round(r["bwd_ms"], 5),
         "kernel_ms_traced": {k: round(x["avg_ms"], 5) for k, x in r["kernels"].items()},
         "dominant_kernel": dict({k: rl[k] for k in ("kernel", "avg_launch_ms", "frac", "untraced_call_ms",
                                                     "frac_untraced_call")},
                                 traffic=traffic_for(wl, rl["kernel"])),
         "bytes_per_step": byts}
    if parity is not None:
        e["parity"] = parity
    return e


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on one GPU only; the path shards across GPUs by rows, "
              "but no multi-GPU run is measured. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    torch.cuda.set_device(0)
    if args.probe_only:
        import row_wise_normalization_dyt_amd as rwn
        nb = (args.probe_only + 15) // 16 * 16
        a, c = torch.ones(nb, dtype=torch.uint8, device="cuda"), torch.empty(nb, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            rwn.stream_probe(a, c, None, unroll=4, nontemporal=True, wg_per_cu=8)
        torch.cuda.synchronize()
        print(json.dumps({"probe_only_bytes": nb, "launches": 3}))
        return
    name = args.workload or workloads.HEADLINE
    wl = workloads.WORKLOADS[name]

    # Headline: K untraced steps (the value), then the call loops, chunked and traced regions.
    r = time_workload(wl, args.steps, args.warmup)
    byts = wl.algorithmic_bytes()["total"]
    value = byts / (r["ms_per_step"] * 1e-3) / 1e9
    rl = roofline(wl, r["kernels"], r)
    rl["traffic"] = traffic_for(wl, rl["kernel"])
    cfg = {"workload": wl.name, "layer": wl.layer, "M": wl.M, "N": wl.N, "x_dtype": wl.xdt,
           "param_dtype": wl.pdt, "bytes_per_step": byts, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
           "rotating_input_sets": r["nsets"],
           "ms_per_step_p10_p50_p90": [round(_pct(r["chunk_ms"], q), 5) for q in (0.1, 0.5, 0.9)],
           "fwd_ms": round(r["fwd_ms"], 5), "bwd_ms": round(r["bwd_ms"], 5),
           "ms_per_step_traced": round(r["ms_per_step_traced"], 5),
           "kernel_ms_traced": {k: round(v["avg_ms"], 5) for k, v in r["kernels"].items()},
           "timing_note": "fwd_ms/bwd_ms: untraced back-to-back loops of each call (they add up to "
                          "ms_per_step); kernel_ms_traced: in-packet dispatch timestamps in a traced region, "
                          "which lengthen every kernel by ~1 us"}
    head_parity = None if args.no_parity else parity_spot_check(wl, r["inputs"], r["outputs"])
    if head_parity is not None:
        cfg["parity"] = head_parity
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, r["inputs"], args.cpu_seconds)
    del r
    torch.cuda.empty_cache()

    if not args.no_probe:
        sx = 4 if wl.xdt == "f32" else 2
        cfg["stream_probe"] = stream_probes([wl.M * wl.N * sx, 512 << 20])

    per = []
    names = (CONFIG_WORKLOADS if args.configs is None else
             ([] if args.configs == "none" else args.configs.split(",")))
    for n in names:
        w = workloads.WORKLOADS[n]
        rr = time_workload(w, steps_for(w), 5)
        par = None if args.no_parity else parity_spot_check(w, rr["inputs"], rr["outputs"])
        ent = config_entry(w, rr, par)
        print("config", json.dumps(ent), file=sys.stderr, flush=True)
        per.append(ent)
        del rr
        torch.cuda.empty_cache()
    if per:
        cfg["per_config"] = per
        cfg["per_config_parity_ok"] = all(e.get("parity", {}).get("ok", True) for e in per)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(byts / value / 1e6, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.xdt, "data": "synthetic", "config": cfg,
        "roofline": rl,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)

    if args.sweep:
        with open(args.sweep, "w") as f:
            only = args.only.split(",") if args.only else None
            for n, w in workloads.WORKLOADS.items():
                if only and not any(o in n for o in only):
                    continue
                torch.cuda.empty_cache()
                rr = time_workload(w, max(10, min(args.steps, 100)), 5)
                rec = config_entry(w, rr, None)
                rec["env"] = {k: v for k, v in os.environ.items() if k.startswith("RWN_")}
                f.write(json.dumps(rec) + "\n")
                f.flush()
                print("sweep", json.dumps(rec), file=sys.stderr, flush=True)
                del rr


if __name__ == "__main__":
    main()
