#!/usr/bin/env python3
"""Benchmark of the normal-form batched adapter layer on one MI355X.

A step is one forward of the whole layer (rotation, shrink, base GEMM with
the s / b epilogue, expand, shared VeRA term) over one batch. The default
workload is the mixed five-method decode batch: 4096 -> 4096, 128 tokens
over 40 adapters (8 each of LoRA r16, DoRA r16, (IA)^3, VeRA with a shared
rank-256 pair, OFT block 32), tokens assigned uniformly at random.

Inputs are resident in HBM when timing starts. The timed loop cycles over
several complete copies of the workload (x, W, y, every adapter, the VeRA
pair) whose total exceeds twice the 256 MB Infinity Cache, so each forward
streams its bytes from HBM rather than from the cache.

Prints ONE JSON line. Also reports the roofline of the dominant kernel
(algorithmic bytes per launch / its mean launch time from HIP events), the
CPU oracle timed on the host, and the mixed-method overhead two ways: against
the all-LoRA workload (4096 -> 4096, 128 tokens over 64 LoRA r16 adapters),
and against a matched batch with the mixed workload's token assignment where
every one of its 40 adapters is LoRA r16 (the same number of adapters, as the
explainer's mixed-pool comparison has it).
"""

import argparse
import json
import math
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("mixed-adapter layer tokens/s + achieved HBM GB/s (% peak), 4096², 128 tok")
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="named workload index (0..4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overhead", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", type=float, default=0.0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (HBM-counter calibration)")
    return ap.parse_args()


def rotating_copies(wl, n_sets):
    from lora_normal_form_amd import workload as glue
    sets = []
    for i in range(n_sets):
        sets.append(glue.load(wl, device=0))
    return sets


def footprint_bytes(ld, wl, cost):
    # bytes one copy of the workload occupies (x, W, y, adapters, VeRA pair)
    return cost["bytes"] + (wl.vera_rank * (wl.d_in + wl.d_out) * 2 if wl.A_sh is not None else 0)


def time_forwards(torch, sets, steps, warmup, profile=False):
    from lora_normal_form_amd import scute
    if profile:
        for s in sets:
            scute.scute_profile_enable(s.layer.h, True)
            scute.scute_profile_read(s.layer.h)
    for i in range(warmup):
        s = sets[i % len(sets)]
        s.layer.forward(s.batch, s.x, s.W, s.y)
    torch.cuda.synchronize()
    if profile:
        for s in sets:
            scute.scute_profile_read(s.layer.h)
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        s = sets[i % len(sets)]
        s.layer.forward(s.batch, s.x, s.W, s.y)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    kernels = {}
    if profile:
        for s in sets:
            for name, v in scute.scute_profile_read(s.layer.h).items():
                k = kernels.setdefault(name, {"launches": 0, "total_ms": 0.0})
                k["launches"] += v["launches"]
                k["total_ms"] += v["total_ms"]
            scute.scute_profile_enable(s.layer.h, False)
    return gpu_ms, wall, kernels


MFMA_BF16_PEAK_TFLOPS = 2500.0


def dominant_kernel_flops(name, cost):
    """Algorithmic flops of one launch of an MFMA-bound kernel (None for the
    HBM-bound ones): prefill_main computes the base GEMM (x W) and the
    expands (t B', u B_sh); its second pass over W for the rotated rows'
    Delta is not counted, since the method itself computes (x R) W once."""
    if name == "prefill_main":
        return cost["gemm_flops"]
    return None


def dominant_kernel_bytes(name, wl, cost):
    """Algorithmic bytes one launch of kernel ``name`` must move.

    decode_main (base GEMM + fused expand): x, W, y, touched adapters' B', s,
    b, VeRA e, and the shared B_sh once; decode_prologue (rotation, shrinks):
    x, A', P, VeRA d, shared A_sh; fd_main (the fused decode kernel): all of
    the forward's bytes but the rotation blocks; generic gemm: x, W, y.
    """
    es = 2 if wl.dtype == "bf16" else 4
    xwy = wl.n * wl.d_in * es + wl.d_in * wl.d_out * es + wl.n * wl.d_out * 4
    if name == "decode_main":
        return cost["gemm_bytes"]
    if name == "decode_prologue":
        return cost["prologue_bytes"]
    if name == "fd_main":
        # the fused kernel moves everything but the rotation blocks, which
        # fd_rotate reads: x, W, y, touched adapters' factors and vectors,
        # the shared VeRA pair
        return cost["bytes"] - rotation_bytes(wl)
    if name == "gemm":
        return xwy
    return None


def rotation_bytes(wl):
    """Stored rotation blocks (R - I) of the adapters that have tokens: d_in x
    blk elements each, at the activation size."""
    es = 2 if wl.dtype == "bf16" else 4
    touched = set(int(a) for a in wl.token_adapter if a >= 0)
    total = 0
    for a in wl.adapters:
        if a.id in touched and (a.Q is not None or a.R is not None):
            total += wl.d_in * a.blk * es
    return total


def measured_traffic(kernel, wl):
    """HBM bytes per launch of ``kernel`` from the committed counter summary
    for this workload, or None when there is none or the kernel sources have
    changed since the counters were taken."""
    from lora_normal_form_amd import profsum
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != profsum.source_sha():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("fetch_bytes") is None or k.get("write_bytes") is None:
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def calib_copy(torch, mib):
    n = int(mib * 2 ** 20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def matched_lora(wl):
    """The same batch (shape, tokens, token -> adapter assignment, seed) with
    every adapter replaced by a LoRA adapter of rank 16 (c = 2)."""
    from synth import AdapterSpec, WorkloadSpec, make_workload
    ads = [AdapterSpec("lora", rank=16, c=2.0) for _ in wl.adapters]
    return make_workload(WorkloadSpec(wl.name + "_matched_lora_r16", wl.dtype, wl.d_in, wl.d_out,
                                      wl.n, ads, assign="explicit",
                                      token_adapter=wl.token_adapter, seed=wl.seed))


def cpu_baseline(wl, seconds):
    """The oracle on the host cores: three timed runs of whole batches of the
    same workload (each at least seconds / 3), reporting the median rate."""
    import statistics
    import numpy as np  # noqa: F401
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    rates, reps_all, dt_all = [], 0, 0.0
    for _ in range(3):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.forward(wl)
            reps += 1
            if time.perf_counter() - t0 >= seconds / 3:
                break
        dt = time.perf_counter() - t0
        rates.append(wl.n * reps / dt)
        reps_all += reps
        dt_all += dt
    return {"value": statistics.median(rates), "unit": "tokens/s", "cores": int(cores),
            "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"median of 3 runs of whole batches ({wl.n} tokens) of the same workload, "
                      f"{reps_all} repetition(s) in {dt_all:.1f} s of numpy fp64 on {cores} BLAS "
                      f"thread(s) (host reports {os.cpu_count()} CPUs)",
            "runs": [round(r, 3) for r in rates]}


def measure(torch, wl, steps, warmup):
    from lora_normal_form_amd import scute
    first = rotating_copies(wl, 1)
    cost = first[0].layer.cost(first[0].batch)
    fp = footprint_bytes(first[0], wl, cost)
    n_sets = max(2, int(math.ceil(2.2 * MALL_BYTES / fp)))
    sets = first + rotating_copies(wl, n_sets - 1)
    gpu_ms, wall, _ = time_forwards(torch, sets, steps, warmup)
    _, _, kernels = time_forwards(torch, sets, steps, warmup, profile=True)
    return {"cost": cost, "n_sets": n_sets, "gpu_ms": gpu_ms, "wall": wall, "kernels": kernels,
            "sets": sets, "plan_us": plan_host_us(torch, first[0], wl)}


def plan_host_us(torch, ld, wl, reps=20):
    """Host time of building the batch plan (segment builder and its tables'
    upload), median of `reps` builds; the plan is built once, outside the
    timed loop."""
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        b = ld.layer.plan(wl.token_adapter)
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e6)
        b.close()
    return round(statistics.median(ts), 1)


def main():
    args = parse()
    if args.gpus != 1:
        sys.stderr.write("bench.py: this build measures one GPU only; --gpus must be 1 "
                         "(the layer is token-parallel and shards with no in-layer "
                         "communication, but nothing here runs on a second GPU)\n")
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        sys.stderr.write("bench.py: no GPU visible\n")
        sys.exit(1)
    from synth import make_config
    from lora_normal_form_amd import scute  # noqa: F401  (fails loudly if not built)

    wl = make_config(args.workload)
    print(f"bench: workload {wl.name}, building rotating copies", file=sys.stderr, flush=True)
    m = measure(torch, wl, args.steps, args.warmup)
    cost = m["cost"]
    ms = m["gpu_ms"] / args.steps
    tok_s = wl.n / (ms * 1e-3)
    gbps = cost["bytes"] / (ms * 1e-3) / 1e9
    print(f"bench: {ms * 1e3:.2f} us/forward, {gbps:.0f} GB/s", file=sys.stderr, flush=True)

    # dominant kernel roofline
    kern = m["kernels"]
    dom = max(kern.items(), key=lambda kv: kv[1]["total_ms"])[0] if kern else None
    roof = None
    if dom is not None:
        k = kern[dom]
        avg_s = k["total_ms"] / max(1, k["launches"]) * 1e-3
        kb = dominant_kernel_bytes(dom, wl, cost)
        kf = dominant_kernel_flops(dom, cost)
        if kf is not None:
            ach = kf / avg_s / 1e12
            tr = measured_traffic(dom, wl)
            roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": None if tr is None else round(tr),
                    "kernel": dom, "avg_launch_us": round(avg_s * 1e6, 3),
                    "flops_per_launch": kf}
        elif kb is not None:
            ach = kb / avg_s / 1e9
            tr = measured_traffic(dom, wl)
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                    "traffic": None if tr is None else round(tr),
                    "kernel": dom, "avg_launch_us": round(avg_s * 1e6, 3),
                    "bytes_per_launch": kb}

    extra = {"gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
             "bytes_per_forward": cost["bytes"], "adapter_bytes": cost["adapter_bytes"],
             "flops_per_forward": cost["flops"], "launches_per_forward": cost["launches"],
             "kernels_us": {k: round(v["total_ms"] / max(1, v["launches"]) * 1e3, 3)
                            for k, v in kern.items()},
             "rotating_sets": m["n_sets"], "wall_s": round(m["wall"], 4),
             "plan_host_us": m["plan_us"]}
    del m

    if not args.no_overhead and args.workload == 2:
        wl1 = make_config(1)
        print("bench: all-LoRA comparison workload", file=sys.stderr, flush=True)
        m1 = measure(torch, wl1, args.steps, args.warmup)
        ms1 = m1["gpu_ms"] / args.steps
        extra["all_lora_us"] = round(ms1 * 1e3, 3)
        extra["all_lora_gbps"] = round(m1["cost"]["bytes"] / (ms1 * 1e-3) / 1e9, 1)
        extra["mixed_over_all_lora_time"] = round(ms / ms1, 4)
        del m1
        print("bench: matched all-LoRA batch (same assignment, 40 x LoRA r16)", file=sys.stderr,
              flush=True)
        wlm = matched_lora(wl)
        m2 = measure(torch, wlm, args.steps, args.warmup)
        ms2 = m2["gpu_ms"] / args.steps
        extra["matched_lora_us"] = round(ms2 * 1e3, 3)
        extra["matched_lora_gbps"] = round(m2["cost"]["bytes"] / (ms2 * 1e-3) / 1e9, 1)
        extra["mixed_over_matched_lora_time"] = round(ms / ms2, 4)
        del m2

    if args.calib_copy > 0:
        calib_copy(torch, args.calib_copy)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds)

    out = {"metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic (seeded; shapes and distributions of the named workload)",
           "config": {"workload": wl.name, "tokens": wl.n, "d_in": wl.d_in, "d_out": wl.d_out,
                      "adapters": len(wl.adapters), "seed": wl.seed},
           "roofline": roof, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
