"""Route comparison and time-model check for the decode path on one GPU.

"Where is the cheapest place to compute the remaining slots?" (paper-daily.com
explainer of "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA")
prices a route by the bytes it moves and the kernels it launches: added time
= extra bytes / memory bandwidth + extra launches x launch cost, with no
fitted parameter. This tool measures, on the decode workloads, what each route
variant of the decode path (plan flags SCUTE_PLAN_ROUTE_*) adds to the time of
the route it is compared with, and sets that against the model:

    expand_pass  vs fused        s, b and the own term in an expand pass, the
                                 VeRA term in a VeRA pass, after the GEMM
    separate_s   vs expand_pass  s by a pass of its own (s copied to every
                                 row, then multiplied) before the expand
    vera_pass    vs fused        the VeRA term in a pass of its own
    rotate_pass  vs fused        the OFT rotation in a pass of its own

The bandwidth is MI355X's published 8 TB/s and the launch cost is measured
here: back-to-back empty kernels on one stream, each timed as the stream
sees it. Forward times are medians over repetitions of many forwards on one
resident copy of the workload (x, W, adapters hot in the 256 MB MALL), so
the extra bytes of a route are mostly y, which the passes re-read while it
is still cached. Every route also has a -m gpu parity test against the
oracle (tests/test_routes_gpu.py).

    python -m lora_normal_form_amd.routes [--iters 200] [--reps 7] [--out PATH]
"""

from __future__ import annotations

import argparse
import json
import statistics
import sys

from . import costmodel

ROUTE_FLAGS = {"fused": 0, "expand_pass": 2, "separate_s": 2 | 4, "vera_pass": 8, "rotate_pass": 16}
COMPARE = [("expand_pass", "fused"), ("separate_s", "expand_pass"), ("vera_pass", "fused"),
           ("rotate_pass", "fused")]


def launch_cost_us(torch, count=2000, reps=5):
    """Median time per empty kernel launched back to back on one stream."""
    from . import scute
    scute.scute_launch_empty(100)
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        scute.scute_launch_empty(count, torch.cuda.current_stream().cuda_stream)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / count)
    return statistics.median(out)


def row_counts(ld, wl):
    """Rows by the slots the route passes touch (from the loaded adapters)."""
    import numpy as np
    info = {a.id: ld.layer.info(a.id) for a in wl.adapters}
    ta = np.asarray(wl.token_adapter)
    c = {"n": int(wl.n), "d_out": int(wl.d_out), "exp_rows": 0, "s_rows": 0, "s_chunks": 0,
         "vera_rows": 0, "rot_rows": 0}
    for aid, inf in info.items():
        k = int(np.sum(ta == aid))
        if k == 0:
            continue
        if inf["has_s"] or inf["has_b"] or inf["has_term"]:
            c["exp_rows"] += k
        if inf["has_s"]:
            c["s_rows"] += k
            c["s_chunks"] += -(-k // 16)
        if inf["has_vera"]:
            c["vera_rows"] += k
        if inf["has_R"]:
            c["rot_rows"] += k
    return c


def time_route(torch, wl, flags, iters, reps, shared=None):
    """Median us per forward and per-kernel us (event-timed) of one route."""
    from . import scute
    from . import workload as glue
    ld = glue.load(wl, device=0, flags=flags, shared=shared)
    for _ in range(20):
        ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / iters)
    scute.scute_profile_enable(ld.layer.h, True)
    scute.scute_profile_read(ld.layer.h)
    for _ in range(iters):
        ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    kern = {k: v["total_ms"] / max(1, v["launches"]) * 1e3
            for k, v in scute.scute_profile_read(ld.layer.h).items()}
    scute.scute_profile_enable(ld.layer.h, False)
    counts = row_counts(ld, wl)
    cost = ld.layer.cost(ld.batch)
    keep = (ld.x, ld.W, ld.A_sh, ld.B_sh)
    ld.batch.close()
    ld.layer.close()
    return statistics.median(ts), kern, counts, cost, keep


def dora_workload():
    """128 decode tokens over 16 DoRA r16 adapters on a 4096 x 4096 layer
    (the explainer's s comparison is on DoRA tenants)."""
    import numpy as np
    from synth import AdapterSpec, WorkloadSpec, make_workload
    ta = np.random.default_rng(7).integers(0, 16, size=128)
    return make_workload(WorkloadSpec("dora_bf16_4096x4096_128tok_16xr16", "bf16", 4096, 4096, 128,
                                      [AdapterSpec("dora", rank=16) for _ in range(16)],
                                      assign="explicit", token_adapter=ta, seed=7,
                                      sigma_l=0.1, sigma_m=0.05))


def run(iters=200, reps=7, workloads=(1, 2, 3, "dora")):
    import os
    import torch
    from synth import make_config
    os.environ["SCUTE_DECODE"] = "2"  # the fused route is the two-launch decode path
    lc = launch_cost_us(torch)
    print(f"routes: launch cost {lc:.3f} us per empty kernel", file=sys.stderr, flush=True)
    rows, routes = [], {}
    for w in workloads:
        wl = dora_workload() if w == "dora" else make_config(w)
        shared = None
        res = {}
        counts = None
        for name, flags in ROUTE_FLAGS.items():
            if counts is not None and ((name == "rotate_pass" and counts["rot_rows"] == 0) or
                                       (name == "vera_pass" and counts["vera_rows"] == 0)):
                continue
            us, kern, counts, cost, shared = time_route(torch, wl, flags, iters, reps, shared)
            res[name] = {"us": us, "kernels_us": kern, "launches": cost["launches"]}
            print(f"routes: {wl.name} {name}: {us:.2f} us/forward {cost['launches']} launches "
                  f"{ {k: round(v, 2) for k, v in kern.items()} }", file=sys.stderr, flush=True)
        routes[wl.name] = {"counts": counts, "routes": res}
        for route, ref in COMPARE:
            if route not in res or ref not in res:
                continue
            b, l = costmodel.route_extra(route, **counts)
            pred = costmodel.added_time(b, costmodel.HBM_BYTES_PER_S, l, lc * 1e-6) * 1e6
            meas = res[route]["us"] - res[ref]["us"]
            rows.append({"workload": wl.name, "route": route, "vs": ref, "extra_bytes": b,
                         "extra_launches": l, "launches": res[route]["launches"],
                         "predicted_us": pred, "measured_us": meas,
                         "total_us": res[route]["us"],
                         "error_of_total": abs(pred - meas) / res[route]["us"]})
    errs = [r["error_of_total"] for r in rows]
    return {"launch_cost_us": lc, "rows": rows, "routes": routes,
            "median_error_of_total": statistics.median(errs) if errs else None}


def markdown(res):
    out = [f"launch cost (empty kernel, back to back): {res['launch_cost_us']:.3f} us", "",
           "| workload | route | vs | extra MB | extra launches | predicted µs | measured µs | "
           "route total µs | error / total |", "|---|---|---|---|---|---|---|---|---|"]
    for r in res["rows"]:
        out.append(f"| {r['workload']} | {r['route']} | {r['vs']} | {r['extra_bytes'] / 1e6:.2f} | "
                   f"{r['extra_launches']} | {r['predicted_us']:.2f} | {r['measured_us']:.2f} | "
                   f"{r['total_us']:.2f} | {100 * r['error_of_total']:.1f}% |")
    if res["median_error_of_total"] is not None:
        out += ["", f"median error of total time: {100 * res['median_error_of_total']:.1f}%"]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=200)
    ap.add_argument("--reps", type=int, default=7)
    ap.add_argument("--out", default=None, help="also write the results as JSON here")
    a = ap.parse_args()
    res = run(a.iters, a.reps)
    if a.out:
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1)
    print(markdown(res))


if __name__ == "__main__":
    main()
