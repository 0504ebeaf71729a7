"""The exact path against LoRA conversions on decode batches: time per
forward, adapter bytes, and the cost of padding every adapter to the pool's
largest rank.

"Does it actually work better?" (paper-daily.com explainer of "Scute: Exact
Batched Serving for PEFT Adapters Beyond LoRA") compares serving each method
exactly with converting it to LoRA by truncated SVD: VeRA at rank 256 (or
64) brings its own pair per tenant where the exact path reads the shared pair
once per step; a LoRA-only engine also pads every adapter to the pool's
largest rank. This tool builds those conversions from the loaded adapters
(lora_normal_form_amd.convert) and times them on this library's decode path:

    vera_tenants   128 tokens over T = 1, 2, 4, 8, 16 VeRA tenants (shared
                   rank-256 pair): exact against rank-256 LoRA conversions
    mixed_pool     128 tokens over 20 tenants, four each of LoRA r16, DoRA
                   r16, (IA)^3, VeRA (rank-256 pair) and OFT (blocks of 32):
                   exact; plain LoRA r16 for every tenant; (IA)^3, OFT, DoRA
                   converted at rank 64 with VeRA at 256 or at 64; and the
                   conversions padded to the pool's largest rank

Layer 4096 x 4096, bf16, synthetic adapters with the named workloads'
distributions. Forward times are medians over repetitions of many forwards
on one resident copy (HIP events). Conversion quality is the relative
Frobenius error of the truncated weight change (task accuracy needs data and
trained adapters and is not measured).

    python -m lora_normal_form_amd.conversion [--out PATH]
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import statistics
import sys

import numpy as np

from . import convert

D = 4096
N_TOK = 128


def _vera_wl(T, seed):
    from synth import AdapterSpec, WorkloadSpec, make_workload
    ta = np.random.default_rng(seed).integers(0, T, size=N_TOK)
    return make_workload(WorkloadSpec(f"vera_{T}tenants", "bf16", D, D, N_TOK,
                                      [AdapterSpec("vera") for _ in range(T)], vera_rank=256,
                                      assign="explicit", token_adapter=ta, seed=seed))


def _mixed_wl(seed, methods=None):
    from synth import AdapterSpec, WorkloadSpec, make_workload
    specs = methods or ([AdapterSpec("lora", rank=16)] * 4 + [AdapterSpec("dora", rank=16)] * 4 +
                        [AdapterSpec("ia3")] * 4 + [AdapterSpec("vera")] * 4 +
                        [AdapterSpec("oft", blk=32)] * 4)
    ta = np.random.default_rng(seed).integers(0, len(specs), size=N_TOK)
    return make_workload(WorkloadSpec("mixed_20tenants" if methods is None else "lora_20tenants",
                                      "bf16", D, D, N_TOK, specs, vera_rank=256, assign="explicit",
                                      token_adapter=ta, seed=seed))


def converted(wl, ranks: dict, pad_to: int = 0, seed: int = 0):
    """The workload with every adapter whose method is in `ranks` replaced by
    its rank-ranks[method] LoRA (truncated SVD of its weight change); LoRA
    adapters stay. pad_to > 0 zero-pads every LoRA to that rank. Returns the
    workload and {method: [relative errors]}."""
    from synth.workloads import Adapter
    from . import workload as glue
    host = glue.load(wl, device=-1, plan=False)
    ads, errs = [], {}
    for a in wl.adapters:
        if a.method == "lora":
            A, B, b, c = a.A, a.B, a.b, a.c
        else:
            sl = convert.slots(host.layer, a.id, wl.d_in, wl.d_out, wl.vera_rank)
            A, B, b, err = convert.to_lora(sl, wl.W, wl.A_sh, wl.B_sh, ranks[a.method], seed=seed + a.id)
            c = 1.0
            errs.setdefault(a.method, []).append(err)
        r = A.shape[0]
        if pad_to > r:
            A = np.concatenate([A, np.zeros((pad_to - r, wl.d_in))], 0)
            B = np.concatenate([B, np.zeros((wl.d_out, pad_to - r))], 1)
        ads.append(Adapter(a.id, "lora", rank=A.shape[0], c=c, A=A, B=B, b=b))
    host.layer.close()
    name = wl.name + "_lora" + "_".join(f"{m}{r}" for m, r in sorted(ranks.items())) + \
        (f"_pad{pad_to}" if pad_to else "")
    return dataclasses.replace(wl, name=name, adapters=ads, A_sh=None, B_sh=None), errs


def time_forward(torch, wl, iters=200, reps=7):
    from . import workload as glue
    ld = glue.load(wl, device=0)
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
    cost = ld.layer.cost(ld.batch)
    info = ld.batch.info()
    ld.batch.close()
    ld.layer.close()
    return {"us": statistics.median(ts), "adapter_mb": cost["adapter_bytes"] / 1e6,
            "bytes_mb": cost["bytes"] / 1e6, "path": info["path"], "max_rank": info["max_rank"]}


def run():
    import torch
    rows = []

    def rec(group, variant, wl, errs=None):
        t = time_forward(torch, wl)
        t.update(group=group, variant=variant, workload=wl.name,
                 conv_err={m: float(np.mean(v)) for m, v in (errs or {}).items()})
        rows.append(t)
        print(f"conversion: {group} {variant}: {t['us']:.2f} us, adapters {t['adapter_mb']:.1f} MB, "
              f"path {t['path']}, max rank {t['max_rank']} {t['conv_err']}", file=sys.stderr, flush=True)

    for T in (1, 2, 4, 8, 16):
        wl = _vera_wl(T, seed=100 + T)
        rec(f"vera_{T}", "exact", wl)
        cw, errs = converted(wl, {"vera": 256})
        rec(f"vera_{T}", "lora256", cw, errs)
    wl = _mixed_wl(seed=7)
    rec("mixed_20", "exact", wl)
    from synth import AdapterSpec
    rec("mixed_20", "plain_lora_r16", _mixed_wl(seed=7, methods=[AdapterSpec("lora", rank=16)] * 20))
    for vr in (256, 64):
        ranks = {"dora": 64, "ia3": 64, "oft": 64, "vera": vr}
        cw, errs = converted(wl, ranks)
        rec("mixed_20", f"lora64_vera{vr}", cw, errs)
        pw, _ = converted(wl, ranks, pad_to=vr)
        rec("mixed_20", f"lora64_vera{vr}_padded{vr}", pw, errs)
    return rows


def markdown(rows):
    out = ["| group | variant | µs / forward | vs exact | adapter MB | max rank | path | conversion error (rel. Frobenius, mean) |",
           "|---|---|---|---|---|---|---|---|"]
    exact = {r["group"]: r["us"] for r in rows if r["variant"] == "exact"}
    for r in rows:
        ce = ", ".join(f"{m} {100 * e:.1f}%" for m, e in sorted(r["conv_err"].items())) or "—"
        out.append(f"| {r['group']} | {r['variant']} | {r['us']:.2f} | {r['us'] / exact[r['group']]:.2f}× | "
                   f"{r['adapter_mb']:.1f} | {r['max_rank']} | {r['path']} | {ce} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    rows = run()
    if a.out:
        with open(a.out, "w") as f:
            json.dump(rows, f, indent=1)
    print(markdown(rows))


if __name__ == "__main__":
    main()
