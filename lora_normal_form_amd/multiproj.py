"""Multi-projection layers built on the single-layer library: the attention
input projections q, k, v, and the FFN's gated up projection.

"How does Scute plug into vLLM?" (paper-daily.com explainer of "Scute:
Exact Batched Serving for PEFT Adapters Beyond LoRA"): the base GEMM is split
into q, k and v when OFT is present, because each projection has its own
rotation of the input; otherwise q, k and v are one GEMM over the stacked
weights. "What problem is it solving?" and "The big picture": (IA)^3
multiplies the keys, the values and the FFN intermediate silu(x W_g) (.)
x W_u by learned vectors; the first two are s slots of the k and v
projections, the last (products reorder) the s slot of the up projection.

QKV, fused   one layer over W_qkv = [W_q; W_k; W_v] ([d_q + d_k + d_v][d_in]).
             Each tenant's per-projection slots, as the library folds them
             (read back with scute_read_slot), become one normal-form
             adapter: s and b concatenated (ones / zeros on projections the
             tenant leaves alone), one own term with the A' stacked and the
             B' block diagonal (its rank the sum of theirs), and, when the
             tenant rotates, one rotation per projection (the identity where
             it does not): the layer's projections are set to the q / k / v
             column ranges and the adapter loads with
             scute_load_adapter_proj, so OFT tenants keep the single GEMM.
             VeRA: each projection has its own shared pair, so the fused
             layer's pair is theirs side by side, A_sh stacked and B_sh
             block diagonal (its rank the sum of theirs), and a tenant's d
             and e are its projections' concatenated (d zero on projections
             without its VeRA term). Exact.
QKV, split   three layers and three forwards; any method.
FFN          a gate layer (base weight only) and the up layer with the
             tenants' adapters ((IA)^3's l on its s slot), then
             scute_silu_gate: h = silu(g) (.) u.

    python -m lora_normal_form_amd.multiproj [--out PATH]   (timing on one GPU)
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import statistics
import sys

import numpy as np

from . import convert, scute


# ---- workloads -----------------------------------------------------------------------------

def projection_workloads(tenants, n_tok, d_in, d_outs, seed, vera_rank=0, dtype="bf16",
                         none_frac=0.0):
    """One synthetic workload per projection sharing x and the tokens'
    tenants. tenants: list of per-projection AdapterSpec tuples (None: the
    tenant leaves that projection alone). Returns (workloads, tenant of each
    token (-1: none))."""
    from synth import WorkloadSpec, make_workload
    rng = np.random.default_rng(seed)
    tt = rng.integers(0, len(tenants), size=n_tok)
    tt[rng.random(n_tok) < none_frac] = -1
    wls, x = [], None
    for p, d_out in enumerate(d_outs):
        specs, ids = [], {}
        for t, per in enumerate(tenants):
            if per[p] is not None:
                ids[t] = len(specs)
                specs.append(per[p])
        ta = np.array([ids.get(int(t), -1) if t >= 0 else -1 for t in tt], dtype=np.int64)
        wl = make_workload(WorkloadSpec(f"proj{p}", dtype, d_in, d_out, n_tok, specs,
                                        vera_rank=vera_rank, assign="explicit", token_adapter=ta,
                                        seed=seed + 1 + p))
        if x is None:
            x = wl.x
        else:
            wl = dataclasses.replace(wl, x=x)
        wls.append((wl, ids))
    return wls, tt


# ---- QKV ---------------------------------------------------------------------------------------

class QKVSplit:
    """q, k and v as three layers (any method); forward returns the three outputs."""

    def __init__(self, wls, device=0, flags=0):
        from . import workload as glue
        self.parts = [glue.load(wl, device=device, flags=flags) for wl, _ in wls]

    def forward(self):
        for ld in self.parts:
            ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
        return [ld.y for ld in self.parts]

    def close(self):
        for ld in self.parts:
            ld.batch.close()
            ld.layer.close()


def fused_vera_pair(wls):
    """The fused layer's shared VeRA pair from the projections' pairs: A_sh
    [sum r][d_in] stacked, B_sh [sum d_out][sum r] block diagonal; with the
    projections' ranks. None when no projection has a pair."""
    ranks = [wl.vera_rank for wl, _ in wls]
    if not any(ranks):
        return None
    d_in, d_outs = wls[0][0].d_in, [wl.d_out for wl, _ in wls]
    A = np.zeros((sum(ranks), d_in))
    B = np.zeros((sum(d_outs), sum(ranks)))
    r0 = c0 = 0
    for (wl, _), r, d in zip(wls, ranks, d_outs):
        if r:
            A[r0:r0 + r] = wl.A_sh
            B[c0:c0 + d, r0:r0 + r] = wl.B_sh
        r0, c0 = r0 + r, c0 + d
    return A, B, ranks


def fused_slots(per_proj, d_outs, vera_ranks=None):
    """One normal-form adapter's arrays from a tenant's per-projection folded
    slots (None for a projection it leaves alone). "R_proj" is None when no
    projection rotates, else one rotation per projection (None: identity).
    vera_ranks: each projection's shared-pair rank (needed with a VeRA term)."""
    d_in = None
    for sl in per_proj:
        if sl is None:
            continue
        if sl["A"] is not None:
            d_in = sl["A"].shape[1]
    rot = [sl is not None and sl["R_minus_I"] is not None for sl in per_proj]
    blks = {sl["R_minus_I"].shape[1] for sl, r in zip(per_proj, rot) if r}
    if len(blks) > 1:
        raise ValueError("rotations of different block sizes need the split q / k / v layers")
    s = np.concatenate([sl["s"] if sl is not None and sl["s"] is not None else np.ones(d)
                        for sl, d in zip(per_proj, d_outs)])
    b = np.concatenate([sl["b"] if sl is not None and sl["b"] is not None else np.zeros(d)
                        for sl, d in zip(per_proj, d_outs)])
    has_s = any(sl is not None and sl["s"] is not None for sl in per_proj)
    has_b = any(sl is not None and sl["b"] is not None for sl in per_proj)
    terms = [(p, sl["A"], sl["B"]) for p, sl in enumerate(per_proj) if sl is not None and sl["A"] is not None]
    out = {"s": s if has_s else None, "b": b if has_b else None, "rank": 0, "A": None, "B": None,
           "R_proj": None, "blk": 0, "vd": None, "ve": None}
    has_v = [sl is not None and sl["vd"] is not None for sl in per_proj]
    if any(has_v):
        if vera_ranks is None:
            raise ValueError("a VeRA term needs the projections' shared-pair ranks")
        out["vd"] = np.concatenate([sl["vd"] if v else np.zeros(r)
                                    for sl, v, r in zip(per_proj, has_v, vera_ranks)])
        out["ve"] = np.concatenate([sl["ve"] if v else np.ones(d)
                                    for sl, v, d in zip(per_proj, has_v, d_outs)])
    if blks:
        blk = blks.pop()
        out["blk"] = blk
        out["R_proj"] = [np.eye(blk)[None] + sl["R_minus_I"] if r else None for sl, r in zip(per_proj, rot)]
    if terms:
        r = sum(A.shape[0] for _, A, _ in terms)
        A = np.zeros((r, d_in))
        B = np.zeros((sum(d_outs), r))
        k = 0
        offs = np.concatenate([[0], np.cumsum(d_outs)])
        for p, Ap, Bp in terms:
            A[k:k + Ap.shape[0]] = Ap
            B[offs[p]:offs[p + 1], k:k + Ap.shape[0]] = Bp
            k += Ap.shape[0]
        out.update(rank=r, A=A, B=B)
    return out


def fused_layer(wls, n_tenants, device=0):
    """The q / k / v layer over the stacked weights with every tenant's fused
    normal-form adapter loaded (device -1: a host-only layer)."""
    from . import workload as glue
    d_outs = [wl.d_out for wl, _ in wls]
    wl0 = wls[0][0]
    hosts = [glue.load(wl, device=-1, plan=False) for wl, _ in wls]
    layer = scute.Layer(wl0.d_in, sum(d_outs), wl0.dtype, max_adapters=max(1, n_tenants), device=device)
    pair = fused_vera_pair(wls)
    ranks = pair[2] if pair else None
    fused = []
    for t in range(n_tenants):
        per = [convert.slots(h.layer, ids[t], wl.d_in, wl.d_out, wl.vera_rank) if t in ids else None
               for (wl, ids), h in zip(wls, hosts)]
        fused.append(None if all(p is None for p in per) else fused_slots(per, d_outs, ranks))
    if pair is not None and any(f is not None and f["vd"] is not None for f in fused):
        if device >= 0:
            import torch
            dev = torch.device("cuda", device)
            A_f, B_f = glue.to_device(pair[0], wl0.dtype, dev), glue.to_device(pair[1], wl0.dtype, dev)
        else:  # (a host-only layer keeps the pointers without reading them)
            A_f, B_f = pair[0], pair[1]
        layer.set_vera_shared(A_f, B_f, sum(ranks))
    if any(f is not None and f["R_proj"] is not None for f in fused):
        if any(d % 64 for d in d_outs[:-1]):
            raise ValueError("rotations per projection need q and k widths that are multiples of 64")
        layer.set_projections(np.cumsum(d_outs))
    for t, f in enumerate(fused):
        if f is None:
            continue
        if f["R_proj"] is not None:
            layer.load_proj(t, f["R_proj"], f["blk"], rank=f["rank"], c=1.0, A=f["A"], B=f["B"], s=f["s"],
                            b=f["b"], vd=f["vd"], ve=f["ve"])
        else:
            layer.load(t, "nf", rank=f["rank"], c=1.0, A=f["A"], B=f["B"], s=f["s"], b=f["b"], vd=f["vd"],
                       ve=f["ve"])
    for h in hosts:
        h.layer.close()
    return layer


class QKVFused:
    """q, k and v as one layer over the stacked weights (any method: rotations
    per projection, the projections' VeRA pairs side by side); forward
    returns the three column slices."""

    def __init__(self, wls, tenant_of_token, n_tenants, device=0, flags=0):
        import torch
        from . import workload as glue
        self.d_outs = [wl.d_out for wl, _ in wls]
        wl0 = wls[0][0]
        self.layer = fused_layer(wls, n_tenants, device)
        dev = torch.device("cuda", device)
        W = np.concatenate([wl.W for wl, _ in wls], 0)
        self.x = glue.to_device(wl0.x, wl0.dtype, dev)
        self.W = glue.to_device(W, wl0.dtype, dev)
        self.y = torch.empty((wl0.n, sum(self.d_outs)), dtype=torch.float32, device=dev)
        self.batch = self.layer.plan(np.asarray(tenant_of_token), flags=flags)

    def forward(self):
        self.layer.forward(self.batch, self.x, self.W, self.y)
        offs = np.concatenate([[0], np.cumsum(self.d_outs)])
        return [self.y[:, offs[p]:offs[p + 1]] for p in range(len(self.d_outs))]

    def close(self):
        self.batch.close()
        self.layer.close()


# ---- FFN ---------------------------------------------------------------------------------------

class GatedUp:
    """h = silu(x W_g) (.) up(x): the gate projection (base weight only) and
    the up projection with the tenants' adapters ((IA)^3's l on s)."""

    def __init__(self, wl_up, W_gate, device=0):
        import torch
        from . import workload as glue
        self.up = glue.load(wl_up, device=device)
        gate_wl = dataclasses.replace(wl_up, name=wl_up.name + "_gate", W=W_gate, adapters=[],
                                      token_adapter=np.full(wl_up.n, -1), A_sh=None, B_sh=None)
        self.gate = glue.load(gate_wl, device=device)
        self.h = torch.empty_like(self.up.y)

    def forward(self):
        g, u = self.gate, self.up
        g.layer.forward(g.batch, g.x, g.W, g.y)
        u.layer.forward(u.batch, u.x, u.W, u.y)
        scute.scute_silu_gate(g.y, u.y, self.h)
        return self.h

    def close(self):
        for ld in (self.gate, self.up):
            ld.batch.close()
            ld.layer.close()


# ---- timing ------------------------------------------------------------------------------------

def _time(torch, fn, iters=200, reps=7):
    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / iters)
    return statistics.median(ts)


def qkv_tenants(with_oft: bool, with_vera: bool = False):
    from synth import AdapterSpec
    L, Dr, I3 = AdapterSpec("lora", rank=16), AdapterSpec("dora", rank=16), AdapterSpec("ia3")
    ten = [(L, L, L)] * 8 + [(Dr, Dr, Dr)] * 6 + [(None, I3, I3)] * 6
    if with_oft:
        O = AdapterSpec("oft", blk=32)
        ten = ten[:16] + [(O, O, O)] * 4
    if with_vera:
        V = AdapterSpec("vera")
        ten = ten[:4] + [(V, V, V)] * 4 + ten[8:]
    return ten


def run():
    import torch
    rows = []
    d_in, d_outs, n = 4096, (4096, 1024, 1024), 128
    for with_oft, with_vera in ((False, False), (True, False), (True, True)):
        ten = qkv_tenants(with_oft, with_vera)
        wls, tt = projection_workloads(ten, n, d_in, d_outs, seed=11, vera_rank=256 if with_vera else 0)
        sp = QKVSplit(wls)
        t_split = _time(torch, sp.forward)
        sp.close()
        name = "lora+dora+ia3(k,v)" + ("+oft" if with_oft else "") + ("+vera" if with_vera else "")
        rows.append({"layer": "qkv", "tenants": name, "route": "split", "us": t_split})
        fu = QKVFused(wls, tt, len(ten))
        t_fused = _time(torch, fu.forward)
        fu.close()
        rows.append({"layer": "qkv", "tenants": name, "route": "fused", "us": t_fused})
        print(f"multiproj: {rows[-1]}", file=sys.stderr, flush=True)
    # prefill: 2048 tokens with the OFT tenants (the fused layer takes the
    # prefill path, its projections ending on 256-column tiles)
    wls, tt = projection_workloads(qkv_tenants(True), 2048, d_in, d_outs, seed=12)
    sp = QKVSplit(wls)
    t_split = _time(torch, sp.forward, iters=50)
    sp.close()
    fu = QKVFused(wls, tt, len(qkv_tenants(True)))
    t_fused = _time(torch, fu.forward, iters=50)
    fu.close()
    name = "lora+dora+ia3(k,v)+oft, 2048 tok"
    rows += [{"layer": "qkv", "tenants": name, "route": "split", "us": t_split},
             {"layer": "qkv", "tenants": name, "route": "fused", "us": t_fused}]
    print(f"multiproj: {rows[-1]}", file=sys.stderr, flush=True)
    from synth import make_config
    up = make_config(3)  # FFN up 4096 -> 14336, 256 tokens, (IA)^3 + VeRA tenants
    Wg = np.random.default_rng(5).normal(0.0, 1.0 / np.sqrt(up.d_in), size=up.W.shape)
    gu = GatedUp(up, Wg)
    t_gated = _time(torch, gu.forward)
    t_up = _time(torch, lambda: gu.up.layer.forward(gu.up.batch, gu.up.x, gu.up.W, gu.up.y))
    gu.close()
    rows.append({"layer": "ffn_up_gated", "tenants": up.name, "route": "gate + up + silu_gate", "us": t_gated})
    rows.append({"layer": "ffn_up_gated", "tenants": up.name, "route": "up only", "us": t_up})
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    rows = run()
    if a.out:
        with open(a.out, "w") as f:
            json.dump(rows, f, indent=1)
    print("| layer | tenants | route | µs / forward |\n|---|---|---|---|")
    for r in rows:
        print(f"| {r['layer']} | {r['tenants']} | {r['route']} | {r['us']:.2f} |")


if __name__ == "__main__":
    main()
