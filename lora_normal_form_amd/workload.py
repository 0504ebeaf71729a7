"""Load a synthetic workload (``synth.Workload``) into a library layer.

Marshalling only: copies the workload's arrays to device memory with torch
and hands each adapter's parameters to ``scute_load_adapter``, which does
the fold. Used by the tests, the smoke check and the benchmark.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import scute


def to_device(arr: np.ndarray, dtype: str, device):
    """Exactly-rounded float64 array -> torch tensor in the activation dtype."""
    import torch
    if dtype == "bf16":
        f = np.ascontiguousarray(arr, dtype=np.float64).astype(np.float32)
        bits = (f.view(np.uint32) >> 16).astype(np.uint16)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device) if device is not None else t


def adapter_arrays(wl, a):
    """Keyword arguments of ``Layer.load`` for one synthetic adapter."""
    m = a.method
    kw = dict(method=m, rank=a.rank, blk=a.blk, c=a.c, b=a.b)
    if m in ("lora", "dora"):
        kw.update(A=a.A, B=a.B)
        if m == "dora":
            kw.update(m=a.m, W_host=wl.W)
    elif m == "ia3":
        kw.update(l=a.l)
    elif m == "vera":
        kw.update(vd=a.vd, ve=a.ve)
    elif m == "oft":
        kw.update(Q=a.Q)
    elif m == "nf":
        kw.update(A=a.A, B=a.B, d=a.d, e=a.e, R=a.R, s=a.s, vd=a.vd, ve=a.ve)
        if a.A is None:
            kw["rank"] = 0
    return kw


@dataclass
class Loaded:
    layer: scute.Layer
    batch: scute.Batch
    x: object       # device tensor [n][d_in]
    W: object       # device tensor [d_out][d_in]
    y: object       # device float32 tensor [n][d_out]
    A_sh: Optional[object] = None
    B_sh: Optional[object] = None


def load(wl, device=0, max_adapters: Optional[int] = None, plan: bool = True,
         shared=None, deterministic: bool = False, flags: int = 0) -> Loaded:
    """Create a layer on ``device``, load every adapter, plan the batch.

    ``shared``: optional (x, W, A_sh, B_sh) device tensors to reuse instead of
    uploading new copies. ``deterministic``: plan with bit-repeatable
    forwards (SCUTE_PLAN_DETERMINISTIC); ``flags``: other scute_plan_flag bits.
    """
    import torch
    dev = torch.device("cuda", device) if device >= 0 else None
    L = scute.Layer(wl.d_in, wl.d_out, wl.dtype, max_adapters or max(1, len(wl.adapters)),
                    device=device)
    if shared is not None:
        x, W, A_sh, B_sh = shared
    else:
        x = to_device(wl.x, wl.dtype, dev)
        W = to_device(wl.W, wl.dtype, dev)
        A_sh = B_sh = None
        if wl.A_sh is not None:
            A_sh = to_device(wl.A_sh, wl.dtype, dev)
            B_sh = to_device(wl.B_sh, wl.dtype, dev)
    if A_sh is not None:
        L.set_vera_shared(A_sh, B_sh, wl.vera_rank)
    for a in wl.adapters:
        kw = adapter_arrays(wl, a)
        L.load(a.id, **kw)
    y = torch.empty((wl.n, wl.d_out), dtype=torch.float32, device=dev)
    B = L.plan(wl.token_adapter, deterministic=deterministic, flags=flags) if plan else None
    return Loaded(L, B, x, W, y, A_sh, B_sh)
