"""Seeded synthetic workloads (inputs only, no layer arithmetic).

Every array is drawn with numpy's PCG64 from one seed in a fixed order:
x, W, the shared VeRA pair (if the workload has VeRA adapters), then each
adapter in id order with its tensors in the order listed in ``_draw_adapter``,
then the token-to-adapter assignment. Values are rounded to the workload's
storage precision (bf16 round-to-nearest-even, or fp32) and returned as
float64 arrays holding exactly those rounded values, so every consumer sees
identical numbers.

Buffer layouts (PyTorch ``nn.Linear`` convention, not the pages' row-vector
formula, which uses the transposes):
  x      [n][d_in]           W      [d_out][d_in]
  A      [rank][d_in]        B      [d_out][rank]
  A_sh   [r_v][d_in]         B_sh   [d_out][r_v]
  Q, R   [d_in/blk][blk][blk]   (row-vector blocks: out_j = sum_i in_i * M[i][j])

Distributions follow the tiny fp32 workload's recipe with every 1/256
variance replaced by 1/d_in: x ~ N(0,1); W, A, A_sh, B_sh ~ N(0, 1/d_in);
B ~ N(0, 0.02^2); LoRA/DoRA c = 2; (IA)^3 l = 1 + N(0, 0.1^2); VeRA
d, e ~ N(0, 0.1^2); OFT skew blocks with strict-upper entries N(0, 0.01^2);
DoRA magnitude m = colnorm(W + cAB) * (1 + N(0, 0.05^2)); b = 0.

The DoRA magnitude is the one drawn input that depends on other inputs:
it is defined relative to the column norms of W + cAB so that DoRA's
rescale factor lands near 1 + N(0, 0.05^2).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

METHODS = ("lora", "dora", "ia3", "vera", "oft", "nf")


# --------------------------------------------------------------------------
# rounding helpers (storage precision of the generated values)
# --------------------------------------------------------------------------

def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even).

    bf16 keeps 7 explicit mantissa bits; a float64 keeps 52. Rounding drops
    the low 45 bits of the float64 pattern with round-half-to-even, which is
    exact for every value inside bf16's normal range. Values are returned as
    float64 (exactly representable in bf16).
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + (np.uint64((1 << 44) - 1) + lsb)) & np.uint64(~((1 << 45) - 1) & 0xFFFFFFFFFFFFFFFF)
    return bits.view(np.float64)


def round_f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(a) -> np.ndarray:
    """uint16 bit patterns of values that are already exactly bf16."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("bf16_bits: input is not exactly representable in bf16")
    return (bits >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# specs
# --------------------------------------------------------------------------

@dataclass
class AdapterSpec:
    method: str
    rank: int = 0          # own low-rank term rank (lora, dora, nf term)
    blk: int = 0           # OFT / nf rotation block size
    c: float = 2.0         # scalar c of the own term
    # normal-form adapters: which slots to fill
    nf_R: bool = False
    nf_s: bool = False
    nf_b: bool = False
    nf_term: bool = False
    nf_vera: bool = False
    bias: bool = False     # draw a nonzero b for any method


@dataclass
class WorkloadSpec:
    name: str
    dtype: str             # "f32" or "bf16"
    d_in: int
    d_out: int
    n: int
    adapters: List[AdapterSpec]
    vera_rank: int = 0     # r_v of the shared VeRA pair (0: none)
    assign: str = "uniform"   # c0 | composition | uniform | blocks | explicit
    token_adapter: Optional[Sequence[int]] = None  # for assign == "explicit"
    seed: int = 0
    # distribution knobs (defaults are the tiny-workload recipe)
    sigma_l: float = 0.1
    sigma_m: float = 0.05
    sigma_vd: float = 0.1
    sigma_ve: float = 0.1
    sigma_q: float = 0.01
    sigma_B: float = 0.02
    sigma_b: float = 0.1


@dataclass
class Adapter:
    id: int
    method: str
    rank: int = 0
    blk: int = 0
    c: float = 1.0
    A: Optional[np.ndarray] = None   # [rank][d_in]
    B: Optional[np.ndarray] = None   # [d_out][rank]
    m: Optional[np.ndarray] = None   # [d_out]   DoRA magnitude
    l: Optional[np.ndarray] = None   # [d_out]   (IA)^3 vector
    vd: Optional[np.ndarray] = None  # [r_v]     VeRA d
    ve: Optional[np.ndarray] = None  # [d_out]   VeRA e
    Q: Optional[np.ndarray] = None   # [nb][blk][blk] OFT skew blocks
    # explicit normal-form slots (method == "nf")
    R: Optional[np.ndarray] = None   # [nb][blk][blk]
    s: Optional[np.ndarray] = None   # [d_out]
    b: Optional[np.ndarray] = None   # [d_out]
    d: Optional[np.ndarray] = None   # [rank]   own-term d
    e: Optional[np.ndarray] = None   # [d_out]  own-term e


@dataclass
class Workload:
    name: str
    dtype: str
    d_in: int
    d_out: int
    n: int
    x: np.ndarray                 # [n][d_in]
    W: np.ndarray                 # [d_out][d_in]
    adapters: List[Adapter]
    token_adapter: np.ndarray     # int32 [n], -1 = base only
    A_sh: Optional[np.ndarray] = None  # [r_v][d_in]
    B_sh: Optional[np.ndarray] = None  # [d_out][r_v]
    seed: int = 0

    @property
    def vera_rank(self) -> int:
        return 0 if self.A_sh is None else int(self.A_sh.shape[0])

    def adapter_by_id(self):
        return {a.id: a for a in self.adapters}


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------

def _skew_blocks(rng, nb, blk, sigma):
    """Skew-symmetric blocks: strict-upper entries N(0, sigma^2), Q_ji = -Q_ij."""
    Q = np.zeros((nb, blk, blk))
    iu = np.triu_indices(blk, k=1)
    for kb in range(nb):
        q = rng.normal(0.0, sigma, size=len(iu[0]))
        Q[kb][iu] = q
        Q[kb][(iu[1], iu[0])] = -q
    return Q


def _draw_adapter(rng, aid, spec: AdapterSpec, ws: WorkloadSpec, W, rnd):
    d_in, d_out = ws.d_in, ws.d_out
    a = Adapter(id=aid, method=spec.method, rank=spec.rank, blk=spec.blk, c=spec.c)
    meth = spec.method
    sd_in = 1.0 / np.sqrt(d_in)
    if meth in ("lora", "dora"):
        a.A = rnd(rng.normal(0.0, sd_in, size=(spec.rank, d_in)))
        a.B = rnd(rng.normal(0.0, ws.sigma_B, size=(d_out, spec.rank)))
        if meth == "dora":
            # magnitude drawn relative to the column norms of W + cAB
            # (output column j of the row-vector formula = buffer row j)
            wplus = W + spec.c * (a.B @ a.A)
            cn = np.sqrt(np.sum(wplus * wplus, axis=1))
            a.m = rnd(cn * (1.0 + rng.normal(0.0, ws.sigma_m, size=d_out)))
    elif meth == "ia3":
        a.l = rnd(1.0 + rng.normal(0.0, ws.sigma_l, size=d_out))
        a.c = 1.0
    elif meth == "vera":
        a.vd = rnd(rng.normal(0.0, ws.sigma_vd, size=ws.vera_rank))
        a.ve = rnd(rng.normal(0.0, ws.sigma_ve, size=d_out))
        a.c = 1.0
    elif meth == "oft":
        if spec.blk <= 0 or d_in % spec.blk:
            raise ValueError("OFT block size must divide d_in")
        a.Q = rnd(_skew_blocks(rng, d_in // spec.blk, spec.blk, ws.sigma_q))
        a.c = 1.0
    elif meth == "nf":
        if spec.nf_R:
            nb = d_in // spec.blk
            a.R = rnd(np.eye(spec.blk)[None, :, :]
                      + rng.normal(0.0, ws.sigma_q, size=(nb, spec.blk, spec.blk)))
        if spec.nf_s:
            a.s = rnd(1.0 + rng.normal(0.0, ws.sigma_l, size=d_out))
        if spec.nf_term:
            a.A = rnd(rng.normal(0.0, sd_in, size=(spec.rank, d_in)))
            a.B = rnd(rng.normal(0.0, ws.sigma_B, size=(d_out, spec.rank)))
            a.d = rnd(1.0 + rng.normal(0.0, ws.sigma_l, size=spec.rank))
            a.e = rnd(1.0 + rng.normal(0.0, ws.sigma_l, size=d_out))
        else:
            a.rank = 0
        if spec.nf_vera:
            a.vd = rnd(rng.normal(0.0, ws.sigma_vd, size=ws.vera_rank))
            a.ve = rnd(rng.normal(0.0, ws.sigma_ve, size=d_out))
    else:
        raise ValueError(f"unknown method {meth}")
    if spec.bias or (meth == "nf" and spec.nf_b):
        a.b = rnd(rng.normal(0.0, ws.sigma_b, size=d_out))
    return a


def _assign(rng, ws: WorkloadSpec, ids: List[int]) -> np.ndarray:
    n, k = ws.n, len(ids)
    if ws.assign == "explicit":
        ta = np.asarray(ws.token_adapter, dtype=np.int32)
        if ta.shape != (n,):
            raise ValueError("explicit token_adapter must have n entries")
        return ta
    if ws.assign == "uniform":
        return np.asarray(ids, dtype=np.int32)[rng.integers(0, k, size=n)]
    if ws.assign == "c0":
        # k contiguous segments of floor(n/k) tokens; the n mod k extra tokens
        # go to seeded distinct segments; segments in adapter-id order
        lens = np.full(k, n // k, dtype=np.int64)
        extra = rng.choice(k, size=n - int(lens.sum()), replace=False)
        lens[extra] += 1
    elif ws.assign == "composition":
        # uniformly random composition of n into k positive parts
        cuts = np.sort(rng.choice(np.arange(1, n), size=k - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [n]]))
    elif ws.assign == "blocks":
        if n % k:
            raise ValueError("blocks assignment needs n divisible by #adapters")
        lens = np.full(k, n // k, dtype=np.int64)
    else:
        raise ValueError(f"unknown assignment {ws.assign}")
    return np.repeat(np.asarray(ids, dtype=np.int32), lens).astype(np.int32)


def make_workload(ws: WorkloadSpec) -> Workload:
    if ws.dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be f32 or bf16")
    rnd = round_bf16 if ws.dtype == "bf16" else round_f32
    rng = np.random.Generator(np.random.PCG64(ws.seed))
    sd_in = 1.0 / np.sqrt(ws.d_in)
    x = rnd(rng.normal(0.0, 1.0, size=(ws.n, ws.d_in)))
    W = rnd(rng.normal(0.0, sd_in, size=(ws.d_out, ws.d_in)))
    A_sh = B_sh = None
    if ws.vera_rank > 0:
        A_sh = rnd(rng.normal(0.0, sd_in, size=(ws.vera_rank, ws.d_in)))
        B_sh = rnd(rng.normal(0.0, sd_in, size=(ws.d_out, ws.vera_rank)))
    adapters = [_draw_adapter(rng, i, s, ws, W, rnd) for i, s in enumerate(ws.adapters)]
    ids = [a.id for a in adapters]
    ta = _assign(rng, ws, ids) if ids or ws.assign == "explicit" else np.full(ws.n, -1, np.int32)
    return Workload(name=ws.name, dtype=ws.dtype, d_in=ws.d_in, d_out=ws.d_out, n=ws.n,
                    x=x, W=W, adapters=adapters, token_adapter=ta,
                    A_sh=A_sh, B_sh=B_sh, seed=ws.seed)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

CONFIG_NAMES = (
    "tiny_f32_256x256_16tok_5methods",
    "lora_bf16_4096x4096_128tok_64xr16",
    "mixed_bf16_4096x4096_128tok_40adapters",
    "ffnup_bf16_4096x14336_256tok_1024ia3_1024vera",
    "prefill_bf16_4096x4096_2048tok_16seg",
)


def config_spec(idx: int, seed: Optional[int] = None) -> WorkloadSpec:
    seed = 1000 + idx if seed is None else seed
    name = CONFIG_NAMES[idx]
    if idx == 0:
        ads = [AdapterSpec("lora", rank=8, c=2.0), AdapterSpec("dora", rank=8, c=2.0),
               AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=32)]
        return WorkloadSpec(name, "f32", 256, 256, 16, ads, vera_rank=32, assign="c0", seed=seed)
    if idx == 1:
        ads = [AdapterSpec("lora", rank=16, c=2.0) for _ in range(64)]
        return WorkloadSpec(name, "bf16", 4096, 4096, 128, ads, assign="composition", seed=seed)
    if idx == 2:
        ads = ([AdapterSpec("lora", rank=16, c=2.0) for _ in range(8)]
               + [AdapterSpec("dora", rank=16, c=2.0) for _ in range(8)]
               + [AdapterSpec("ia3") for _ in range(8)]
               + [AdapterSpec("vera") for _ in range(8)]
               + [AdapterSpec("oft", blk=32) for _ in range(8)])
        return WorkloadSpec(name, "bf16", 4096, 4096, 128, ads, vera_rank=256,
                            assign="uniform", seed=seed)
    if idx == 3:
        ads = [AdapterSpec("ia3") for _ in range(1024)] + [AdapterSpec("vera") for _ in range(1024)]
        return WorkloadSpec(name, "bf16", 4096, 14336, 256, ads, vera_rank=256,
                            assign="uniform", seed=seed)
    if idx == 4:
        cycle = [AdapterSpec("lora", rank=64, c=2.0), AdapterSpec("dora", rank=64, c=2.0),
                 AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=64)]
        ads = [dataclasses.replace(cycle[k % 5]) for k in range(16)]
        return WorkloadSpec(name, "bf16", 4096, 4096, 2048, ads, vera_rank=256,
                            assign="blocks", seed=seed)
    raise ValueError("config index must be 0..4")


def make_config(idx: int, seed: Optional[int] = None) -> Workload:
    return make_workload(config_spec(idx, seed))
