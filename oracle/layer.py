"""Plain fp64 evaluation of each adapter method from its own definition.

TEST INFRASTRUCTURE ONLY (see the package docstring). Slow and direct on
purpose: no blocking, no fusion, no reordering beyond what each definition
states. Library primitives used as steps: ``numpy.matmul`` and
``numpy.linalg.solve``.

Conventions. The pages write the layer with row vectors, x W, where
x is 1 x d_in and W is d_in x d_out. The synthetic buffers use the
PyTorch nn.Linear layout (W stored [d_out][d_in], A [r][d_in], B [d_out][r],
A_sh [r_v][d_in], B_sh [d_out][r_v]); this module transposes them into the
pages' orientation first (``Wf = W.T`` and so on) and then writes every
formula exactly as the pages do.

Readings taken where the pages leave a step open:
  * OFT: the pages name the rotation block-diagonal and nothing more; the
    rotation of each block is the Cayley transform R = (I + Q)(I - Q)^-1 of the adapter's
    skew-symmetric block Q, applied as x R (row vector).
  * DoRA: every column of W + cAB is brought to its learned length m, i.e.
    W_D = (W + cAB) diag(m / colnorm(W + cAB)), column norms over d_in.
  * VeRA: c = 1; d sits between the shared A and B, e after B.
  * Tokens with adapter id -1 take the base path only.
"""

from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np


# --------------------------------------------------------------------------
# OFT rotation ("What problem is it solving?": an OFT adapter rotates the
# layer's input; "Where is the cheapest place...": a kernel ahead of the GEMM
# applies each row's own block-diagonal matrix)
# --------------------------------------------------------------------------

def cayley(Q: np.ndarray) -> np.ndarray:
    """Cayley transform of one skew-symmetric block: R = (I + Q)(I - Q)^-1.

    (I + Q) and (I - Q)^-1 commute, so R also equals (I - Q)^-1 (I + Q),
    which is what one linear solve returns.
    """
    Q = np.asarray(Q, dtype=np.float64)
    eye = np.eye(Q.shape[0])
    return np.linalg.solve(eye - Q, eye + Q)


def oft_rotation(Qblocks: np.ndarray) -> np.ndarray:
    """Dense block-diagonal R (d_in x d_in) with one Cayley block per Q block."""
    nb, blk, _ = Qblocks.shape
    R = np.zeros((nb * blk, nb * blk))
    for kb in range(nb):
        R[kb * blk:(kb + 1) * blk, kb * blk:(kb + 1) * blk] = cayley(Qblocks[kb])
    return R


def explicit_rotation(Rblocks: np.ndarray) -> np.ndarray:
    """Dense block-diagonal matrix from explicit blocks (normal-form R slot)."""
    nb, blk, _ = Rblocks.shape
    R = np.zeros((nb * blk, nb * blk))
    for kb in range(nb):
        R[kb * blk:(kb + 1) * blk, kb * blk:(kb + 1) * blk] = Rblocks[kb]
    return R


# --------------------------------------------------------------------------
# DoRA ("What problem is it solving?": each output column of the adapted
# weight gets a learned length; "Which slots can be merged at load?" and "How does Scute
# plug into vLLM?": s = learned length / norm of each column of W + cAB)
# --------------------------------------------------------------------------

def dora_weight(Wf: np.ndarray, Af: np.ndarray, Bf: np.ndarray, c: float,
                m: np.ndarray) -> np.ndarray:
    """W_D = (W + cAB) with column j rescaled to length m_j (pages' orientation)."""
    Wplus = Wf + c * (Af @ Bf)
    colnorm = np.sqrt(np.sum(Wplus * Wplus, axis=0))
    return Wplus * (m / colnorm)[None, :]


# --------------------------------------------------------------------------
# per-method outputs for the rows of one adapter
# --------------------------------------------------------------------------

def _bias(a, d_out):
    return np.zeros(d_out) if getattr(a, "b", None) is None else a.b


def method_output(wl, a, xs: np.ndarray, hs: np.ndarray) -> np.ndarray:
    """Output rows of adapter ``a`` for input rows ``xs`` by its own definition.

    ``hs`` = xs W (the base product, shared by every method that applies W
    to the unrotated input).
    """
    Wf = wl.W.T
    d_out = wl.d_out
    b = _bias(a, d_out)
    meth = a.method
    if meth == "lora":
        # batched LoRA ("The big picture"): h = xW, shrink by A, expand by B
        Af, Bf = a.A.T, a.B.T
        return hs + b + a.c * ((xs @ Af) @ Bf)
    if meth == "dora":
        Af, Bf = a.A.T, a.B.T
        return xs @ dora_weight(Wf, Af, Bf, a.c, a.m) + b
    if meth == "ia3":
        # (IA)^3 on the up projection: the output of x W_u is scaled by l
        return hs * a.l[None, :] + b
    if meth == "vera":
        # shared A/B, per-adapter d between them and e after B
        Ash, Bsh = wl.A_sh.T, wl.B_sh.T
        return hs + b + (((xs @ Ash) * a.vd[None, :]) @ Bsh) * a.ve[None, :]
    if meth == "oft":
        R = oft_rotation(a.Q)
        return (xs @ R) @ Wf + b
    if meth == "nf":
        return normal_form_output(xs, Wf, nf_slots(wl, a))
    raise ValueError(f"unknown method {meth}")


def base_output(wl) -> np.ndarray:
    """xW for every token, no adapter (b = 0 for tokens without adapter)."""
    return wl.x @ wl.W.T


def forward(wl) -> np.ndarray:
    """y for the whole batch: each token by the definition of its adapter."""
    h = base_output(wl)
    y = h.copy()
    by_id = wl.adapter_by_id()
    ta = np.asarray(wl.token_adapter)
    for aid in sorted(set(int(v) for v in ta if v >= 0)):
        rows = np.nonzero(ta == aid)[0]
        y[rows] = method_output(wl, by_id[aid], wl.x[rows], h[rows])
    return y


# --------------------------------------------------------------------------
# The normal form ("The big picture": F_a(x) = ((xR)W) (.) s + b
#   + sum_k c_k (((x A_k) (.) d_k) B_k (.) e_k), unused slots hold the identity)
# --------------------------------------------------------------------------

def nf_slots(wl, a) -> Dict:
    """Slots of adapter ``a`` in the normal form, before any folding.

    Returns {"R": d_in x d_in or None, "s", "b": d_out or None,
             "terms": [{"A": d_in x r, "B": r x d_out, "c", "d": r or None,
                        "e": d_out or None, "shared": bool}]}.
    None means the identity value of that slot.
    """
    Wf = wl.W.T
    sl = {"R": None, "s": None, "b": getattr(a, "b", None), "terms": []}
    meth = a.method
    if meth == "lora":
        sl["terms"].append(dict(A=a.A.T, B=a.B.T, c=a.c, d=None, e=None, shared=False))
    elif meth == "dora":
        # the rescale factor multiplies the base path (s) and, identically,
        # the low-rank path (e)
        Wplus = Wf + a.c * (a.A.T @ a.B.T)
        s = a.m / np.sqrt(np.sum(Wplus * Wplus, axis=0))
        sl["s"] = s
        sl["terms"].append(dict(A=a.A.T, B=a.B.T, c=a.c, d=None, e=s, shared=False))
    elif meth == "ia3":
        sl["s"] = a.l
    elif meth == "vera":
        sl["terms"].append(dict(A=wl.A_sh.T, B=wl.B_sh.T, c=a.c, d=a.vd, e=a.ve, shared=True))
    elif meth == "oft":
        sl["R"] = oft_rotation(a.Q)
    elif meth == "nf":
        if a.R is not None:
            sl["R"] = explicit_rotation(a.R)
        sl["s"] = a.s
        if a.A is not None:
            sl["terms"].append(dict(A=a.A.T, B=a.B.T, c=a.c, d=a.d, e=a.e, shared=False))
        if a.vd is not None:
            sl["terms"].append(dict(A=wl.A_sh.T, B=wl.B_sh.T, c=1.0, d=a.vd, e=a.ve,
                                    shared=True))
    else:
        raise ValueError(f"unknown method {meth}")
    return sl


def fold_slots(sl: Dict) -> Dict:
    """Fold rule ("Which slots can be merged at load?"): a slot next to a
    factor the adapter owns merges into it; a slot whose neighbours are all
    shared stays live.

    Owned term: A' = c A diag(d), B' = B diag(e), and c, d, e become identity.
    Shared term (VeRA): A and B are shared, so d and e stay live; the scalar c
    merges into the adapter's own live vector e.
    R, s and b sit next to the shared W only and stay live.
    """
    out = {"R": sl["R"], "s": sl["s"], "b": sl["b"], "terms": []}
    for t in sl["terms"]:
        r = t["A"].shape[1]
        d = np.ones(r) if t["d"] is None else t["d"]
        e = np.ones(t["B"].shape[1]) if t["e"] is None else t["e"]
        if t["shared"]:
            out["terms"].append(dict(A=t["A"], B=t["B"], c=1.0, d=d, e=t["c"] * e, shared=True))
        else:
            out["terms"].append(dict(A=t["c"] * t["A"] * d[None, :], B=t["B"] * e[None, :],
                                     c=1.0, d=None, e=None, shared=False))
    return out


def normal_form_output(xs: np.ndarray, Wf: np.ndarray, sl: Dict) -> np.ndarray:
    """Evaluate the normal form for rows ``xs`` from slots ``sl``."""
    d_out = Wf.shape[1]
    xr = xs if sl["R"] is None else xs @ sl["R"]
    y = xr @ Wf
    if sl["s"] is not None:
        y = y * sl["s"][None, :]
    if sl["b"] is not None:
        y = y + sl["b"][None, :]
    for t in sl["terms"]:
        u = xs @ t["A"]                       # the low-rank path sees unrotated x
        if t["d"] is not None:
            u = u * t["d"][None, :]
        v = u @ t["B"]
        if t["e"] is not None:
            v = v * t["e"][None, :]
        y = y + t["c"] * v
    assert y.shape[1] == d_out
    return y


def forward_normal_form(wl, fold: bool = False) -> np.ndarray:
    """Whole batch through the normal form (slots unfolded or folded)."""
    Wf = wl.W.T
    ta = np.asarray(wl.token_adapter)
    y = wl.x @ Wf
    by_id = wl.adapter_by_id()
    for aid in sorted(set(int(v) for v in ta if v >= 0)):
        rows = np.nonzero(ta == aid)[0]
        sl = nf_slots(wl, by_id[aid])
        if fold:
            sl = fold_slots(sl)
        y[rows] = normal_form_output(wl.x[rows], Wf, sl)
    return y
