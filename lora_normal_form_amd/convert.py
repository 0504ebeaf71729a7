"""Conversion of a loaded adapter to a plain LoRA adapter by truncated SVD.

This is the baseline the pages argue against ("Which slots can be merged at
load?" and "Does it actually work better?", paper-daily.com explainer of
"Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA"): an engine
that only serves LoRA converts every other method by a truncated SVD of its
weight change, at rank 64 (or 256 for VeRA, whose shared pair has rank 256),
and runs every adapter at the pool's largest rank. Here it is used to build
the converted workloads that the exact path is compared with.

The weight change of an adapter, as the library stores it after the fold
(slots read back with scute_read_slot), in the orientation y_delta = x dM
(dM is [d_in][d_out]):

    base path   ((x R) W^T) (.) s - x W^T  ->  dM = (R - I) W^T diag(s) + W^T diag(s - 1)
    own term    (x A'^T) B'^T              ->  dM = A'^T B'^T
    VeRA term   ((x A_sh^T) (.) d) B_sh^T (.) e  ->  dM = A_sh^T diag(d) B_sh^T diag(e)

(R is block diagonal; s, R default to ones / identity when the adapter has
no such slot). The shift b is not a matrix and carries over as the LoRA's b.
The rank-r LoRA is A = (U_r S_r)^T ([r][d_in]), B = V_r ([d_out][r]), c = 1,
from dM = U S V^T; by Eckart-Young it is the best rank-r approximation of dM
in the Frobenius norm.
"""

from __future__ import annotations

import numpy as np

from . import scute


def slots(layer, aid: int, d_in: int, d_out: int, r_v: int = 0):
    """The loaded adapter's live slots as float64 arrays (None where absent)."""
    info = layer.info(aid)
    dt = "bf16" if layer.act == scute.BF16 else np.float32
    out = {"R_minus_I": None, "s": None, "b": None, "A": None, "B": None, "vd": None, "ve": None,
           "blk": info["blk"]}
    if info["has_R"]:
        blk = info["blk"]
        out["R_minus_I"] = layer.read_slot(aid, scute.SLOT_P, (d_in // blk, blk, blk), dt).astype(np.float64)
    if info["has_s"]:
        out["s"] = layer.read_slot(aid, scute.SLOT_S, (d_out,), np.float32).astype(np.float64)
    if info["has_b"]:
        out["b"] = layer.read_slot(aid, scute.SLOT_BIAS, (d_out,), np.float32).astype(np.float64)
    if info["has_term"]:
        r = info["rank"]
        out["A"] = layer.read_slot(aid, scute.SLOT_A, (r, d_in), dt).astype(np.float64)
        out["B"] = layer.read_slot(aid, scute.SLOT_B, (d_out, r), dt).astype(np.float64)
    if info["has_vera"]:
        out["vd"] = layer.read_slot(aid, scute.SLOT_VD, (r_v,), np.float32).astype(np.float64)
        out["ve"] = layer.read_slot(aid, scute.SLOT_VE, (d_out,), np.float32).astype(np.float64)
    return out


def weight_change(sl, W, A_sh=None, B_sh=None, parts: bool = False):
    """dM [d_in][d_out] of the slots (W [d_out][d_in], A_sh [r_v][d_in],
    B_sh [d_out][r_v]); with parts, the VeRA term comes back as its two
    factors (P, Q with dM_vera = P Q^T) instead of being added in."""
    Wt = np.asarray(W, np.float64).T  # [d_in][d_out]
    d_in, d_out = Wt.shape
    dM = np.zeros((d_in, d_out))
    s = sl["s"]
    if sl["R_minus_I"] is not None:
        P = sl["R_minus_I"]
        blk = P.shape[1]
        for kb in range(P.shape[0]):
            dM[kb * blk:(kb + 1) * blk] += P[kb] @ Wt[kb * blk:(kb + 1) * blk]
        if s is not None:
            dM *= s[None, :]
    if s is not None:
        dM += Wt * (s - 1.0)[None, :]
    if sl["A"] is not None:
        dM += sl["A"].T @ sl["B"].T
    vera = None
    if sl["vd"] is not None:
        Pv = np.asarray(A_sh, np.float64).T * sl["vd"][None, :]          # [d_in][r_v]
        Qv = np.asarray(B_sh, np.float64) * sl["ve"][:, None]            # [d_out][r_v]
        if parts:
            vera = (Pv, Qv)
        else:
            dM += Pv @ Qv.T
    return (dM, vera) if parts else dM


def truncated_svd(M, r: int, exact_below: int = 1536, power_iters: int = 3, oversample: int = 16,
                  seed: int = 0):
    """(U_r S_r, V_r) of M. Exact (LAPACK) when min(M.shape) <= exact_below,
    else randomized range finding with power iterations (Halko, Martinsson
    and Tropp 2011), which is exact to rounding when rank(M) <= r +
    oversample and near-optimal otherwise."""
    M = np.asarray(M, np.float64)
    m, n = M.shape
    r = min(r, m, n)
    if min(m, n) <= exact_below:
        U, S, Vt = np.linalg.svd(M, full_matrices=False)
        return U[:, :r] * S[None, :r], Vt[:r].T
    rng = np.random.default_rng(seed)
    k = min(r + oversample, m, n)
    Y = M @ rng.standard_normal((n, k))
    Qy, _ = np.linalg.qr(Y)
    for _ in range(power_iters):
        Z, _ = np.linalg.qr(M.T @ Qy)
        Qy, _ = np.linalg.qr(M @ Z)
    Bs = Qy.T @ M                                     # [k][n]
    Ub, S, Vt = np.linalg.svd(Bs, full_matrices=False)
    U = Qy @ Ub
    return U[:, :r] * S[None, :r], Vt[:r].T


def factored_svd(P, Q, r: int):
    """(U_r S_r, V_r) of P Q^T from its factors (P [m][k], Q [n][k]) through
    two thin QRs: exact for any k."""
    Qp, Rp = np.linalg.qr(np.asarray(P, np.float64))
    Qq, Rq = np.linalg.qr(np.asarray(Q, np.float64))
    Us, S, Vt = np.linalg.svd(Rp @ Rq.T)
    r = min(r, len(S))
    return (Qp @ Us[:, :r]) * S[None, :r], Qq @ Vt[:r].T


def to_lora(sl, W, A_sh, B_sh, rank: int, seed: int = 0):
    """The rank-`rank` LoRA of the adapter: (A [rank][d_in], B [d_out][rank],
    b or None, relative Frobenius error of the truncated weight change)."""
    dM, vera = weight_change(sl, W, A_sh, B_sh, parts=True)
    if vera is not None and not np.any(dM):
        US, V = factored_svd(vera[0], vera[1], rank)  # VeRA alone: rank <= r_v
        ref = vera[0] @ vera[1].T
    else:
        if vera is not None:
            dM = dM + vera[0] @ vera[1].T
        US, V = truncated_svd(dM, rank, seed=seed)
        ref = dM
    nrm = np.linalg.norm(ref)
    err = float(np.linalg.norm(ref - US @ V.T) / nrm) if nrm > 0 else 0.0
    return US.T.copy(), V.copy(), sl["b"], err
