"""Parity criteria against the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Two criteria:
  * max error: max |y - ref| <= tol * max |ref| over the whole output
    (tol = 1e-4 for fp32 workloads, 1e-2 for bf16-in / fp32-accumulate);
  * adapter-effect error (the evaluation section of the paper-daily page
    measures error as a share of how much each adapter changes the output):
    for every adapter a with tokens T_a,
        E_a = sum_{t in T_a, j} |y - ref| / sum_{t in T_a, j} |ref - base|,
    with base = x W from the same inputs (the shift b is one of the
    adapter's slots, so it counts as part of its effect); E_a <= 1% for bf16
    workloads.
    An adapter whose effect is exactly zero has no E_a (the ratio is
    undefined): it is reported with E_a = nan and left to the max-error
    criterion, which covers every output element.

The thresholds are fixed here and nowhere else: tol = 1e-4 (fp32) or 1e-2
(bf16) on the max error, compared with <=; E_a <= 0.01 for bf16 workloads.
"""

from __future__ import annotations

from typing import Dict

import numpy as np


def effect_errors(y, ref, base, token_adapter) -> Dict[int, float]:
    y = np.asarray(y, dtype=np.float64)
    ta = np.asarray(token_adapter)
    out = {}
    for aid in sorted(set(int(v) for v in ta if v >= 0)):
        rows = ta == aid
        eff = np.sum(np.abs(ref[rows] - base[rows]))
        err = np.sum(np.abs(y[rows] - ref[rows]))
        out[aid] = float("nan") if eff == 0.0 else float(err / eff)
    return out


def max_error_ok(y, ref, tol):
    y = np.asarray(y, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    return err <= tol * scale, err, scale


def check(y, ref, base, token_adapter, dtype: str):
    """Return (ok, report) for the workload's dtype criteria."""
    tol = 1e-4 if dtype == "f32" else 1e-2
    ok_max, err, scale = max_error_ok(y, ref, tol)
    rep = {"max_abs_err": err, "max_abs_ref": scale, "tol": tol, "max_ok": ok_max}
    ok = ok_max
    if dtype != "f32":
        eff = effect_errors(y, ref, base, token_adapter)
        graded = [v for v in eff.values() if not np.isnan(v)]
        worst = max(graded) if graded else 0.0
        rep["worst_effect_err"] = worst
        rep["zero_effect_adapters"] = sorted(k for k, v in eff.items() if np.isnan(v))
        rep["effect_ok"] = worst <= 0.01
        ok = ok and rep["effect_ok"]
    return ok, rep
