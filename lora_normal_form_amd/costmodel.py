"""The zero-parameter time model and roofline helpers.

"Where is the cheapest place to compute the remaining slots?" (paper-daily.com
explainer of "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA"):
adapter work moves many bytes per flop, so its cost is bytes; the added
time of a route is extra bytes / memory bandwidth + extra kernel launches x
launch cost, with no fitted parameter.
"""

from __future__ import annotations

# MI355X published peaks
HBM_BYTES_PER_S = 8.0e12
BF16_DENSE_FLOPS = 2.5e15
FP32_VECTOR_FLOPS = 157.3e12


def added_time(extra_bytes: float, bandwidth: float, extra_launches: int = 0,
               launch_cost: float = 0.0) -> float:
    """Predicted added time in seconds."""
    return extra_bytes / bandwidth + extra_launches * launch_cost


def roofline_time(bytes_: float, flops: float, bw: float = HBM_BYTES_PER_S,
                  peak: float = BF16_DENSE_FLOPS) -> float:
    return max(bytes_ / bw, flops / peak)


def bound(bytes_: float, flops: float, bw: float = HBM_BYTES_PER_S,
          peak: float = BF16_DENSE_FLOPS) -> str:
    return "hbm" if bytes_ / bw >= flops / peak else "mfma"


# ---- route variants of the decode path (plan flags SCUTE_PLAN_ROUTE_*) -------
# Bytes each route moves beyond the route it is compared with, from the
# batch's row counts (fp32 output y of d_out per row). Passes that only move
# an operand read from the fused epilogue (B', s, b, e, t, u, B_sh) or from
# the prologue (x, P) into a kernel of their own add no bytes; what they add
# is their own pass over y, and for the separate s pass the copy of s to
# every row and its read back.

def route_extra(route: str, *, n: int, d_out: int, exp_rows: int = 0, s_rows: int = 0,
                s_chunks: int = 0, vera_rows: int = 0, rot_rows: int = 0):
    """(extra bytes, extra launches) of a route against its reference.

    route          compared with   what it adds
    "expand_pass"  fused           y read + written once more for the rows with
                                   s, b or an own term (the expand pass) and
                                   for the VeRA rows (the VeRA pass)
    "separate_s"   expand_pass     S = s copied to every row (s read for the
                                   s_rows, S written for all n rows), then y
                                   and S read and y written, less the s the
                                   expand pass no longer reads (one d_out
                                   vector per chunk with s)
    "vera_pass"    fused           y read + written once more for the VeRA rows
    "rotate_pass"  fused           nothing: x and P move from the prologue
    """
    row = 4.0 * d_out
    if route == "expand_pass":
        return 2 * row * (exp_rows + vera_rows), int(exp_rows > 0) + int(vera_rows > 0)
    if route == "separate_s":
        return row * (s_rows + n) + 3 * row * n - row * s_chunks, 2
    if route == "vera_pass":
        return 2 * row * vera_rows, int(vera_rows > 0)
    if route == "rotate_pass":
        return 0.0, int(rot_rows > 0)
    raise ValueError(f"unknown route {route!r}")
