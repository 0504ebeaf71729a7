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
