"""Seeded synthetic workloads for the normal-form batched adapter layer.

This package only draws random inputs (activations, base weight, adapter
parameters, token-to-adapter assignment) and rounds them to the storage
precision of the workload. It holds none of the layer's arithmetic: the CPU
oracle and the GPU library both consume exactly the arrays drawn here.
"""

from .workloads import (  # noqa: F401
    Adapter,
    Workload,
    WorkloadSpec,
    AdapterSpec,
    CONFIG_NAMES,
    config_spec,
    make_config,
    make_workload,
    round_bf16,
    round_f32,
    bf16_bits,
)
