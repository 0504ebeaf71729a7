"""CPU fp64 oracle of the normal-form batched adapter layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The GPU library does
not use it, and it uses nothing from the GPU library: the two share only the
seeded inputs drawn by ``synth``.

Source of every formula: "Scute: Exact Batched Serving for PEFT Adapters
Beyond LoRA" as explained on paper-daily.com (sections "What problem is it
solving?", "The big picture: six extra slots in the LoRA computation",
"Which slots can be merged at load?", "Where is the cheapest place to compute
the remaining slots?", "How does Scute plug into vLLM?").
"""

from .layer import (  # noqa: F401
    cayley,
    oft_rotation,
    base_output,
    method_output,
    forward,
    dora_weight,
    nf_slots,
    fold_slots,
    normal_form_output,
    forward_normal_form,
)
from .compare import effect_errors, max_error_ok, check  # noqa: F401
