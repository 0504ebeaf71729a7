"""Normal-form batched adapter layer for MI355X (gfx950).

The compute path lives in libscute.so (C ABI: include/scute.h); ``scute``
is its ctypes binding and ``workload`` loads a synthetic workload into a
layer. Importing ``scute`` without a built library raises ImportError.
"""
