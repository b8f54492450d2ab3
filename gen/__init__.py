"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package draws random numbers and rounds them to the storage dtypes the
layer consumes. It holds none of the layer's arithmetic: no convolution, no
normalisation, no recurrence. Both ``oracle/`` (through the tests) and the GPU
tests / benchmark take their inputs from here, so the two sides see the same
bits without sharing any computation.
"""

from .inputs import (  # noqa: F401
    DECODE_30_LAYERS,
    DECODE_M16_POOL64,
    PREFILL_L4096,
    RAGGED_T15717,
    TINY_FP32,
    WORKLOADS,
    LayerShape,
    bf16_bits_from_f32,
    make_decode_pool,
    make_decode_step,
    make_prefill,
    rng_for,
)
