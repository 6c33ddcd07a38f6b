"""Seeded synthetic rounds shared by the oracle-side tests and the GPU path.

This package only draws random numbers and rounds them to the storage type.
It contains none of the method's arithmetic (no rotation, convolution,
normalisation, recurrence, attention or softmax).
"""
from .synth import (  # noqa: F401
    CONFIGS,
    ConfigSpec,
    LayerShapes,
    Request,
    Round,
    bf16_round,
    custom_round,
    make_round,
    rows_of,
    LAYER_KINDS,
    Stack,
    StackShapes,
    make_stack,
)
