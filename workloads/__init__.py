"""Seeded synthetic inputs for the top-k / top-p logits filter.

This package only draws random numbers and stores them in the logits dtype.
It holds none of the filter's arithmetic, so both the CPU oracle and the HIP
path can take their inputs from it.
"""

from .synth import (  # noqa: F401
    WORKLOAD_SPECS,
    Workload,
    bf16_bits_from_f32,
    bits_to_f32,
    make_workload,
    random_rows,
)
