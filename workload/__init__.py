"""Seeded synthetic MLA decode workloads (inputs only; no method arithmetic)."""
from .configs import ALL, Workload, get  # noqa: F401
from .generate import (DecodeInputs, ProjectionInputs, f32_to_bf16_bits, make_inputs,  # noqa: F401
                       make_projection_inputs, unused_slots)
