"""Seeded synthetic MLA decode workloads (inputs only; no method arithmetic)."""
from .configs import ALL, Workload, get  # noqa: F401
from .generate import DecodeInputs, f32_to_bf16_bits, make_inputs, unused_slots  # noqa: F401
