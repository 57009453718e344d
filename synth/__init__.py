"""Seeded synthetic inputs shared by the oracle tests, the HIP tests and the bench."""
from .fields import (DRIFT, WORKLOADS, Workload, generate, scaled, layer_stack, as_f32,
                     f32_to_bf16_bits, bf16_bits_to_f32)

__all__ = ["DRIFT", "WORKLOADS", "Workload", "generate", "scaled", "layer_stack", "as_f32",
           "f32_to_bf16_bits", "bf16_bits_to_f32"]
