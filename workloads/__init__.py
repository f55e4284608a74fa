"""Seeded synthetic workloads shared by the oracle tests and the HIP path."""
from .synth import (NAMED, Spec, Workload, bf16_bits_to_f32, custom, f32_to_bf16_bits, random_cu,
                    spec)

__all__ = ["NAMED", "Spec", "Workload", "bf16_bits_to_f32", "custom", "f32_to_bf16_bits",
           "random_cu", "spec"]
