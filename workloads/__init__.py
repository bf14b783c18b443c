"""Seeded synthetic workloads shared by the oracle checks, the HIP parity
tests and the benchmark (random draws only; none of the method's arithmetic)."""
from .gen import (Workload, describe, generate, random_qkv, f32_to_bf16_bits,
                  bf16_to_f32, bf16_to_f64, sha256, digests)

__all__ = ["Workload", "describe", "generate", "random_qkv", "f32_to_bf16_bits",
           "bf16_to_f32", "bf16_to_f64", "sha256", "digests"]
