"""Seeded synthetic inputs shared by the fp64 oracle and the HIP library."""
from .gen import (WORKLOADS, TILE, SPLIT, workload, make_prefill, make_decode,
                  make_inputs, f32_to_bf16_bits, bf16_bits_to_f32,
                  bf16_bits_to_f64)

__all__ = ["WORKLOADS", "TILE", "SPLIT", "workload", "make_prefill",
           "make_decode", "make_inputs", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "bf16_bits_to_f64"]
