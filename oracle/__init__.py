"""fp64 CPU oracle for Skip-Softmax tiled attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package entry's smoke
check and by the benchmark's CPU-baseline leg, never by the library's product
path. It shares no code with the HIP kernels.
"""
from .attention import (TILE, SPLIT, KEPT, SKIPPED, NOT_VISITED, prefill,
                        prefill_blocks, prefill_decisions, decode, decode_head,
                        decode_heads)
from . import fp8, fp8pv, int8, kvq2, kvq4, kvq_hybrid, sas

__all__ = ["TILE", "SPLIT", "KEPT", "SKIPPED", "NOT_VISITED", "prefill",
           "prefill_blocks", "prefill_decisions", "decode", "decode_head", "decode_heads", "fp8", "fp8pv", "int8", "kvq2", "kvq4",
           "kvq_hybrid", "sas"]
