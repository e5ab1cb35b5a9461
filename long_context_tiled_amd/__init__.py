"""libskipattn: exact tiled softmax attention with the Skip-Softmax rule on
MI355X (gfx950). The computation lives in the HIP library built from csrc/;
this package is its thin Python binding."""
from ._lib import (OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, TILE, SPLIT,
                   KEPT, SKIPPED, NOT_VISITED, EXPORTS, LIB_PATH, SkipAttnError,
                   load, attn_prefill, attn_decode, attn_decode_sas, attn_decode_workspace_bytes,
                   attn_last_error, prefill, decode, q4_shapes, attn_kv_quantize_q4,
                   attn_decode_q4, quantize_q4, decode_q4, attn_prefill_chunk, prefill_chunk,
                   empty_q4, q2_shapes, attn_kv_quantize_q2, attn_decode_q2, quantize_q2,
                   decode_q2, empty_q2, attn_decode_noalloc,
                   DECODE_SCRATCH_BYTES, attn_prefill_qk8, attn_prefill_qk8_workspace_bytes,
                   qk8_workspace_parts, prefill_qk8, attn_prefill_sas, hybrid_shapes,
                   attn_kv_quantize_hybrid, attn_decode_hybrid, empty_hybrid, quantize_hybrid,
                   decode_hybrid, attn_prefill_pv8, attn_prefill_pv8_workspace_bytes,
                   pv8_workspace_parts, prefill_pv8)

__all__ = ["OK", "EINVAL", "EUNSUPPORTED", "EWORKSPACE", "EHIP", "TILE", "SPLIT",
           "KEPT", "SKIPPED", "NOT_VISITED", "EXPORTS", "LIB_PATH", "SkipAttnError",
           "load", "attn_prefill", "attn_decode", "attn_decode_sas", "attn_decode_workspace_bytes",
           "attn_last_error", "prefill", "decode", "q4_shapes", "attn_kv_quantize_q4",
           "attn_decode_q4", "quantize_q4", "decode_q4", "attn_prefill_chunk",
           "prefill_chunk", "empty_q4", "q2_shapes", "attn_kv_quantize_q2",
           "attn_decode_q2", "quantize_q2", "decode_q2", "empty_q2",
           "attn_decode_noalloc", "DECODE_SCRATCH_BYTES", "attn_prefill_qk8",
           "attn_prefill_qk8_workspace_bytes", "qk8_workspace_parts", "prefill_qk8",
           "attn_prefill_sas", "hybrid_shapes", "attn_kv_quantize_hybrid",
           "attn_decode_hybrid", "empty_hybrid", "quantize_hybrid", "decode_hybrid",
           "attn_prefill_pv8", "attn_prefill_pv8_workspace_bytes", "pv8_workspace_parts",
           "prefill_pv8"]
