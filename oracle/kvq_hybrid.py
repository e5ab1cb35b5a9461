"""Oracle for the hybrid 2/4-bit KV cache: per-head widths in one cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive"): the
compressed cache mixes two widths, keeping the parts that matter less at 2
bits and those that matter more at 4. They say neither what a "part" is nor
how importance is judged. The readings taken here:

* The part is the KV head (one head's keys and values share one width), and
  the width of each head is an input chosen by the caller: bits[g] in {4, 2}
  for KV head g. No selection rule is implemented.
* Each width's heads are stored as a cache of that width (``kvq4`` or
  ``kvq2``, blocks, rounding and layout unchanged) holding just those heads,
  in increasing head order, batch leading as in the full cache.
* Decoding attends each query head to its KV head's keys and values as that
  width dequantises them; the attention itself is the exact decode.

Parity unpinned for the choice of unit and of widths (readings, not the
pages'). What the tests pin: the placement (hand-derived parameter words of
constant heads), reduction to the single-width caches when every head has
one width, and head-by-head equality with the single-width codec.
"""
from __future__ import annotations

import numpy as np

from . import kvq2, kvq4

CODECS = {4: kvq4, 2: kvq2}


def heads_of(bits, width: int) -> list:
    """KV heads stored at ``width`` bits, in increasing order."""
    for b in bits:
        if int(b) not in CODECS:
            raise ValueError(f"head width must be 4 or 2, got {b}")
    return [g for g, b in enumerate(bits) if int(b) == width]


def encode(k: np.ndarray, v: np.ndarray, bits) -> dict:
    """K, V fp32 (B, Hkv, L, d) holding bf16 values -> {4: arrays or None,
    2: arrays or None}, each width's heads quantised by its codec."""
    assert k.shape[1] == len(bits)
    out = {}
    for w, codec in CODECS.items():
        hs = heads_of(bits, w)
        out[w] = codec.encode(k[:, hs], v[:, hs]) if hs else None
    return out


def decode_kv(enc: dict, bits, L: int):
    """The dequantised cache: fp64 K^, V^ (B, Hkv, L, d), head g from the
    cache of width bits[g]."""
    parts = {}
    for w, codec in CODECS.items():
        if enc[w] is not None:
            e = enc[w]
            parts[w] = (codec.decode_k(e["kq"], e["kp"]), codec.decode_v(e["vq"], e["vp"], L))
    some = next(iter(parts.values()))
    B, d = some[0].shape[0], some[0].shape[-1]
    K = np.empty((B, len(bits), L, d))
    V = np.empty((B, len(bits), L, d))
    for w in parts:
        for i, g in enumerate(heads_of(bits, w)):
            K[:, g] = parts[w][0][:, i]
            V[:, g] = parts[w][1][:, i]
    return K, V
