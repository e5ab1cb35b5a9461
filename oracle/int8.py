"""Oracle for prefill attention with block-quantised symmetric int8 QK^T.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive" and "Key
Findings"; its pre-fill workflow): the matrix products of blockwise attention
run on symmetric int8 operands, quantised block-wise inside the blocks of
the flash computation; here the QK^T product (V and PV stay bf16).

Readings, where the pages are silent:

* Blocks: as for the fp8 reading, a Q block is one 64-row query tile of one
  head, a K block one 64-key tile of one KV head, one fp32 scale each.
* Scale: s = m / 127 with m the block's largest |x| (fp32 division rounded
  to nearest even); a block of zeros takes s = 1.
* Codes: c = clamp(rint(x / s), -127, 127), the division in fp32 rounded to
  nearest even and rint rounding half to even (symmetric: -128 unused).
* Dequantised value: c x s (exact in fp64). Scores s_ij = q^_i . k^_j /
  sqrt(d); the rest is the exact oracle.

Parity unpinned: block size, scale rule and rounding are readings. The
tests pin the code: hand-derived scales and codes (ties to even included),
symmetry, the uniform-quantisation bound |x - x^| <= s / 2, and exactness
of the attention oracle on inputs that sit on the int8 grid.
"""
from __future__ import annotations

import numpy as np

from .attention import TILE, prefill as exact_prefill

CODE_MAX = 127


def block_scales(x: np.ndarray, rows: int = TILE) -> np.ndarray:
    """x fp32 (..., N, d) -> fp32 scale per block of ``rows`` rows (..., nb)."""
    x = np.asarray(x, np.float32)
    N = x.shape[-2]
    nb = (N + rows - 1) // rows
    out = np.empty(x.shape[:-2] + (nb,), np.float32)
    for b in range(nb):
        m = np.abs(x[..., b * rows:min(N, (b + 1) * rows), :]).max(axis=(-1, -2))
        s = np.divide(m, np.float32(CODE_MAX), dtype=np.float32)
        out[..., b] = np.where(m > 0, s, np.float32(1.0))
    return out


def quantize(x: np.ndarray, rows: int = TILE):
    """x fp32 (..., N, d) -> (codes int8 (..., N, d), scales fp32 (..., nb))."""
    x = np.asarray(x, np.float32)
    s = block_scales(x, rows)
    srow = np.repeat(s, rows, axis=-1)[..., :x.shape[-2]][..., None]
    y = np.divide(x, srow, dtype=np.float32)
    c = np.clip(np.rint(y), -CODE_MAX, CODE_MAX)
    return c.astype(np.int8), s


def dequantize(codes: np.ndarray, scales: np.ndarray, rows: int = TILE) -> np.ndarray:
    N = codes.shape[-2]
    srow = np.repeat(np.asarray(scales, np.float64), rows, axis=-1)[..., :N][..., None]
    return np.asarray(codes, np.float64) * srow


def prefill_qk8(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, tau: float,
                forced=None):
    """The prefill oracle on int8-quantised Q and K (fp32 inputs holding bf16
    values); V as given."""
    qc, qs = quantize(q)
    kc, ks = quantize(k)
    return exact_prefill(dequantize(qc, qs), dequantize(kc, ks), np.asarray(v, np.float64),
                         causal, tau, forced)
