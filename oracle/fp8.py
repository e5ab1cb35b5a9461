"""Oracle for prefill attention with block-quantised 8-bit QK^T.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive" and "Key
Findings"; its pre-fill workflow): the matrix products of blockwise attention
run on symmetric 8-bit quantised operands, quantised block-wise inside the
blocks of the flash computation, with the softmax and the rest in higher
precision. The pages use int8 on their hardware; gfx950's 8-bit matrix
cores take the OCP fp8 formats, and this build takes fp8 E4M3 for Q and K
(the QK^T product) and keeps V and the PV product in bf16.

Readings, where the pages are silent:

* Blocks: a Q block is one 64-row query tile of one head (64 x d values), a
  K block one 64-key tile of one KV head: the decision tiles of the rule.
  Each has one fp32 scale.
* Scale: s = m / 448 with m the block's largest |x| (fp32 division rounded
  to nearest even; 448 is E4M3's largest finite value); a block of zeros
  takes s = 1 (its codes are 0 whatever s is).
* Codes: E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals from 2^-9, largest finite 448) of y = x / s, the division in
  fp32 rounded to nearest even, y clamped to [-448, 448], then rounded to
  the nearest E4M3 value, ties to the even mantissa. Code bits: sign << 7,
  biased exponent << 3, mantissa; subnormals have exponent 0. A value that
  rounds to zero is code 0 (no negative zero).
* The dequantised value is code value x s (exact in fp64). Scores are then
  s_ij = q^_i . k^_j / sqrt(d), and the rest is the exact oracle: the skip
  rule, softmax and PV on V as given (bf16 values).

Parity unpinned: the choice of E4M3, the block sizes, the scale rule and
the handling of zero blocks are readings. The tests pin that the code
implements them: hand-derived E4M3 encodings (normal, subnormal, largest,
ties to even, the clamp), every finite code decoding and re-encoding to
itself, scales and codes of hand-built blocks, and the error bound of the
format.
"""
from __future__ import annotations

import numpy as np

from .attention import TILE, prefill as exact_prefill

FP8_MAX = 448.0
MIN_NORMAL_EXP = -6      # 2^-6, the smallest normal E4M3 magnitude
SUB_STEP = 2.0 ** -9     # spacing of the subnormals


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """E4M3 code bits (uint8, no NaN codes) -> values (fp64)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * SUB_STEP, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return sign * mag


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """fp32 values with |y| <= 448 -> nearest E4M3 codes, ties to even."""
    y = np.asarray(y, np.float64)
    if np.any(np.abs(y) > FP8_MAX) or np.any(~np.isfinite(y)):
        raise ValueError("E4M3 encoding takes finite |y| <= 448")
    a = np.abs(y)
    # binade exponent e (2^e <= a < 2^(e+1)); the subnormal range shares the
    # spacing of the 2^-6 binade
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.float64) - 1.0, MIN_NORMAL_EXP)
    step = np.exp2(e - 3.0)                # spacing of E4M3 values in that binade
    q = np.rint(a / step)                  # multiple of the spacing, ties to even
    # q == 16 is the next binade's first value; in the subnormal range q < 8
    normal = (a >= 2.0 ** MIN_NORMAL_EXP) | (q >= 8)
    bump = q >= 16
    e = np.where(bump, e + 1, e)
    q = np.where(bump, 8, q)
    code = np.where(normal, (e + 7) * 8 + (q - 8), q).astype(np.int64)
    # a value that rounds to zero takes code 0 whatever its sign (the format's
    # negative zero, 0x80, is never produced)
    code = np.where(np.signbit(y) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8)


def block_scales(x: np.ndarray, rows: int = TILE) -> np.ndarray:
    """Per block of ``rows`` consecutive rows (last axis d): fp32 scale.

    x (..., N, d) fp32 -> (..., ceil(N / rows)) fp32."""
    x = np.asarray(x, np.float32)
    N = x.shape[-2]
    nb = (N + rows - 1) // rows
    out = np.empty(x.shape[:-2] + (nb,), np.float32)
    for b in range(nb):
        m = np.abs(x[..., b * rows:min(N, (b + 1) * rows), :]).max(axis=(-1, -2))
        s = np.divide(m, np.float32(FP8_MAX), dtype=np.float32)
        out[..., b] = np.where(m > 0, s, np.float32(1.0))
    return out


def quantize(x: np.ndarray, rows: int = TILE):
    """x fp32 (..., N, d) -> (codes uint8 (..., N, d), scales fp32 (..., nb))."""
    x = np.asarray(x, np.float32)
    s = block_scales(x, rows)
    srow = np.repeat(s, rows, axis=-1)[..., :x.shape[-2]][..., None]
    y = np.divide(x, srow, dtype=np.float32)
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return e4m3_encode(y), s


def dequantize(codes: np.ndarray, scales: np.ndarray, rows: int = TILE) -> np.ndarray:
    """codes (..., N, d), scales (..., nb) -> fp64 values."""
    N = codes.shape[-2]
    srow = np.repeat(np.asarray(scales, np.float64), rows, axis=-1)[..., :N][..., None]
    return e4m3_value(codes) * srow


def prefill_qk8(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, tau: float,
                forced=None):
    """The prefill oracle on the quantised Q and K (fp32 inputs holding bf16
    values); V as given. Returns the exact oracle's dict (o, lse, mask,
    margin)."""
    qc, qs = quantize(q)
    kc, ks = quantize(k)
    return exact_prefill(dequantize(qc, qs), dequantize(kc, ks), np.asarray(v, np.float64),
                         causal, tau, forced)
