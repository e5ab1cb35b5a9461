"""Oracle for the 2-bit asymmetric KV-cache format: quantise, pack, dequantise.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive", the
pre-fill / decoding workflow and the trade-offs it lists): KV-cache storage
in low-bit asymmetric integers with a floating zero point per block, in a
4-bit (near-lossless) and a 2-bit (lossy, faster) option. This module is the
2-bit option; the 4-bit one is ``kvq4``; ``kvq_hybrid`` mixes the two in
one cache, one width per KV head.

Readings, as for the 4-bit format except where stated:

* Blocks: a K block is one key's row of d values; a V block is one channel
  of one 64-key tile (its keys that exist).
* Parameters: z = block minimum; s = (max - z) / 3 in fp32 (subtract, then
  divide, each rounded to nearest even), then rounded up to bf16.
* Codes: c = 0 when s == 0, else clamp(rint((x - z) / s), 0, 3) in fp32.
* Dequantised value: x^ = c * s + z; |x - x^| <= s / 2.
* Packing, per 32-bit little-endian word of 16 consecutive elements
  e0..e15: the even elements e0, e2, .., e14 in 2-bit fields 0..7 of bits
  0-15 and the odd ones e1, e3, .., e15 in fields 0..7 of bits 16-31; i.e.
  bytes [e0 | e2 << 2 | e4 << 4 | e6 << 6, e8 | e10 << 2 | e12 << 4 | e14 << 6,
  e1 | e3 << 2 | e5 << 4 | e7 << 6, e9 | e11 << 2 | e13 << 4 | e15 << 6].
* Parameter word: bf16 s (low half), bf16 z (high half), as for 4-bit.
* Arrays: kq uint8 [B, Hkv, L, d/4]; kp uint32 [B, Hkv, L];
  vq uint8 [B, Hkv, T, d, 16] (per tile and channel, the 64 keys' codes;
  keys at or past L: code 0, outside the minimum and maximum);
  vp uint32 [B, Hkv, T, d]; T = ceil(L / 64).

Parity unpinned: these format choices are readings, not the pages'. The
tests pin that the code implements them: hand-derived layout bytes, exact
round trips of caches built on the code grid, hand-derived codes where
(x - z) / s is exactly k + 1/2 (ties go to the even code), and the error
bound of uniform quantisation.
"""
from __future__ import annotations

import numpy as np

from .kvq4 import bf16_round_up, pack_params, unpack_params

CODE_MAX = 3
TILE = 64


def block_params(lo: np.ndarray, hi: np.ndarray):
    """(s, z) of blocks with fp32 minimum ``lo`` and maximum ``hi``."""
    lo = np.asarray(lo, np.float32)
    hi = np.asarray(hi, np.float32)
    span = np.subtract(hi, lo, dtype=np.float32)
    s = bf16_round_up(np.divide(span, np.float32(CODE_MAX), dtype=np.float32))
    return s, lo.copy()


def codes(x: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """2-bit codes of fp32 values x under broadcastable block parameters."""
    x = np.asarray(x, np.float32)
    s = np.asarray(s, np.float32)
    diff = np.subtract(x, np.asarray(z, np.float32), dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qv = np.divide(diff, s, dtype=np.float32)
    c = np.clip(np.rint(qv), 0, CODE_MAX)
    c = np.where(np.broadcast_to(s, c.shape) > 0, c, 0)
    return c.astype(np.uint8)


def quantize_k(k: np.ndarray):
    """K blocks = key rows. k fp32 (..., L, d) -> codes (..., L, d), s, z (..., L)."""
    k = np.asarray(k, np.float32)
    s, z = block_params(k.min(axis=-1), k.max(axis=-1))
    return codes(k, s[..., None], z[..., None]), s, z


def quantize_v(v: np.ndarray):
    """V blocks = one channel of one 64-key tile.

    v fp32 (..., L, d) -> codes (..., T, d, 64) (keys past L: 0), s, z (..., T, d).
    """
    v = np.asarray(v, np.float32)
    L, d = v.shape[-2], v.shape[-1]
    T = (L + TILE - 1) // TILE
    lead = v.shape[:-2]
    cs = np.zeros(lead + (T, d, TILE), np.uint8)
    ss = np.zeros(lead + (T, d), np.float32)
    zs = np.zeros(lead + (T, d), np.float32)
    for t in range(T):
        blk = np.swapaxes(v[..., TILE * t:min(L, TILE * (t + 1)), :], -1, -2)  # (..., d, n)
        s, z = block_params(blk.min(axis=-1), blk.max(axis=-1))
        cs[..., t, :, :blk.shape[-1]] = codes(blk, s[..., None], z[..., None])
        ss[..., t, :], zs[..., t, :] = s, z
    return cs, ss, zs


def pack_words(c: np.ndarray) -> np.ndarray:
    """Codes (..., n), n a multiple of 16 -> bytes (..., n / 4) in the word layout."""
    c = np.asarray(c, np.uint8)
    n = c.shape[-1]
    if n % 16:
        raise ValueError("element count must be a multiple of 16")
    e = c.reshape(c.shape[:-1] + (n // 16, 16))
    out = np.empty(c.shape[:-1] + (n // 16, 4), np.uint8)
    for byte, first in ((0, 0), (1, 8), (2, 1), (3, 9)):
        out[..., byte] = (e[..., first] | (e[..., first + 2] << 2) | (e[..., first + 4] << 4)
                          | (e[..., first + 6] << 6))
    return out.reshape(c.shape[:-1] + (n // 4,))


def unpack_words(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_words: bytes (..., n / 4) -> codes (..., n)."""
    b = np.asarray(b, np.uint8)
    m = b.shape[-1]
    w = b.reshape(b.shape[:-1] + (m // 4, 4))
    e = np.empty(b.shape[:-1] + (m // 4, 16), np.uint8)
    for byte, first in ((0, 0), (1, 8), (2, 1), (3, 9)):
        for f in range(4):
            e[..., first + 2 * f] = (w[..., byte] >> (2 * f)) & 3
    return e.reshape(b.shape[:-1] + (4 * m,))


def encode(k: np.ndarray, v: np.ndarray) -> dict:
    """K, V fp32 (B, Hkv, L, d) holding bf16 values -> the stored arrays."""
    kc, ks, kz = quantize_k(k)
    vc, vs, vz = quantize_v(v)
    return dict(kq=pack_words(kc), kp=pack_params(ks, kz),
                vq=pack_words(vc), vp=pack_params(vs, vz))


def decode_k(kq: np.ndarray, kp: np.ndarray) -> np.ndarray:
    """Stored K -> fp64 K^ (B, Hkv, L, d)."""
    s, z = unpack_params(kp)
    return unpack_words(kq).astype(np.float64) * s[..., None] + z[..., None]


def decode_v(vq: np.ndarray, vp: np.ndarray, L: int) -> np.ndarray:
    """Stored V -> fp64 V^ (B, Hkv, L, d)."""
    s, z = unpack_params(vp)
    c = unpack_words(vq).astype(np.float64)                 # (..., T, d, 64)
    x = c * s[..., None] + z[..., None]
    x = np.swapaxes(x, -1, -2)                               # (..., T, 64, d)
    lead = x.shape[:-3]
    x = x.reshape(lead + (x.shape[-3] * TILE, x.shape[-1]))
    return x[..., :L, :]
