"""Oracle for the 4-bit asymmetric KV-cache format: quantise, pack, dequantise.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive" and its
pre-fill / decoding workflow): the KV cache is stored and moved in a low-bit
asymmetric integer format with a floating zero point per block, and decoding
turns it back into numbers inside the attention kernel before the products.
Of the hybrid 2/4-bit choice the 4-bit width is taken, the one the talk calls
near-lossless. Everything else about the format is left open by the pages;
the readings taken here:

* Blocks. A K block is one key's row of d values; a V block is one channel of
  one 64-key tile (keys 64t .. 64t + 63 that exist). Each block runs along the
  contraction index of the product that consumes it (d for q.K, keys for P.V),
  so its scale and zero factor out of that product.
* Parameters, per block: z = the block minimum (a bf16 value already, since
  the inputs are bf16); s = (max - z) / 15 computed in fp32 (subtract, then
  divide, each rounded to nearest even), then rounded up to the next bf16
  value. Rounding s up keeps z + 15 s >= max, so no value is clamped.
* Codes: c = 0 when s == 0, else c = clamp(rint((x - z) / s), 0, 15), with the
  subtraction and the division in fp32 rounded to nearest even and rint
  rounding half to even. These fp32 steps decide an integer, so the kernel
  must take them in the same precision.
* Dequantised value: x^ = c * s + z (exact in fp64). |x - x^| <= s / 2.
* Packing, per 32-bit little-endian word of 8 consecutive elements e0..e7
  (consecutive d for K, consecutive keys for V): the even elements e0, e2, e4,
  e6 sit in nibbles 0..3 (bits 0-15) and the odd ones e1, e3, e5, e7 in
  nibbles 4..7 (bits 16-31); i.e. bytes [e0 | e2 << 4, e4 | e6 << 4,
  e1 | e3 << 4, e5 | e7 << 4].
* Parameters are stored as one 32-bit word per block: s's bf16 bits in the
  low half, z's in the high half.
* Arrays: kq uint8 [B, Hkv, L, d/2]; kp uint32 [B, Hkv, L];
  vq uint8 [B, Hkv, T, d, 32] with T = ceil(L / 64) (per tile and channel,
  the 64 keys' codes; keys at or past L have code 0 and take no part in the
  tile's minimum and maximum); vp uint32 [B, Hkv, T, d].

Parity unpinned: these format choices are readings, not the pages' (which
give no block size, rounding or layout). What the tests pin is that the code
implements them: hand-derived layout bytes, exact round trips of caches
built on the code grid, hand-derived codes where (x - z) / s is exactly
k + 1/2 (ties go to the even code), and the error bound of uniform
quantisation.
"""
from __future__ import annotations

import numpy as np

CODE_MAX = 15
TILE = 64


def bf16_round_up(x: np.ndarray) -> np.ndarray:
    """Non-negative finite fp32 values rounded up to the bf16 grid (as fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    up = np.where(bits & 0xFFFF, (bits + 0x10000) & 0xFFFF0000, bits)
    return up.astype(np.uint32).view(np.float32)


def block_params(lo: np.ndarray, hi: np.ndarray):
    """(s, z) of blocks with fp32 minimum ``lo`` and maximum ``hi``."""
    lo = np.asarray(lo, np.float32)
    hi = np.asarray(hi, np.float32)
    span = np.subtract(hi, lo, dtype=np.float32)
    s = bf16_round_up(np.divide(span, np.float32(CODE_MAX), dtype=np.float32))
    return s, lo.copy()


def codes(x: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """4-bit codes of fp32 values x under broadcastable block parameters."""
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
    """Codes (..., n), n a multiple of 8 -> bytes (..., n / 2) in the word layout."""
    c = np.asarray(c, np.uint8)
    n = c.shape[-1]
    if n % 8:
        raise ValueError("element count must be a multiple of 8")
    e = c.reshape(c.shape[:-1] + (n // 8, 8))
    out = np.empty(c.shape[:-1] + (n // 8, 4), np.uint8)
    out[..., 0] = e[..., 0] | (e[..., 2] << 4)
    out[..., 1] = e[..., 4] | (e[..., 6] << 4)
    out[..., 2] = e[..., 1] | (e[..., 3] << 4)
    out[..., 3] = e[..., 5] | (e[..., 7] << 4)
    return out.reshape(c.shape[:-1] + (n // 2,))


def unpack_words(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_words: bytes (..., n / 2) -> codes (..., n)."""
    b = np.asarray(b, np.uint8)
    m = b.shape[-1]
    w = b.reshape(b.shape[:-1] + (m // 4, 4))
    e = np.empty(b.shape[:-1] + (m // 4, 8), np.uint8)
    e[..., 0], e[..., 2] = w[..., 0] & 15, w[..., 0] >> 4
    e[..., 4], e[..., 6] = w[..., 1] & 15, w[..., 1] >> 4
    e[..., 1], e[..., 3] = w[..., 2] & 15, w[..., 2] >> 4
    e[..., 5], e[..., 7] = w[..., 3] & 15, w[..., 3] >> 4
    return e.reshape(b.shape[:-1] + (2 * m,))


def pack_params(s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """bf16-valued fp32 s and z -> one uint32 per block (s low half, z high)."""
    sb = np.ascontiguousarray(s, np.float32).view(np.uint32) >> 16
    zb = np.ascontiguousarray(z, np.float32).view(np.uint32) >> 16
    return (sb | (zb << 16)).astype(np.uint32)


def unpack_params(p: np.ndarray):
    p = np.ascontiguousarray(p, np.uint32)
    s = (p << 16).astype(np.uint32).view(np.float32)
    z = (p & 0xFFFF0000).astype(np.uint32).view(np.float32)
    return s, z


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
