"""Pins of the hybrid 2/4-bit cache oracle (oracle/kvq_hybrid.py): where
each head's codes go (hand-derived parameter words of constant heads),
reduction to the single-width caches, and head-by-head agreement with the
single-width codecs. The reading (one width per KV head, chosen by the
caller; TurboAttention talk page, "Technical Deep Dive") is stated in the
oracle's header."""
import numpy as np
import pytest

from oracle import kvq2, kvq4, kvq_hybrid


def _bf16(x):
    """fp32 array of the bf16 values nearest x (ties to even)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32)


def _same(a, b):
    assert a.keys() == b.keys()
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_constant_heads_land_in_their_width_in_head_order():
    # B = 2, heads (2, 4, 2) bits; K[b, g] = V[b, g] = 10 b + g + 1 everywhere.
    # A constant block has s = 0 and z = the constant: parameter word =
    # bf16(z) << 16. bf16 bits: 1 -> 0x3F80, 2 -> 0x4000, 3 -> 0x4040,
    # 11 -> 0x4130, 12 -> 0x4140, 13 -> 0x4150.
    B, L, d = 2, 70, 64
    val = np.array([[1, 2, 3], [11, 12, 13]], np.float32)
    k = np.broadcast_to(val[:, :, None, None], (B, 3, L, d)).copy()
    enc = kvq_hybrid.encode(k, k.copy(), (2, 4, 2))
    assert enc[4]["kp"].shape == (B, 1, L) and enc[2]["kp"].shape == (B, 2, L)
    want4 = {0: [0x4000], 1: [0x4140]}
    want2 = {0: [0x3F80, 0x4040], 1: [0x4130, 0x4150]}
    for b in range(B):
        for i, zb in enumerate(want4[b]):
            assert (enc[4]["kp"][b, i] == zb << 16).all()
            assert (enc[4]["vp"][b, i] == zb << 16).all()
        for i, zb in enumerate(want2[b]):
            assert (enc[2]["kp"][b, i] == zb << 16).all()
            assert (enc[2]["vp"][b, i] == zb << 16).all()
    assert not enc[4]["kq"].any() and not enc[2]["vq"].any()
    K, V = kvq_hybrid.decode_kv(enc, (2, 4, 2), L)
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, K)


@pytest.mark.parametrize("w,codec", [(4, kvq4), (2, kvq2)])
def test_one_width_is_that_cache(w, codec):
    rng = np.random.default_rng(40 + w)
    B, H, L, d = 2, 3, 130, 64
    k = rng.standard_normal((B, H, L, d)).astype(np.float32)
    v = rng.standard_normal((B, H, L, d)).astype(np.float32)
    enc = kvq_hybrid.encode(k, v, (w,) * H)
    assert enc[6 - w] is None
    ref = codec.encode(k, v)
    _same(enc[w], ref)
    K, V = kvq_hybrid.decode_kv(enc, (w,) * H, L)
    assert np.array_equal(K, codec.decode_k(ref["kq"], ref["kp"]))
    assert np.array_equal(V, codec.decode_v(ref["vq"], ref["vp"], L))


def test_mixed_heads_match_their_codec_head_by_head():
    rng = np.random.default_rng(44)
    B, L, d = 2, 200, 64
    bits = (4, 2, 2, 4, 2)
    k = _bf16(rng.standard_normal((B, len(bits), L, d)) * 3)
    v = _bf16(rng.standard_normal((B, len(bits), L, d)))
    K, V = kvq_hybrid.decode_kv(kvq_hybrid.encode(k, v, bits), bits, L)
    for g, w in enumerate(bits):
        codec = kvq4 if w == 4 else kvq2
        e = codec.encode(k[:, g:g + 1], v[:, g:g + 1])
        assert np.array_equal(K[:, g], codec.decode_k(e["kq"], e["kp"])[:, 0])
        assert np.array_equal(V[:, g], codec.decode_v(e["vq"], e["vp"], L)[:, 0])
        # the width shows in the error: within s / 2 of the head's own width
        # (s = span / (2^w - 1), rounded up to bf16: at most 2^-7 above)
        span = k[:, g].max(-1).astype(np.float64) - k[:, g].min(-1)
        err = np.abs(K[:, g] - k[:, g]).max(-1)
        assert (err <= span / (15 if w == 4 else 3) * 0.5 * (1 + 2.0 ** -7)).all()
        if w == 2:   # and a 2-bit head is coarser than the 4-bit bound allows
            assert (err > span / 15 * 0.5 * (1 + 2.0 ** -7)).any()


def test_other_widths_are_refused():
    with pytest.raises(ValueError):
        kvq_hybrid.heads_of((4, 3), 4)
