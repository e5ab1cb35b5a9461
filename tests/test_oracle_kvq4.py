"""Pins of the 4-bit KV-cache oracle (oracle/kvq4.py) against facts fixed
outside its code: hand-derived bytes of the storage layout, exactly
representable blocks, and the error bound of uniform quantisation.

Format readings (TurboAttention talk page, "Technical Deep Dive": asymmetric
low-bit KV storage with a floating zero point per block) are listed in the
oracle's header."""
import json
import os

import numpy as np
import pytest

from oracle import kvq4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvq4_layout.json")


def _bf16(x):
    """fp32 values rounded to bf16 (nearest even), returned as fp32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32)


def test_golden_word_and_param_layout():
    g = json.load(open(GOLDEN))
    for case in g["words"]:
        got = kvq4.pack_words(np.array(case["codes"], np.uint8))
        assert [int(b) for b in got] == case["bytes"], case["note"]
        assert list(kvq4.unpack_words(got)) == case["codes"]
    for case in g["params"]:
        p = kvq4.pack_params(np.array([case["s"]], np.float32), np.array([case["z"]], np.float32))
        assert int(p[0]) == int(case["word"], 16), case
        s, z = kvq4.unpack_params(p)
        assert float(s[0]) == case["s"] and float(z[0]) == case["z"]


def test_bf16_round_up_examples():
    f = lambda bits: np.array([bits], np.uint32).view(np.float32)
    assert kvq4.bf16_round_up(f(0x3F800000)).view(np.uint32)[0] == 0x3F800000
    assert kvq4.bf16_round_up(f(0x3F800001)).view(np.uint32)[0] == 0x3F810000
    assert kvq4.bf16_round_up(f(0x3F80FFFF)).view(np.uint32)[0] == 0x3F810000
    assert kvq4.bf16_round_up(f(0x00000000)).view(np.uint32)[0] == 0
    # 1/15 in fp32 is 0x3D888889; the next bf16 above it is 0x3D890000
    s, z = kvq4.block_params(np.zeros(1, np.float32), np.ones(1, np.float32))
    assert s.view(np.uint32)[0] == 0x3D890000 and z[0] == 0.0


def test_exact_grid_row_round_trips():
    # a 16-value K row on the grid 1.5 * c: span 22.5, span / 15 = 1.5 exactly
    perm = np.array([3, 0, 15, 7, 1, 14, 2, 9, 8, 5, 11, 4, 13, 6, 10, 12])
    k = (1.5 * perm).astype(np.float32)[None, None, None, :]      # (1,1,1,16)
    c, s, z = kvq4.quantize_k(k)
    assert s.ravel()[0] == 1.5 and z.ravel()[0] == 0.0
    assert list(c.ravel()) == list(perm)
    enc = kvq4.encode(k, np.zeros((1, 1, 1, 16), np.float32))
    assert np.array_equal(kvq4.decode_k(enc["kq"], enc["kp"]), k.astype(np.float64))


def test_layouts_reproduce_representable_cache():
    # every block built so that 0 and 15 occur and s is a power of two:
    # dequantisation must give the input back exactly, which pins where each
    # element of K (rows) and V (tile x channel) is stored.
    rng = np.random.default_rng(7)
    B, H, L, d = 2, 3, 150, 16
    ck = rng.integers(0, 16, (B, H, L, d))
    ck[..., 0], ck[..., 1] = 0, 15
    sk = 2.0 ** rng.integers(-3, 3, (B, H, L, 1))
    zk = sk * rng.integers(-16, 17, (B, H, L, 1))       # x = s (c + m): |c + m| < 32
    k = (ck * sk + zk).astype(np.float32)
    cv = rng.integers(0, 16, (B, H, L, d))
    T = (L + 63) // 64
    for t in range(T):
        cv[:, :, 64 * t, :], cv[:, :, min(L, 64 * t + 64) - 1, :] = 0, 15
    sv = np.repeat(2.0 ** rng.integers(-3, 3, (B, H, T, 1, d)), 64, axis=2)[:, :, :, 0, :]
    zv = sv * np.repeat(rng.integers(-16, 17, (B, H, T, 1, d)), 64, axis=2)[:, :, :, 0, :]
    v = (cv * sv[:, :, :L] + zv[:, :, :L]).astype(np.float32)
    assert np.array_equal(_bf16(k), k) and np.array_equal(_bf16(v), v)
    enc = kvq4.encode(k, v)
    assert enc["kq"].shape == (B, H, L, d // 2) and enc["kp"].shape == (B, H, L)
    assert enc["vq"].shape == (B, H, T, d, 32) and enc["vp"].shape == (B, H, T, d)
    assert np.array_equal(kvq4.decode_k(enc["kq"], enc["kp"]), k.astype(np.float64))
    assert np.array_equal(kvq4.decode_v(enc["vq"], enc["vp"], L), v.astype(np.float64))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_uniform_quantisation_bounds(seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.normal(scale=rng.uniform(0.01, 50), size=(3, 70, 64)))
    x[0, 5, :] = x[0, 5, 0]                                       # a constant row
    c, s, z = kvq4.quantize_k(x)
    assert c.max() <= 15
    lo, hi = x.min(-1), x.max(-1)
    live = hi > lo
    assert np.all(s[live] * 15 >= (hi - lo)[live])                 # range covered
    assert np.all(s[~live] == 0) and np.all(c[~live] == 0)
    amin = x == lo[..., None]
    amax = x == hi[..., None]
    assert np.all(c[amin] == 0)
    assert np.all(c[amax & live[..., None]] == 15)
    xh = kvq4.decode_k(kvq4.pack_words(c), kvq4.pack_params(s, z))
    err = np.abs(xh - x)
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-6))
    assert np.all(err[~live] == 0)
    # codes are monotone in x inside a block
    order = np.argsort(x, axis=-1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(c, order, -1).astype(int), axis=-1) >= 0)


def test_partial_tile_uses_only_present_keys():
    rng = np.random.default_rng(3)
    L, d = 70, 8
    v = _bf16(rng.normal(size=(1, 1, L, d)))
    _, s, z = kvq4.quantize_v(v)
    tail = v[0, 0, 64:70, :]
    assert np.array_equal(z[0, 0, 1], tail.min(0))
    assert np.all(s[0, 0, 1] * 15 >= tail.max(0) - tail.min(0))
    c, _, _ = kvq4.quantize_v(v)
    assert np.all(c[0, 0, 1, :, 6:] == 0)


def test_golden_rounding_ties_go_to_even():
    # (x - z) / s exactly k + 1/2: hand-derived codes (ties to the even
    # code), both as K rows and as V channels of one 64-key tile.
    g = json.load(open(GOLDEN))["ties"]
    for row in g["rows"]:
        x = np.array(row["x"], np.float32)
        c, s, z = kvq4.quantize_k(x[None, None, None, :])
        assert float(s.ravel()[0]) == row["s"] and float(z.ravel()[0]) == row["z"]
        assert list(c.ravel()) == row["codes"], row
        assert row["codes"] != row["half_up_would_give"]
        v = np.zeros((1, 1, 8, 4), np.float32)
        v[0, 0, :, 1] = x                            # channel 1 over the tile's 8 keys
        cv, sv, zv = kvq4.quantize_v(v)
        assert float(sv[0, 0, 0, 1]) == row["s"] and float(zv[0, 0, 0, 1]) == row["z"]
        assert list(cv[0, 0, 0, 1, :8]) == row["codes"], row
