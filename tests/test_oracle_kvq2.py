"""Pins of the 2-bit KV-cache oracle (oracle/kvq2.py) against facts fixed
outside its code: hand-derived bytes of the storage layout, exactly
representable blocks, and the error bound of uniform quantisation.

Format readings (TurboAttention talk page, "Technical Deep Dive": asymmetric
low-bit KV storage with a floating zero point per block, in a 4-bit and a
lossier 2-bit option) are listed in the oracle's header."""
import json
import os

import numpy as np
import pytest

from oracle import kvq2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvq2_layout.json")


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32)


def test_golden_word_layout_and_scale():
    g = json.load(open(GOLDEN))
    for case in g["words"]:
        got = kvq2.pack_words(np.array(case["codes"], np.uint8))
        assert [int(b) for b in got] == case["bytes"], case["note"]
        assert list(kvq2.unpack_words(got)) == case["codes"]
    sc = g["scale"]
    s, z = kvq2.block_params(np.array([sc["lo"]], np.float32), np.array([sc["hi"]], np.float32))
    assert s.view(np.uint32)[0] == int(sc["s_bits"], 16) and z[0] == sc["lo"]


def test_exact_grid_row_round_trips():
    # a 16-value K row on the grid 1.5 * c: span 4.5, span / 3 = 1.5 exactly
    perm = np.array([3, 0, 1, 2, 2, 1, 0, 3, 1, 1, 3, 0, 2, 0, 3, 2])
    k = (1.5 * perm).astype(np.float32)[None, None, None, :]
    c, s, z = kvq2.quantize_k(k)
    assert s.ravel()[0] == 1.5 and z.ravel()[0] == 0.0
    assert list(c.ravel()) == list(perm)
    enc = kvq2.encode(k, np.zeros((1, 1, 1, 16), np.float32))
    assert np.array_equal(kvq2.decode_k(enc["kq"], enc["kp"]), k.astype(np.float64))


def test_layouts_reproduce_representable_cache():
    # every block holds codes 0 and 3 and has a power-of-two s: dequantisation
    # gives the input back exactly, which pins where each element is stored
    rng = np.random.default_rng(17)
    B, H, L, d = 2, 3, 150, 16
    ck = rng.integers(0, 4, (B, H, L, d))
    ck[..., 0], ck[..., 1] = 0, 3
    sk = 2.0 ** rng.integers(-3, 3, (B, H, L, 1))
    zk = sk * rng.integers(-16, 17, (B, H, L, 1))
    k = (ck * sk + zk).astype(np.float32)
    cv = rng.integers(0, 4, (B, H, L, d))
    T = (L + 63) // 64
    for t in range(T):
        cv[:, :, 64 * t, :], cv[:, :, min(L, 64 * t + 64) - 1, :] = 0, 3
    sv = np.repeat(2.0 ** rng.integers(-3, 3, (B, H, T, 1, d)), 64, axis=2)[:, :, :, 0, :]
    zv = sv * np.repeat(rng.integers(-16, 17, (B, H, T, 1, d)), 64, axis=2)[:, :, :, 0, :]
    v = (cv * sv[:, :, :L] + zv[:, :, :L]).astype(np.float32)
    assert np.array_equal(_bf16(k), k) and np.array_equal(_bf16(v), v)
    enc = kvq2.encode(k, v)
    assert enc["kq"].shape == (B, H, L, d // 4) and enc["kp"].shape == (B, H, L)
    assert enc["vq"].shape == (B, H, T, d, 16) and enc["vp"].shape == (B, H, T, d)
    assert np.array_equal(kvq2.decode_k(enc["kq"], enc["kp"]), k.astype(np.float64))
    assert np.array_equal(kvq2.decode_v(enc["vq"], enc["vp"], L), v.astype(np.float64))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_uniform_quantisation_bounds(seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.normal(scale=rng.uniform(0.01, 50), size=(3, 70, 64)))
    x[0, 5, :] = x[0, 5, 0]
    c, s, z = kvq2.quantize_k(x)
    assert c.max() <= 3
    lo, hi = x.min(-1), x.max(-1)
    live = hi > lo
    assert np.all(s[live] * 3 >= (hi - lo)[live])
    assert np.all(s[~live] == 0) and np.all(c[~live] == 0)
    assert np.all(c[x == lo[..., None]] == 0)
    assert np.all(c[(x == hi[..., None]) & live[..., None]] == 3)
    xh = kvq2.decode_k(kvq2.pack_words(c), kvq2.pack_params(s, z))
    err = np.abs(xh - x)
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-6))
    order = np.argsort(x, axis=-1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(c, order, -1).astype(int), axis=-1) >= 0)


def test_partial_tile_uses_only_present_keys():
    rng = np.random.default_rng(3)
    L, d = 70, 16
    v = _bf16(rng.normal(size=(1, 1, L, d)))
    c, s, z = kvq2.quantize_v(v)
    tail = v[0, 0, 64:70, :]
    assert np.array_equal(z[0, 0, 1], tail.min(0))
    assert np.all(s[0, 0, 1] * 3 >= tail.max(0) - tail.min(0))
    assert np.all(c[0, 0, 1, :, 6:] == 0)


def test_golden_rounding_ties_go_to_even():
    # (x - z) / s exactly k + 1/2: hand-derived codes (ties to the even
    # code), as a K row and as one V channel of a tile.
    g = json.load(open(GOLDEN))["ties"]
    for row in g["rows"]:
        x = np.array(row["x"], np.float32)
        c, s, z = kvq2.quantize_k(x[None, None, None, :])
        assert float(s.ravel()[0]) == row["s"] and float(z.ravel()[0]) == row["z"]
        assert list(c.ravel()) == row["codes"], row
        assert row["codes"] != row["half_up_would_give"]
        v = np.zeros((1, 1, 8, 4), np.float32)
        v[0, 0, :, 1] = x                            # channel 1 over the tile's 8 keys
        cv, sv, zv = kvq2.quantize_v(v)
        assert float(sv[0, 0, 0, 1]) == row["s"] and float(zv[0, 0, 0, 1]) == row["z"]
        assert list(cv[0, 0, 0, 1, :8]) == row["codes"], row
