"""Pins of the 8-bit QK^T oracle (oracle/fp8.py) against facts fixed outside
its code: hand-derived E4M3 encodings (normal, subnormal, largest, ties to
even, zero), every finite code decoding and re-encoding to itself, the
scales and codes of hand-built blocks, the format's error bound, and the
attention oracle it feeds (exact when the inputs sit on the fp8 grid)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3.json")


def test_golden_encodings():
    g = json.load(open(GOLDEN))
    for c in g["codes"]:
        got = int(fp8.e4m3_encode(np.array([c["x"]]))[0])
        assert got == int(c["code"], 16), c
    for b in g["blocks"]:
        x = np.array(b["x"], np.float32).reshape(4, 1)        # one block of 4 rows, d = 1
        codes, s = fp8.quantize(x)
        assert float(s[0]) == b["s"], b
        assert [int(v) for v in codes.ravel()] == [int(h, 16) for h in b["codes"]], b


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and c != 0x80], np.uint8)
    vals = fp8.e4m3_value(codes)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)
    assert np.all(np.diff(vals[codes < 0x80]) > 0)              # positive codes increase
    assert fp8.e4m3_value(np.array([0x7E]))[0] == 448.0
    assert fp8.e4m3_value(np.array([0x01]))[0] == 2.0 ** -9
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([448.5]))


def test_symmetric_and_nearest():
    rng = np.random.default_rng(5)
    y = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-14, 1, 20000))
    c = fp8.e4m3_encode(y)
    cn = fp8.e4m3_encode(-y)
    nz = c != 0
    assert np.array_equal(cn[nz], c[nz] ^ 0x80)
    # nearest: no finite value is closer than the chosen one
    allc = np.array([c for c in range(127)], np.uint8)       # non-negative codes
    allv = fp8.e4m3_value(allc)
    dist = np.abs(np.abs(y)[:, None] - allv[None, :])
    best = dist.min(axis=1)
    got = np.abs(np.abs(y) - np.abs(fp8.e4m3_value(c)))
    assert np.allclose(got, best, rtol=0, atol=0)


def test_quantisation_error_bound():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(3, 200, 64)).astype(np.float32) * np.float32(3.0)
    x[1, 64:128] = 0.0                                        # a zero block
    codes, s = fp8.quantize(x)
    assert codes.shape == x.shape and s.shape == (3, 4)
    assert s[1, 1] == 1.0 and not codes[1, 64:128].any()
    xh = fp8.dequantize(codes, s)
    srow = np.repeat(s, 64, axis=-1)[..., :200, None].astype(np.float64)
    err = np.abs(xh - x)
    # half a spacing: 2^-4 relative in the normal range, 2^-10 s below it
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * srow) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the block maximum is exact (it maps to +-448)
    for b in range(4):
        blk = x[:, 64 * b:64 * b + 64]
        i = np.abs(blk).reshape(3, -1).argmax(axis=1)
        mx = blk.reshape(3, -1)[np.arange(3), i]
        got = xh[:, 64 * b:64 * b + 64].reshape(3, -1)[np.arange(3), i]
        live = mx != 0
        assert np.allclose(got[live], mx[live], rtol=1e-7, atol=0)


def test_prefill_qk8_is_exact_on_the_fp8_grid():
    # Q and K whose blocks hold E4M3 values with largest |x| 448 (scale 1)
    # quantise to themselves: the 8-bit oracle is then the exact oracle
    rng = np.random.default_rng(7)
    grid = fp8.e4m3_value(np.arange(0x40, 0x50, dtype=np.uint8))   # 2 .. 7.5
    B, Hq, Hkv, N, d = 1, 2, 1, 150, 64
    q = rng.choice(grid, (B, Hq, N, d)) * rng.choice([-1, 1], (B, Hq, N, d)) / 64.0
    k = rng.choice(grid, (B, Hkv, N, d)) * rng.choice([-1, 1], (B, Hkv, N, d)) / 64.0
    for t in range(3):                                         # every block's max -> 448 / 64 = 7
        q[..., 64 * t, 0] = 7.0
        k[..., 64 * t, 0] = 7.0
    v = rng.normal(size=(B, Hkv, N, d))
    got = fp8.prefill_qk8(q.astype(np.float32), k.astype(np.float32), v, True, 4.0)
    want = oracle.prefill(q, k, v, True, 4.0)
    assert np.array_equal(got["mask"], want["mask"])
    assert np.abs(got["o"] - want["o"]).max() < 1e-12
    assert np.abs(got["lse"] - want["lse"]).max() < 1e-12
