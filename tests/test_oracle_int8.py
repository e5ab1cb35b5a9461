"""Pins of the int8 QK^T oracle (oracle/int8.py): hand-derived block scales
and codes with ties to even, symmetry, the uniform-quantisation bound, and
exactness of the attention oracle on the int8 grid."""
import json
import os

import numpy as np

import oracle
from oracle import int8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_blocks.json")


def test_golden_blocks():
    for b in json.load(open(GOLDEN))["blocks"]:
        x = np.array(b["x"], np.float32).reshape(4, 1)
        codes, s = int8.quantize(x)
        assert float(s[0]) == b["s"], b
        assert [int(c) for c in codes.ravel()] == b["codes"], b


def test_symmetric_and_bounded():
    rng = np.random.default_rng(3)
    x = (rng.normal(size=(2, 200, 64)) * rng.uniform(0.01, 30, (2, 1, 1))).astype(np.float32)
    x[0, 64:128] = 0.0
    c, s = int8.quantize(x)
    cn, sn = int8.quantize(-x)
    assert np.array_equal(s, sn) and np.array_equal(cn, -c)
    assert c.min() >= -127 and c.max() <= 127
    assert s[0, 1] == 1.0 and not c[0, 64:128].any()
    xh = int8.dequantize(c, s)
    srow = np.repeat(s, 64, axis=-1)[..., :200, None].astype(np.float64)
    assert np.all(np.abs(xh - x) <= srow * (0.5 + 1e-6))
    # each block's largest |x| maps to +-127
    for t in range(4):
        blk = np.abs(c[:, 64 * t:64 * t + 64]).reshape(2, -1).max(axis=1)
        live = np.abs(x[:, 64 * t:64 * t + 64]).reshape(2, -1).max(axis=1) > 0
        assert np.all(blk[live] == 127)


def test_prefill_qk8_is_exact_on_the_int8_grid():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, N, d = 1, 2, 1, 150, 64
    q = rng.integers(-127, 128, (B, Hq, N, d)).astype(np.float64) / 256.0
    k = rng.integers(-127, 128, (B, Hkv, N, d)).astype(np.float64) / 256.0
    for t in range(3):                               # every block's max -> 127 / 256
        q[..., 64 * t, 0] = 127 / 256.0
        k[..., 64 * t, 0] = 127 / 256.0
    v = rng.normal(size=(B, Hkv, N, d))
    got = int8.prefill_qk8(q.astype(np.float32), k.astype(np.float32), v, True, 4.0)
    want = oracle.prefill(q, k, v, True, 4.0)
    assert np.array_equal(got["mask"], want["mask"])
    assert np.abs(got["o"] - want["o"]).max() < 1e-12
    assert np.abs(got["lse"] - want["lse"]).max() < 1e-12
