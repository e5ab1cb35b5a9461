"""Pins of the 8-bit P.V prefill oracle (oracle/fp8pv.py) against facts fixed
outside its code: the exact oracle when nothing is rounded, hand-derived
outputs of a one-tile row and of two-tile rows around the rescale margin,
the scale and codes of a hand-built head, and hand-derived byte positions of
the kernel layout. The readings (TurboAttention talk page, "Technical Deep
Dive": both products on block-quantised 8-bit operands) are listed in the
oracle's header."""
import math

import numpy as np
import pytest

import oracle
from oracle import fp8, fp8pv


def _ident(p):
    return p


@pytest.mark.parametrize("causal,tau,N,spread", [
    (True, math.inf, 300, 3.0), (False, math.inf, 200, 3.0), (True, 2.0, 384, 4.0),
    (False, 6.0, 256, 8.0), (True, math.inf, 512, 12.0),
])
def test_no_rounding_is_the_exact_oracle(causal, tau, N, spread):
    # identity rounding and exact V: the reference-maximum bookkeeping (set,
    # moved past the margin, rescaled) must give exact softmax attention
    rng = np.random.default_rng(int(N + spread))
    d = 16
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d)) * spread
    # rising key norms make the running maximum climb past the margin often
    k *= np.linspace(0.2, 1.5, N)[:, None]
    v = rng.standard_normal((N, d))
    o, lse, dec, margin, slack, amb = fp8pv.pv8_blocks(q, k, v, 1.0, 0, causal, tau,
                                                       round_p=_ident)
    o2, lse2, dec2, margin2 = oracle.prefill_blocks(q, k, v, 0, causal, tau)
    assert np.array_equal(dec, dec2)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)
    assert not slack.any() and not amb.any()


def test_one_tile_row_by_hand():
    # d = 1, q = 1, scores ln p for p = 1, 0.6, 2^-11, 0.3 (4 keys, one
    # partial tile). E4M3 rounds 0.6 -> 0.625 (spacing 1/16 in [1/2, 1)),
    # 0.3 -> 0.3125 (spacing 1/32), 2^-11 -> 0 (below half the smallest
    # subnormal 2^-9); m_ref = 0.
    p = np.array([1.0, 0.6, 2.0 ** -11, 0.3])
    k = np.log(p)[:, None]
    vv = np.array([[1.0], [2.0], [4.0], [-8.0]])
    o, lse, dec, _, _, _ = fp8pv.pv8_blocks(np.ones((1, 1)), k, vv, 0.5, 0, False, math.inf)
    l = 1.9 + 2.0 ** -11
    want = 0.5 * (1.0 + 0.625 * 2.0 + 0.3125 * -8.0) / l
    assert dec.tolist() == [[0]]
    assert abs(o[0, 0] - want) < 1e-15 and abs(lse[0] - math.log(l)) < 1e-15


def _two_tile_row(s1):
    """One row, 128 keys: key 0 scores 0 (V 1), key 64 scores s1 (V 2), the
    rest -50 (V 0)."""
    k = np.full((128, 1), -50.0)
    k[0, 0], k[64, 0] = 0.0, s1
    vv = np.zeros((128, 1))
    vv[0, 0], vv[64, 0] = 1.0, 2.0
    return fp8pv.pv8_blocks(np.ones((1, 1)), k, vv, 1.0, 0, False, math.inf)


def test_reference_stays_below_the_margin():
    # s1 = 3 < 8 ln 2: m_ref stays 0, key 64's weight e^3 = 20.09 rounds to 20
    # (spacing 2 in [16, 32)); a reference moved to 3 would give
    # (E4M3(e^-3) + 2) / (e^-3 + 1) = 1.9535 instead
    o, lse, _, _, _, _ = _two_tile_row(3.0)
    l = 1.0 + math.exp(3.0) + 126 * math.exp(-50.0)
    assert abs(o[0, 0] - (1.0 + 20.0 * 2.0) / l) < 1e-12
    assert abs(lse[0] - math.log(l)) < 1e-12


def test_reference_moves_past_the_margin():
    # s1 = 7 > 8 ln 2: m_ref moves to 7 at tile 1, tile 0's sums are scaled by
    # e^-7 and key 64 enters with weight 1
    o, lse, _, _, _, _ = _two_tile_row(7.0)
    a = math.exp(-7.0)
    l = a * (1.0 + 63 * math.exp(-50.0)) + 1.0 + 63 * math.exp(-57.0)
    assert abs(o[0, 0] - (a * 1.0 + 2.0) / l) < 1e-12
    assert abs(lse[0] - (7.0 + math.log(l))) < 1e-12


def test_head_scale_and_codes():
    # largest |v| 3.5 -> s = 3.5 / 448 = 2^-7; 3.5 / s = 448 = 1.75 * 2^8:
    # code 15 << 3 | 6 = 0x7E; -0.25 / s = -32 = -2^5: 0x80 | 12 << 3 = 0xE0;
    # 0.01 / s = 1.28 (fp32): spacing 1/8 in [1, 2), 10.24 -> 10: 1.25 =
    # 7 << 3 | 2 = 0x3A
    v = np.zeros((2, 1, 70, 4), np.float32)
    v[1, 0, 5, 2] = 3.5
    v[1, 0, 9, 1] = -0.25
    v[1, 0, 69, 3] = 0.01
    codes, s = fp8pv.quantize_v(v)
    assert s.shape == (2, 1) and s[0, 0] == 1.0 and s[1, 0] == np.float32(2.0 ** -7)
    assert codes[1, 0, 5, 2] == 0x7E and codes[1, 0, 9, 1] == 0xE0 and codes[1, 0, 69, 3] == 0x3A
    assert not codes[0].any()


def test_layout_positions_by_hand():
    N, d = 70, 16
    codes = ((np.arange(N)[:, None] * 3 + np.arange(d)[None, :]) % 251 + 1).astype(np.uint8)
    out = fp8pv.v_layout(codes)
    assert out.shape == (2, d, 64)
    # key 9 = 8 * 1 + 1 -> index 4 * 1 + 1 = 5, chunk 0; channel 5: chunk 0 ^ 1
    assert out[0, 5, 21] == codes[9, 5]
    # key 44 = 32 + 8 + 4 -> index 32 + 16 + 4 = 52, chunk 3; channel 12: 3 ^ 3 = 0
    assert out[0, 12, 4] == codes[44, 12]
    # key 66 (tile 1, key 2) -> index 2; channel 0
    assert out[1, 0, 2] == codes[66, 0]
    # key 69 (tile 1, key 5 = 4 + 1) -> index 33, chunk 2; channel 7: 2 ^ 1 = 3
    assert out[1, 7, 49] == codes[69, 7]
    # tile 1, key 6 (= key 70, past N) -> index 34; channel 0: code 0
    assert out[1, 0, 34] == 0
    # every full tile row is a permutation of its channel's 64 codes
    for c in range(d):
        assert sorted(out[0, c].tolist()) == sorted(codes[:64, c].tolist())


def test_prefill_decisions_are_the_qk8_oracles():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, d = 1, 2, 1, 200, 32

    def bf16(x):
        b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
        return (((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)).view(np.float32)
    q = bf16(rng.standard_normal((B, Hq, N, d)))
    k = bf16(rng.standard_normal((B, Hkv, N, d)) * 2)
    v = bf16(rng.standard_normal((B, Hkv, N, d)))
    for tau in (math.inf, 1.0):
        got = fp8pv.prefill(q, k, v, True, tau, qk8=True)
        want = fp8.prefill_qk8(q, k, v, True, tau)
        assert np.array_equal(got["mask"], want["mask"])
        # 3-bit probabilities and V: close to, not equal to, the 16-bit path
        assert np.abs(got["o"] - want["o"]).max() < 0.2
        assert np.abs(got["lse"] - want["lse"]).max() < 1e-12


def test_every_grown_row_moves_with_the_block():
    # two rows of one block; at tile 1 row A grows by 7 (past 8 ln 2) and row
    # B by 2: the move takes every grown row to its running maximum, so row
    # B's key 64 enters with weight 1 (not E4M3(e^2) = 7.5) and its tile 0
    # sums are scaled by e^-2
    d = 2
    k = np.full((128, d), -50.0)
    k[0] = [0.0, 0.0]
    k[64] = [7.0, 2.0]
    k *= math.sqrt(d)
    vv = np.zeros((128, 1))
    vv[0, 0], vv[64, 0] = 1.0, 2.0
    q = np.eye(2)
    o, lse, _, _, _, _ = fp8pv.pv8_blocks(q, k, vv, 1.0, 0, False, math.inf)
    for row, grow in ((0, 7.0), (1, 2.0)):
        a = math.exp(-grow)
        l = a * (1.0 + 63 * math.exp(-50.0)) + 1.0 + 63 * math.exp(-50.0 - grow)
        assert abs(o[row, 0] - (a + 2.0) / l) < 1e-12
        assert abs(lse[row] - (grow + math.log(l))) < 1e-12
