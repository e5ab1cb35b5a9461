"""Pins of the SAS oracle (oracle/sas.py) against facts outside its own
code: the least-squares property of the fit under numerical quadrature, the
table's values and cut, the approximation's error bounds, the exact decode
oracle (the online loop with exact exponentials) and the direct formula on
a single tile."""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle
from oracle import sas

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("degree", [2, 3])
def test_fit_residual_is_orthogonal_to_the_polynomials(degree):
    a = sas.poly_coeffs(degree)
    for i in range(degree + 1):
        val, err = integrate.quad(
            lambda f: (math.exp(-f) - np.polyval(a[::-1], f)) * f ** i, 0.0, 1.0,
            epsabs=1e-14)
        assert abs(val) < 1e-12, (degree, i, val)


def test_fit_errors_match_the_claims():
    f = np.linspace(0.0, 1.0, 200001)
    err = {dg: np.abs(np.exp(-f) - np.polyval(sas.poly_coeffs(dg)[::-1], f)).max()
           for dg in (2, 3)}
    # degree 2 "near lossless", degree 3 "almost lossless": a few 1e-3 and
    # a few 1e-4 of the largest output
    assert 5e-3 < err[2] < 6e-3
    assert 3e-4 < err[3] < 4e-4


@pytest.mark.parametrize("degree", [2, 3])
def test_table_and_cut(degree):
    a0 = sas.poly_coeffs(degree)[0]
    n = np.arange(6, dtype=np.float64)
    assert np.allclose(sas.sas_exp(n, degree), np.exp(-n) * a0, rtol=1e-15, atol=0)
    assert np.all(sas.sas_exp(np.array([6.0, 6.5, 40.0, np.inf]), degree) == 0.0)
    assert sas.sas_exp(np.array([5.999]), degree)[0] > 0.0
    with pytest.raises(ValueError):
        sas.sas_exp(np.array([-0.5]), degree)
    with pytest.raises(ValueError):
        sas.poly_coeffs(4)


@pytest.mark.parametrize("degree,bound", [(2, 1.3e-2), (3, 9.5e-4)])
def test_relative_error_below_the_cut(degree, bound):
    # SAS / e^-x = p(f) / e^-f: the table rows are exact
    x = np.linspace(0.0, 5.9999, 60001)
    rel = np.abs(sas.sas_exp(x, degree) / np.exp(-x) - 1.0)
    assert rel.max() < bound


def _head(seed, L, d=64, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=d) * scale
    k = rng.normal(size=(L, d))
    v = rng.normal(size=(L, d))
    # rising scores late in the sequence, so the running maximum rises often
    k[L // 2:] += 0.05 * q * np.linspace(0, 4, L - L // 2)[:, None]
    return q, k, v


@pytest.mark.parametrize("tau", [math.inf, 3.0, 0.5])
def test_online_loop_with_exact_exp_is_the_exact_oracle(tau):
    q, k, v = _head(1, 9000)
    o, lse, dec, _ = oracle.decode_head(q, k, v, tau, 4096)
    o2, lse2, dec2, _, _ = sas.decode_head(q, k, v, tau, 2, 4096,
                                           exp_fn=lambda x: np.exp(-x))
    assert np.array_equal(dec, dec2)
    assert abs(lse - lse2) < 1e-12
    assert np.abs(o - o2).max() < 1e-12


@pytest.mark.parametrize("degree", [2, 3])
def test_single_tile_is_the_direct_formula(degree):
    q, k, v = _head(2, 50)
    o, lse, dec, _, _ = sas.decode_head(q, k, v, math.inf, degree)
    s = k @ q / math.sqrt(q.size)
    p = sas.sas_exp(s.max() - s, degree)
    assert np.allclose(o, p @ v / p.sum(), rtol=0, atol=1e-13)
    assert abs(lse - (s.max() + math.log(p.sum()))) < 1e-13


def test_drift_from_exact_shrinks_with_degree_below_the_cut():
    # scores spread over less than 6 logits: only the polynomial differs
    q, k, v = _head(3, 9000, scale=0.5)
    s = k @ q / math.sqrt(q.size)
    assert s.max() - s.min() < 6.0
    o, lse, _, _ = oracle.decode_head(q, k, v, math.inf, 4096)
    err = {}
    for dg in (2, 3):
        o2, lse2, _, _, _ = sas.decode_head(q, k, v, math.inf, dg)
        err[dg] = (np.abs(o2 - o).max(), abs(lse2 - lse))
    assert err[3][0] < err[2][0] and err[3][1] < err[2][1]
    assert err[2][1] < 1.3e-2 and err[3][1] < 9.5e-4   # the relative error bounds


def test_the_cut_drops_keys_beyond_six_logits():
    # one dominant key and many keys 6.5 logits below it: SAS drops them all
    d = 8
    L = 200
    q = np.zeros(d)
    q[0] = math.sqrt(d)              # score = k[:, 0]
    k = np.zeros((L, d))
    k[0, 0] = 6.5
    v = np.zeros((L, d))
    v[0, 1] = 1.0
    v[1:, 2] = 1.0
    for dg in (2, 3):
        o, lse, _, _, _ = sas.decode_head(q, k, v, math.inf, dg)
        assert o[2] == 0.0 and o[1] == 1.0
        assert abs(lse - (6.5 + math.log(sas.poly_coeffs(dg)[0]))) < 1e-14
    o, lse, _, _ = oracle.decode_head(q, k, v, math.inf)
    assert o[2] > 0.2                # exact softmax keeps their mass


def test_slack_counts_arguments_at_the_steps():
    # one key exactly one unit below the maximum sits on a step of SAS
    d = 4
    k = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0]])
    q = np.array([1.0, 0, 0, 0])     # scores 1 and 0: the second at x = 1
    v = np.eye(2, d)
    _, _, _, _, (ls, os_) = sas.decode_head(q, k, v, math.inf, 2)
    assert ls > 0 and os_ > 0
    k[1, 0] = 0.5                    # x = 0.75: no step nearby
    _, _, _, _, (ls, os_) = sas.decode_head(q, k, v, math.inf, 2)
    assert ls == 0 and os_ == 0


def test_golden_two_tile_rescale_uses_sas():
    # A hand-derived case whose running maximum rises by 2.25 logits between
    # the two tiles: the expected O and LSE apply T[n] p(f) to the
    # probabilities and to the rescale factor alike (tests/golden).
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sas_two_tile.json")))
    d, L = 4, 128
    q = np.array([2.0, 0.0, 0.0, 0.0])
    k = np.zeros((L, d))
    k[:, 0] = -100.0
    k[0, 0] = 0.0
    k[64, 0] = 2.25
    v = np.zeros((L, d))
    v[:, 2] = 1.0
    v[0] = [1.0, 0.0, 0.0, 0.0]
    v[64] = [0.0, 1.0, 0.0, 0.0]
    for case in g["cases"]:
        dg = case["degree"]
        assert np.allclose(sas.poly_coeffs(dg), case["coeffs"], rtol=0, atol=1e-14)
        assert abs(float(sas.sas_exp(np.array([2.25]), dg)[0]) - case["alpha"]) < 1e-15
        o, lse, dec, _, _ = sas.decode_head(q, k, v, math.inf, dg)
        assert np.all(dec == oracle.KEPT)
        assert np.abs(o - np.array(case["o"])).max() < 1e-12, (dg, o)
        assert abs(lse - case["lse"]) < 1e-12, (dg, lse)
        # the case separates SAS on the rescale factor from an exact one
        assert np.abs(np.array(case["o"]) - np.array(case["o_if_alpha_exact"])).max() > 1e-6
        assert abs(case["lse"] - case["lse_if_alpha_exact"]) > 1e-6


# ---------------------------------------------------------------- prefill

def _prefill_case(seed, N, d=64, Hq=2, rising=True):
    """Rows whose running maximum rises over the tiles: later keys carry a
    growing share of a direction every query has."""
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(1, Hq, N, d)) / d ** 0.25
    k = rng.normal(size=(1, 1, N, d)) / d ** 0.25
    v = rng.normal(size=(1, 1, N, d))
    if rising:
        u = rng.normal(size=d)
        u /= np.linalg.norm(u)
        q += 1.5 * u
        k += (np.arange(N) / N * 3.0)[:, None] * u * d ** 0.5 / 1.5
    return q, k, v


@pytest.mark.parametrize("causal,tau", [(True, math.inf), (True, 2.0), (False, 1.0)])
def test_prefill_online_loop_with_exact_exp_is_the_exact_oracle(causal, tau):
    q, k, v = _prefill_case(11, 300)
    ex = oracle.prefill(q, k, v, causal, tau)
    r = sas.prefill(q, k, v, causal, tau, 2, exp_fn=lambda x: np.exp(-np.asarray(x)))
    assert np.array_equal(r["mask"], ex["mask"])
    assert np.abs(r["o"] - ex["o"]).max() < 1e-12
    assert np.abs(r["lse"] - ex["lse"]).max() < 1e-12


@pytest.mark.parametrize("degree", [2, 3])
def test_prefill_single_tile_is_the_direct_formula(degree):
    q, k, v = _prefill_case(12, 50, rising=False)
    r = sas.prefill(q, k, v, False, math.inf, degree)
    s = (q[0, 0] @ k[0, 0].T) / 8.0
    mx = s.max(axis=1, keepdims=True)
    p = sas.sas_exp(mx - s, degree)
    o = (p @ v[0, 0]) / p.sum(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(p.sum(axis=1))
    assert np.abs(r["o"][0, 0] - o).max() < 1e-12
    assert np.abs(r["lse"][0, 0] - lse).max() < 1e-12


@pytest.mark.parametrize("degree", [2, 3])
def test_prefill_rows_are_the_sas_decode_of_each_row(degree):
    """With no tile skipped, row i of a causal prefill attends keys 0..i in
    ascending tiles exactly as a one-token decode over those keys (one
    split): the SAS decode oracle, pinned by its own hand-derived two-tile
    case, fixes SAS on both the probabilities and the rescale factor here."""
    q, k, v = _prefill_case(13, 700, d=64)
    r = sas.prefill(q, k, v, True, math.inf, degree)
    rises = 0
    for h in range(2):
        for i in (0, 63, 64, 200, 411, 699):
            o, lse, dec, _, _ = sas.decode_head(q[0, h, i], k[0, 0, :i + 1], v[0, 0, :i + 1],
                                               math.inf, degree)
            assert np.abs(r["o"][0, h, i] - o).max() < 1e-12, (h, i)
            assert abs(r["lse"][0, h, i] - lse) < 1e-12, (h, i)
        s = (q[0, 0] @ k[0, 0].T) / 8.0
        tm = np.array([s[699, 64 * t:64 * t + 64].max() for t in range(11)])
        rises += int((np.diff(np.maximum.accumulate(tm)) > 0).sum())
    assert rises > 4  # the case does exercise the rescale factor


def test_prefill_differs_from_exact_alpha():
    """An oracle that used the exact exponential for the rescale factor (and
    SAS only on the probabilities) is told apart by these inputs."""
    q, k, v = _prefill_case(14, 640)
    r = sas.prefill(q, k, v, True, math.inf, 2)

    def mixed(x):
        return sas.sas_exp(x, 2)
    # rebuild the per-row loop with exact alpha by brute force for one row
    i, d = 639, 64
    s = (q[0, 0, i] @ k[0, 0, :i + 1].T) / 8.0
    m, acc, l = -np.inf, np.zeros(d), 0.0
    for t in range(10):
        st = s[64 * t:64 * t + 64]
        mn = max(m, st.max())
        if mn > m:
            a = 0.0 if not np.isfinite(m) else math.exp(-(mn - m))
            acc, l, m = acc * a, l * a, mn
        p = mixed(m - st)
        acc += p @ v[0, 0, 64 * t:64 * t + 64]
        l += p.sum()
    assert abs(m + math.log(l) - r["lse"][0, 0, i]) > 1e-4
