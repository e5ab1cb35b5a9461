"""Pins for the fp64 oracle, against things other than itself.

* brute force: the literal scalar online-softmax loop (tests/_brute.py);
* the textbook special case tau = inf: torch's scaled_dot_product_attention
  and logsumexp in float64 on the CPU;
* hand-built cases whose decisions and outputs follow by hand
  (tests/golden/planted_tiles.json);
* closed forms and invariants: prefix-max form of the decisions, the
  dropped-mass bound 64 e^-tau per skipped tile, monotonicity in tau, the
  single-tile case, the decode split/merge identity.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "planted_tiles.json")
INF = math.inf


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _planted_prefill(N, d, causal, Hq=1, Hkv=1, seed=0, sink=8.0, band=0.0):
    """Random q/k/v whose first two keys score about ``sink`` logits above the
    rest for every query, so that later tiles get skipped; ``band`` adds a
    shared direction to the second half of queries and keys."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, N, d))
    k = rng.standard_normal((1, Hkv, N, d))
    v = rng.standard_normal((1, Hkv, N, d))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    c = math.sqrt(sink * math.sqrt(d))
    q += c * u
    k[:, :, :2] += c * u
    if band:
        w = rng.standard_normal(d)
        w /= np.linalg.norm(w)
        c = math.sqrt(band * math.sqrt(d))
        q[:, :, N // 2:] += c * w
        k[:, :, N // 2:] += c * w
    return q, k, v


def _np(x):
    return x.tolist()


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    # N, d, causal, tau, seed, sink
    (64, 8, False, 1.0, 1, 12.0),
    (100, 8, True, 0.0, 2, 6.0),
    (128, 8, False, 2.0, 3, 14.0),
    (128, 8, True, 4.0, 4, 16.0),
    (192, 8, True, 1.0, 5, 10.0),
    (200, 8, False, 0.5, 6, 12.0),
    (200, 8, True, INF, 7, 12.0),
    (130, 4, True, 3.0, 8, 12.0),
    (256, 8, True, 6.0, 9, 20.0),
]


@pytest.mark.parametrize("N,d,causal,tau,seed,sink", BRUTE_CASES)
def test_prefill_matches_brute_force(N, d, causal, tau, seed, sink):
    q, k, v = _planted_prefill(N, d, causal, seed=seed, sink=sink)
    ref = oracle.prefill(q, k, v, causal, tau)
    o, lse, dec = _brute.prefill_head(_np(q[0, 0]), _np(k[0, 0]), _np(v[0, 0]),
                                      causal, tau)
    np.testing.assert_array_equal(ref["mask"][0, 0], np.array(dec, np.uint8))
    np.testing.assert_allclose(ref["o"][0, 0], np.array(o), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"][0, 0], np.array(lse), rtol=0, atol=1e-12)


def test_brute_force_cases_exercise_skipping():
    """The planted cases above must actually skip tiles, or they pin nothing."""
    skipped = 0
    for N, d, causal, tau, seed, sink in BRUTE_CASES:
        q, k, v = _planted_prefill(N, d, causal, seed=seed, sink=sink)
        skipped += int((oracle.prefill(q, k, v, causal, tau)["mask"] == 1).sum())
    assert skipped >= 10


@pytest.mark.parametrize("L,split,tau,seed", [
    (256, 128, 1.0, 11), (300, 128, 0.5, 12), (448, 192, 2.0, 13),
    (512, 512, 0.0, 14), (257, 64, 1.5, 15), (384, 128, INF, 16)])
def test_decode_matches_brute_force(L, split, tau, seed):
    rng = np.random.default_rng(seed)
    d = 8
    qv = rng.standard_normal(d)
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    qv += 2.0 * u
    k[:3] += 4.0 * u                       # sinks in split 0 only
    k[-40:] += 3.0 * u                     # a recent window
    o, lse, dec, _ = oracle.decode_head(qv, k, v, tau, split=split)
    bo, blse, bdec = _brute.decode_head(_np(qv), _np(k), _np(v), tau, split)
    np.testing.assert_array_equal(dec, np.array(bdec, np.uint8))
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    assert abs(lse - blse) < 1e-12


# ---------------------------------------------------- textbook: tau = inf

@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [
    (1, 2, 2, 256, 64, False), (2, 4, 2, 130, 16, True), (1, 8, 1, 200, 32, True),
    (1, 3, 3, 64, 8, False), (1, 6, 2, 1, 16, True), (2, 4, 4, 70, 128, False)])
def test_dense_equals_torch_sdpa(B, Hq, Hkv, N, d, causal):
    rng = np.random.default_rng(B * 1000 + N)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    ref = oracle.prefill(q, k, v, causal, INF)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, enable_gqa=(Hq != Hkv))
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=1)
    s = (tq @ kk.transpose(-1, -2)) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    np.testing.assert_allclose(ref["o"], o.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"], lse.numpy(), rtol=0, atol=1e-12)
    assert (ref["mask"] != 1).all()


def test_decode_dense_equals_torch():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, d = 2, 8, 2, 1000, 32
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    ref = oracle.decode(q, k, v, INF, split=256)
    tq = torch.from_numpy(q)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, torch.from_numpy(k), torch.from_numpy(v), enable_gqa=True)[:, :, 0]
    s = (tq @ torch.from_numpy(k).repeat_interleave(Hq // Hkv, 1).transpose(-1, -2))
    lse = torch.logsumexp(s[:, :, 0] / math.sqrt(d), dim=-1)
    np.testing.assert_allclose(ref["o"], o.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"], lse.numpy(), rtol=0, atol=1e-12)
    assert (ref["mask"] == 0).all()


# ------------------------------------------------------------ golden cases

def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _planted_arrays(n, planted):
    d = 4
    q = np.zeros((n, d))
    q[:, 0] = 2.0
    k = np.zeros((n, d))
    v = np.zeros((n, d))
    v[:, 1] = 1.0
    for j, s in planted.items():
        k[int(j), 0] = s
        v[int(j), 0] = 1.0
    return q, k, v


def _tau(x):
    return INF if x == "inf" else float(x)


@pytest.mark.parametrize("case", _golden()["prefill"], ids=lambda c: c["name"])
def test_golden_prefill(case):
    n = case["N"]
    q, k, v = _planted_arrays(n, case["planted"])
    scores = np.zeros(n)
    for j, s in case["planted"].items():
        scores[int(j)] = s
    for c in case["cases"]:
        tau = _tau(c["tau"])
        ref = oracle.prefill(q[None, None], k[None, None], v[None, None],
                             case["causal"], tau)
        np.testing.assert_array_equal(ref["mask"][0, 0], np.array(c["mask"]))
        # closed form: softmax over the kept, causally valid keys of each row
        mask = np.array(c["mask"])
        for i in range(n):
            keys = [j for j in range(n)
                    if mask[i // 64, j // 64] == 0 and (not case["causal"] or j <= i)]
            z = sum(math.exp(scores[j]) for j in keys)
            lse = math.log(z)
            o0 = sum(math.exp(scores[j]) * v[j, 0] for j in keys) / z
            assert abs(ref["lse"][0, 0, i] - lse) < 1e-12
            assert abs(ref["o"][0, 0, i, 0] - o0) < 1e-12
            assert abs(ref["o"][0, 0, i, 1] - 1.0) < 1e-12


def _ranges(spec):
    out = set()
    for part in filter(None, spec.split(",")):
        a, _, b = part.partition("-")
        out.update(range(int(a), int(b or a) + 1))
    return out


@pytest.mark.parametrize("case", _golden()["decode"], ids=lambda c: c["name"])
def test_golden_decode(case):
    L = case["L"]
    q, k, v = _planted_arrays(L, case["planted"])
    scores = np.zeros(L)
    for j, s in case["planted"].items():
        scores[int(j)] = s
    for c in case["cases"]:
        tau = _tau(c["tau"])
        o, lse, dec, _ = oracle.decode_head(q[0], k, v, tau, split=case["split"])
        skipped = _ranges(c["skipped_tiles"])
        assert set(np.nonzero(dec == 1)[0].tolist()) == skipped
        keys = [j for j in range(L) if (j // 64) not in skipped]
        z = sum(math.exp(scores[j]) for j in keys)
        assert abs(lse - math.log(z)) < 1e-12
        assert abs(o[0] - sum(math.exp(scores[j]) * v[j, 0] for j in keys) / z) < 1e-12


# ------------------------------------------------- closed forms, invariants

def _scores_np(q, k, causal):
    n, d = q.shape
    s = q @ k.T / math.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    return s


@pytest.mark.parametrize("seed", range(6))
def test_decisions_equal_prefix_max_closed_form(seed):
    """For tau >= 0 a skipped tile never exceeds the running max, so the
    running max before tile kb equals the max over ALL keys before it."""
    rng = np.random.default_rng(100 + seed)
    N, d = 320, 16
    causal = bool(seed % 2)
    tau = [0.0, 0.5, 1.0, 2.0, 4.0, 3.0][seed]
    q, k, v = _planted_prefill(N, d, causal, seed=200 + seed, sink=14.0, band=3.0)
    ref = oracle.prefill(q, k, v, causal, tau)
    s = _scores_np(q[0, 0], k[0, 0], causal)
    nt = N // 64
    for qb in range(nt):
        rows = slice(qb * 64, qb * 64 + 64)
        for kb in range(nt):
            if causal and kb > qb:
                assert ref["mask"][0, 0, qb, kb] == 2
                continue
            t = s[rows, kb * 64:kb * 64 + 64].max(axis=1)
            p = s[rows, :kb * 64].max(axis=1) if kb else np.full(64, -np.inf)
            expect = bool(np.all(t < p - tau))
            assert ref["mask"][0, 0, qb, kb] == int(expect)


@pytest.mark.parametrize("tau", [0.0, 1.0, 2.0, 4.0])
def test_dropped_mass_bound_and_output_bounds(tau):
    """Per skipped tile and row: sum over the tile of e^(s-M) is at most
    64 e^-tau times the kept mass; hence bounds on LSE and O versus dense."""
    N, d = 384, 16
    q, k, v = _planted_prefill(N, d, True, seed=int(tau * 10) + 7, sink=20.0)
    sk = oracle.prefill(q, k, v, True, tau)
    dense = oracle.prefill(q, k, v, True, INF)
    assert (sk["mask"] == 1).sum() > 0
    s = _scores_np(q[0, 0], k[0, 0], True)
    mask = sk["mask"][0, 0]
    vmax = np.abs(v).max()
    for i in range(N):
        qb = i // 64
        row = s[i]
        M = sk["lse"][0, 0, i]  # LSE over kept keys = ln(kept mass)
        kept_mass = 1.0
        dropped = 0.0
        for kb in range(qb + 1):
            if mask[qb, kb] == 1:
                tile = np.exp(row[kb * 64:kb * 64 + 64] - M)
                tile = tile[np.isfinite(row[kb * 64:kb * 64 + 64])]
                assert tile.sum() <= 64 * math.exp(-tau) * kept_mass * (1 + 1e-12)
                dropped += tile.sum()
        delta = dropped / kept_mass
        gap = dense["lse"][0, 0, i] - sk["lse"][0, 0, i]
        assert -1e-12 <= gap <= math.log1p(delta) + 1e-12
        err = np.abs(dense["o"][0, 0, i] - sk["o"][0, 0, i]).max()
        assert err <= 2 * delta / (1 + delta) * vmax + 1e-12


def test_global_row_max_is_never_dropped():
    q, k, v = _planted_prefill(448, 16, True, seed=3, sink=16.0, band=4.0)
    for tau in (0.0, 1.0, 3.0):
        r = oracle.prefill(q, k, v, True, tau)
        s = _scores_np(q[0, 0], k[0, 0], True)
        mask = np.repeat(np.repeat(r["mask"][0, 0] == 0, 64, 0), 64, 1)
        kept_max = np.where(mask & np.isfinite(s), s, -np.inf).max(axis=1)
        np.testing.assert_array_equal(kept_max, s.max(axis=1))


def test_monotone_in_tau():
    q, k, v = _planted_prefill(512, 16, True, seed=9, sink=16.0, band=4.0)
    taus = [INF, 8.0, 4.0, 2.0, 1.0, 0.0]
    masks = [oracle.prefill(q, k, v, True, t)["mask"] == 1 for t in taus]
    assert not masks[0].any()
    for a, b in zip(masks, masks[1:]):
        assert (a <= b).all()  # skip(tau1) is a subset of skip(tau2), tau1 > tau2
    assert masks[-1].sum() > masks[2].sum() > 0


def test_single_tile_is_dense():
    q, k, v = _planted_prefill(64, 32, False, seed=4, sink=20.0)
    for tau in (0.0, 1.0):
        a = oracle.prefill(q, k, v, False, tau)
        b = oracle.prefill(q, k, v, False, INF)
        assert (a["mask"] == 0).all()
        np.testing.assert_array_equal(a["o"], b["o"])


def test_decode_split_merge_identity():
    """Each split's kept-set softmax, merged by log-sum-exp, equals the
    decode oracle's direct softmax over the union of kept keys."""
    rng = np.random.default_rng(21)
    L, d, split = 1000, 16, 256
    qv = rng.standard_normal(d) * 1.5
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    k[:2] += 3 * qv / np.linalg.norm(qv)
    for tau in (INF, 2.0, 0.5):
        o, lse, dec, _ = oracle.decode_head(qv, k, v, tau, split=split)
        parts = []
        for s0 in range(0, L, split):
            po, pl, pd, _ = oracle.decode_head(qv, k[s0:s0 + split], v[s0:s0 + split],
                                               tau, split=split)
            parts.append((pl, po))
            np.testing.assert_array_equal(pd, dec[s0 // 64:s0 // 64 + len(pd)])
        big = max(p[0] for p in parts)
        w = np.array([math.exp(p[0] - big) for p in parts])
        merged_lse = big + math.log(w.sum())
        merged_o = sum(wi * p[1] for wi, p in zip(w, parts)) / w.sum()
        assert abs(merged_lse - lse) < 1e-12
        np.testing.assert_allclose(merged_o, o, rtol=0, atol=1e-12)


def test_decode_single_split_equals_prefill_row_rule():
    """With one split, decode of a query equals a one-row non-causal block."""
    rng = np.random.default_rng(31)
    L, d = 640, 16
    qv = rng.standard_normal(d)
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    k[5] += 4 * qv
    for tau in (INF, 1.0, 3.0):
        o, lse, dec, _ = oracle.decode_head(qv, k, v, tau, split=4096)
        po, pl, pd, _ = oracle.prefill_blocks(qv[None, :], k, v, 0, False, tau)
        np.testing.assert_array_equal(dec, pd[0])
        np.testing.assert_allclose(o, po[0], rtol=0, atol=1e-13)
        assert abs(lse - pl[0]) < 1e-13


def test_forced_decisions_override():
    q, k, v = _planted_prefill(256, 16, False, seed=41, sink=16.0)
    r = oracle.prefill(q, k, v, False, 1.0)
    forced = np.full(r["mask"].shape, -1, np.int8)
    flip = np.argwhere(r["mask"] == 1)
    assert len(flip) > 0
    b, h, qb, kb = flip[0]
    forced[b, h, qb, kb] = 0
    r2 = oracle.prefill(q, k, v, False, 1.0, forced=forced)
    assert r2["mask"][b, h, qb, kb] == 0
    assert (np.delete(r2["mask"].ravel(), np.ravel_multi_index((b, h, qb, kb), r2["mask"].shape))
            == np.delete(r["mask"].ravel(), np.ravel_multi_index((b, h, qb, kb), r["mask"].shape))).all()
    dense = oracle.prefill(q, k, v, False, INF)
    rows = slice(qb * 64, qb * 64 + 64)
    # the q-block with the tile restored is closer to dense than before
    assert np.abs(r2["lse"][b, h, rows] - dense["lse"][b, h, rows]).max() <= \
        np.abs(r["lse"][b, h, rows] - dense["lse"][b, h, rows]).max()


def test_margin_sign_matches_decision():
    q, k, v = _planted_prefill(384, 16, True, seed=51, sink=16.0, band=4.0)
    for tau in (0.5, 2.0):
        r = oracle.prefill(q, k, v, True, tau)
        vis = r["mask"] != 2
        assert ((r["margin"][vis] > 0) == (r["mask"][vis] == 1)).all()


def test_parity_error_measure_refuses_nan():
    from tests import _parity
    assert _parity.max_abs_err([1.0, 2.0], [1.0, 2.5]) == 0.5
    assert _parity.max_abs_err([1.0, float("nan")], [1.0, 2.0]) == float("inf")
    assert _parity.max_abs_err([1.0], [float("inf")]) == float("inf")
    r = _parity.Report(o_err=_parity.max_abs_err([float("nan")], [0.0]))
    assert not r.ok()


def test_decisions_only_path_equals_full_blocks():
    # the decisions-only entry (scores and tile maxima once, the rule per tau)
    # gives the decisions and margins of the full block oracle
    rng = np.random.default_rng(11)
    N, d = 700, 64
    u = rng.normal(size=d)
    u /= np.linalg.norm(u)
    q = rng.normal(size=(N, d)) + 0.5 * math.sqrt(d) * u
    k = rng.normal(size=(N, d))
    k[:3] += 6.0 * math.sqrt(d) * u   # sink keys ~24 logits up: later tiles skip
    v = rng.normal(size=(N, d))
    for causal in (True, False):
        for qb0, nrows in ((0, 256), (4, 700 - 256)):
            rows = q[qb0 * 64:qb0 * 64 + nrows]
            got = oracle.prefill_decisions(rows, k, qb0, causal, (math.inf, 4.0, 1.0))
            for tau, (dec, margin) in got.items():
                _, _, dref, mref = oracle.prefill_blocks(rows, k, v, qb0, causal, tau)
                assert np.array_equal(dec, dref)
                assert np.array_equal(margin, mref, equal_nan=True)
            assert (got[1.0][0] == oracle.SKIPPED).any()


def test_decode_heads_is_decode_head_per_head():
    # the multi-head decode oracle: per head, the decisions and margins of
    # the one-head call, outputs to rounding, forced decisions honoured
    rng = np.random.default_rng(12)
    L, d = 9000, 64
    u = rng.normal(size=d)
    u /= np.linalg.norm(u)
    qs = rng.normal(size=(5, d)) + 0.5 * math.sqrt(d) * u
    k = rng.normal(size=(L, d))
    k[[0, 4100, 8200]] += 6.0 * math.sqrt(d) * u
    v = rng.normal(size=(L, d))
    for tau in (math.inf, 4.0):
        o, lse, dec, margin = oracle.decode_heads(qs, k, v, tau)
        for i in range(5):
            o1, l1, d1, m1 = oracle.decode_head(qs[i], k, v, tau)
            assert np.array_equal(dec[i], d1)
            assert np.allclose(margin[i], m1, rtol=0, atol=1e-12)
            assert np.abs(o[i] - o1).max() < 1e-13 and abs(lse[i] - l1) < 1e-13
    assert (dec == oracle.SKIPPED).any()
    forced = np.full(dec.shape, -1, np.int8)
    forced[2, 3] = 1 - dec[2, 3]
    _, _, dec2, _ = oracle.decode_heads(qs, k, v, 4.0, forced=forced)
    assert dec2[2, 3] == forced[2, 3]
    assert np.array_equal(np.delete(dec2, 2, axis=0), np.delete(dec, 2, axis=0))
