"""The seeded input generator: determinism, bf16 encoding, structure."""
import math

import numpy as np
import pytest
import torch

import synth
from synth import gen


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        # exact ties between two bf16 neighbours, both parities
        ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3895314e38, 65504.0], np.float32),
    ])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_thread_independent(monkeypatch):
    cfg = dict(kind="prefill", B=2, Hq=4, Hkv=2, N=300, d=64, causal=True,
               sinks=True, band=True)
    a = synth.make_prefill(cfg, seed=7)
    monkeypatch.setattr(gen, "_threads", lambda: 1)
    b = synth.make_prefill(cfg, seed=7)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    c = synth.make_prefill(cfg, seed=8)
    assert not np.array_equal(a[0], c[0])


def test_decode_deterministic(monkeypatch):
    cfg = dict(kind="decode", B=2, Hq=8, Hkv=2, L=5000, d=128, sinks=True,
               window=True)
    a = synth.make_decode(cfg, seed=3)
    monkeypatch.setattr(gen, "_threads", lambda: 1)
    b = synth.make_decode(cfg, seed=3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_slice_independent_of_shape():
    """A (tensor, b, head) slice depends only on its own seed key."""
    small = dict(kind="prefill", id=5, B=1, Hq=2, Hkv=1, N=128, d=64)
    big = dict(kind="prefill", id=5, B=1, Hq=4, Hkv=2, N=128, d=64)
    a = synth.make_prefill(small)
    b = synth.make_prefill(big)
    np.testing.assert_array_equal(a[0][0, :2], b[0][0, :2])
    np.testing.assert_array_equal(a[1][0, 0], b[1][0, 0])


def test_sink_structure_reading_s():
    """Reading S: the 4 sink keys score about 0.5*6*sqrt(d) above the rest."""
    cfg = dict(kind="prefill", B=1, Hq=2, Hkv=1, N=512, d=128, causal=True,
               sinks=True, band=False)
    q, k, _ = (synth.bf16_bits_to_f64(x) for x in synth.make_prefill(cfg, reading="S"))
    s = q[0, 0] @ k[0, 0].T / math.sqrt(128)
    bonus = s[:, :4].mean() - s[:, 4:].mean()
    assert abs(bonus - 3 * math.sqrt(128)) < 2.0
    qp, kp, _ = (synth.bf16_bits_to_f64(x) for x in synth.make_prefill(cfg, reading="P"))
    sp = qp[0, 0] @ kp[0, 0].T / math.sqrt(128)
    assert abs(sp[:, :4].mean() - sp[:, 4:].mean()) < 1.0


def test_band_structure():
    """Same-chunk and previous-chunk keys get about sqrt(d) extra logits."""
    cfg = dict(kind="prefill", B=1, Hq=1, Hkv=1, N=1024, d=128, causal=True,
               sinks=False, band=True)
    q, k, _ = (synth.bf16_bits_to_f64(x) for x in synth.make_prefill(cfg))
    s = q[0, 0] @ k[0, 0].T / math.sqrt(128)
    i = np.arange(1024)
    c = i // 256
    same = (c[:, None] == c[None, :]) | (c[:, None] == c[None, :] + 1)
    far = c[:, None] >= c[None, :] + 2
    assert abs(s[same].mean() - s[far].mean() - math.sqrt(128)) < 1.5


def test_window_structure():
    cfg = dict(kind="decode", B=1, Hq=2, Hkv=1, L=8192, d=128, sinks=True,
               window=True)
    q, k, _ = (synth.bf16_bits_to_f64(x) for x in synth.make_decode(cfg))
    s = k[0, 0] @ q[0, 0] / math.sqrt(128)
    assert s[8192 - 4096:].mean() - s[4:4096].mean() > 0.8 * math.sqrt(128)
    assert s[:4].mean() - s[4:4096].mean() > 0.8 * 3 * math.sqrt(128)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_table(name):
    w = synth.workload(name)
    assert w["Hq"] % w["Hkv"] == 0 and w["d"] in (64, 128)
    assert math.isinf(w["taus"][0])
