"""Seeded synthetic inputs for the Skip-Softmax attention workloads.

This module holds no attention arithmetic. It draws Gaussian base tensors,
adds the additive structure each workload asks for (attention-sink keys, a
local band, a recent window), and encodes the result once to bfloat16 with
round-to-nearest-even. The fp64 oracle and the HIP library receive the same
bf16 bit patterns from here; neither side generates its own inputs.

Tensors are returned as ``numpy.uint16`` arrays holding bf16 bit patterns:
prefill ``q [B,Hq,N,d]``, ``k``/``v [B,Hkv,N,d]``; decode ``q [B,Hq,d]``,
``k``/``v [B,Hkv,L,d]`` (one query token per sequence). Every
(tensor, batch, head) slice has its own ``numpy`` PCG64 stream, seeded by
``SeedSequence([seed, workload_id, tensor_id, b, head])``, so a slice's bytes
do not depend on how many threads fill the array.

Structure (the "reading" argument, ``"S"`` canonical, ``"P"`` literal):
amplitudes are multiplied by ``f = sqrt(d)`` under reading S (per-coordinate
amplitudes, so a sink adds 0.5*6*sqrt(d) logits) and by ``f = 1`` under
reading P (unit-norm additions, a sink adds 3/sqrt(d) logits).

* sinks:  keys 0..3 of every (b, kv head) get ``+6 f u``, every query gets
  ``+0.5 f u``; ``u`` is one random unit vector per sequence, shared by all
  heads.
* band:   for kv head g and 256-position chunk c, a unit vector w[g,c];
  query i gets ``+a w[g, i//256]`` and key j gets
  ``+a (w[g, j//256] + w[g, j//256 + 1])`` with ``a = 1.0 f``. A query and
  a key in the same chunk, or the key one chunk earlier, share a direction,
  which covers every causal pair with ``i - j < 256``.
* window (decode): a unit vector w[b,g]; keys ``L-4096 .. L-1`` get
  ``+a w`` and the queries of the heads of g get ``+a w``, ``a = 1.0 f``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TILE = 64
SPLIT = 4096
BAND_CHUNK = 256
N_SINKS = 4
SINK_K_AMP = 6.0
SINK_Q_AMP = 0.5
BAND_AMP = 1.0
WINDOW_AMP = 1.0
WINDOW_KEYS = 4096
DEFAULT_SEED = 2026

INF = math.inf

# The five workloads: a tiny correctness case, three causal GQA prefills and
# one split-K decode, all at d = 128 except the tiny one.
WORKLOADS = {
    "tiny": dict(id=0, kind="prefill", B=1, Hq=2, Hkv=2, N=256, d=64,
                 causal=False, sinks=False, band=False, taus=(INF, 4.0)),
    "prefill_8k": dict(id=1, kind="prefill", B=1, Hq=32, Hkv=8, N=8192, d=128,
                       causal=True, sinks=True, band=False,
                       taus=(INF, 8.0, 4.0)),
    "prefill_32k": dict(id=2, kind="prefill", B=1, Hq=64, Hkv=8, N=32768,
                        d=128, causal=True, sinks=True, band=True,
                        taus=(INF, 8.0, 4.0, 2.0)),
    "prefill_128k": dict(id=3, kind="prefill", B=1, Hq=8, Hkv=1, N=131072,
                         d=128, causal=True, sinks=True, band=True,
                         taus=(INF, 12.0, 8.0, 4.0)),
    "decode_128k": dict(id=4, kind="decode", B=16, Hq=64, Hkv=8, L=131072,
                        d=128, sinks=True, window=True, taus=(INF, 8.0, 4.0)),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    v = rng.standard_normal(d)
    return (v / np.linalg.norm(v)).astype(np.float32)


def _amp_factor(d: int, reading: str) -> float:
    if reading == "S":
        return math.sqrt(d)
    if reading == "P":
        return 1.0
    raise ValueError(f"reading must be 'S' or 'P', got {reading!r}")


def workload(name_or_cfg) -> dict:
    """Return a workload dict (a copy) by name, or validate a custom dict."""
    if isinstance(name_or_cfg, str):
        cfg = dict(WORKLOADS[name_or_cfg])
        cfg["name"] = name_or_cfg
        return cfg
    cfg = dict(name_or_cfg)
    cfg.setdefault("id", 99)
    cfg.setdefault("name", "custom")
    cfg.setdefault("sinks", False)
    cfg.setdefault("band", False)
    cfg.setdefault("window", False)
    return cfg


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def _sink_vec(seed, wid, b, d):
    return _unit(_rng(seed, wid, 90, b), d)


def _band_vecs(seed, wid, b, g, n, d):
    nchunk = (n + BAND_CHUNK - 1) // BAND_CHUNK + 1
    rng = _rng(seed, wid, 91, b, g)
    return np.stack([_unit(rng, d) for _ in range(nchunk)])


def make_prefill(cfg, seed: int = DEFAULT_SEED, reading: str = "S"):
    """Generate bf16 (q, k, v) for a prefill workload.

    ``cfg`` is a workload name or a dict with keys B, Hq, Hkv, N, d and
    optional sinks / band flags (causality does not change the inputs).
    """
    cfg = workload(cfg)
    B, Hq, Hkv, N, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["d"]
    G = Hq // Hkv
    wid = cfg["id"]
    f = _amp_factor(d, reading)
    q = np.empty((B, Hq, N, d), np.uint16)
    k = np.empty((B, Hkv, N, d), np.uint16)
    v = np.empty((B, Hkv, N, d), np.uint16)
    chunk_of = np.arange(N) // BAND_CHUNK

    def job(args):
        tensor, b, h = args
        x = _rng(seed, wid, tensor, b, h).standard_normal(N * d, dtype=np.float32)
        x = x.reshape(N, d)
        if tensor == 0:  # query head h
            if cfg["sinks"]:
                x += np.float32(SINK_Q_AMP * f) * _sink_vec(seed, wid, b, d)
            if cfg["band"]:
                w = _band_vecs(seed, wid, b, h // G, N, d)
                x += np.float32(BAND_AMP * f) * w[chunk_of]
            q[b, h] = f32_to_bf16_bits(x)
        elif tensor == 1:  # key head h
            if cfg["sinks"]:
                x[:N_SINKS] += np.float32(SINK_K_AMP * f) * _sink_vec(seed, wid, b, d)
            if cfg["band"]:
                w = _band_vecs(seed, wid, b, h, N, d)
                x += np.float32(BAND_AMP * f) * (w[chunk_of] + w[chunk_of + 1])
            k[b, h] = f32_to_bf16_bits(x)
        else:  # value head h: no structure
            v[b, h] = f32_to_bf16_bits(x)

    jobs = [(0, b, h) for b in range(B) for h in range(Hq)]
    jobs += [(t, b, g) for t in (1, 2) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, jobs))
    return q, k, v


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _window_vec(seed, wid, b, g, d):
    return _unit(_rng(seed, wid, 92, b, g), d)


def make_decode(cfg, seed: int = DEFAULT_SEED, reading: str = "S"):
    """Generate bf16 (q [B,Hq,d], k [B,Hkv,L,d], v [B,Hkv,L,d]) for decode."""
    cfg = workload(cfg)
    B, Hq, Hkv, L, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["L"], cfg["d"]
    G = Hq // Hkv
    wid = cfg["id"]
    f = _amp_factor(d, reading)
    q = np.empty((B, Hq, d), np.uint16)
    k = np.empty((B, Hkv, L, d), np.uint16)
    v = np.empty((B, Hkv, L, d), np.uint16)
    wlo = max(0, L - WINDOW_KEYS)

    def job(args):
        tensor, b, h = args
        if tensor == 0:
            x = _rng(seed, wid, 0, b, h).standard_normal(d, dtype=np.float32)
            if cfg["sinks"]:
                x += np.float32(SINK_Q_AMP * f) * _sink_vec(seed, wid, b, d)
            if cfg.get("window"):
                x += np.float32(WINDOW_AMP * f) * _window_vec(seed, wid, b, h // G, d)
            q[b, h] = f32_to_bf16_bits(x)
            return
        x = _rng(seed, wid, tensor, b, h).standard_normal(L * d, dtype=np.float32)
        x = x.reshape(L, d)
        if tensor == 1:
            if cfg["sinks"]:
                x[:N_SINKS] += np.float32(SINK_K_AMP * f) * _sink_vec(seed, wid, b, d)
            if cfg.get("window"):
                x[wlo:] += np.float32(WINDOW_AMP * f) * _window_vec(seed, wid, b, h, d)
            k[b, h] = f32_to_bf16_bits(x)
        else:
            v[b, h] = f32_to_bf16_bits(x)

    jobs = [(0, b, h) for b in range(B) for h in range(Hq)]
    jobs += [(t, b, g) for t in (1, 2) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, jobs))
    return q, k, v


def make_inputs(cfg, seed: int = DEFAULT_SEED, reading: str = "S"):
    cfg = workload(cfg)
    if cfg["kind"] == "decode":
        return make_decode(cfg, seed, reading)
    return make_prefill(cfg, seed, reading)
