"""GPU parity on seeded random shapes: batch, head counts and group sizes,
ragged lengths, both head sizes, causal or not, structured or plain inputs,
several tau. Every case compares full outputs with the fp64 oracle through
the C ABI (skip masks exact except near-margin tiles, O within 1e-2, LSE
within 1e-3; 4-bit and 2-bit codes bit for bit; the SAS decodes against the
SAS oracle)."""
import math

import numpy as np
import pytest

import synth
from oracle import kvq2, kvq4
from tests import _parity

pytestmark = pytest.mark.gpu
INF = math.inf


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _taus(rng):
    return (INF, float(np.round(rng.uniform(0.5, 8.0), 2)), 0.0)


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        cfg = dict(kind="prefill", id=200 + i, B=int(rng.integers(1, 3)), Hq=G * Hkv,
                   Hkv=Hkv, N=int(rng.integers(1, 700)), d=int(rng.choice([64, 128])),
                   causal=bool(rng.integers(2)), sinks=bool(rng.integers(2)),
                   band=bool(rng.integers(2)))
        out.append((f"p{i}_B{cfg['B']}_H{cfg['Hq']}x{Hkv}_N{cfg['N']}_d{cfg['d']}"
                    f"{'_c' if cfg['causal'] else ''}", cfg, _taus(rng)))
    return out


def _decode_cases(n, seed, base_id):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.integers(1, 3))
        G = int(rng.integers(1, 17))
        cfg = dict(kind="decode", id=base_id + i, B=int(rng.integers(1, 4)), Hq=G * Hkv,
                   Hkv=Hkv, L=int(rng.integers(1, 9000)), d=int(rng.choice([64, 128])),
                   sinks=bool(rng.integers(2)), window=bool(rng.integers(2)))
        out.append((f"d{i}_B{cfg['B']}_H{cfg['Hq']}x{Hkv}_L{cfg['L']}_d{cfg['d']}", cfg,
                    _taus(rng)))
    return out


PREFILL = _prefill_cases(24, 2026)
DECODE = _decode_cases(16, 2027, 240)
DECODE_Q4 = _decode_cases(12, 2028, 270)
DECODE_Q2 = _decode_cases(8, 2029, 290)
DECODE_SAS = _decode_cases(10, 2030, 300)


@pytest.mark.parametrize("name,cfg,taus", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_random_shape(name, cfg, taus):
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    for tau in taus:
        print(f"[random] {name} tau={tau}", flush=True)
        o, lse, mask = lib.prefill(dq, dk, dv, cfg["causal"], tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_prefill(q, k, v, cfg["causal"], tau, o.cpu().numpy(),
                                    lse.cpu().numpy(), mask.cpu().numpy())
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("name,cfg,taus", PREFILL[:10], ids=[c[0] for c in PREFILL[:10]])
def test_prefill_chunk_random_start(name, cfg, taus):
    """A chunk at the end of the sequence: causal chunks start on a tile
    boundary, non-causal ones anywhere."""
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_prefill(cfg)
    N = q.shape[2]
    rng = np.random.default_rng(cfg["id"])
    q0 = int(rng.integers(0, N))
    if cfg["causal"]:
        q0 -= q0 % 64
    dk, dv = _dev(k), _dev(v)
    for tau in taus[:2]:
        print(f"[random] chunk {name} q0={q0} tau={tau}", flush=True)
        o, lse, mask = lib.prefill_chunk(_dev(q[:, :, q0:]), dk, dv, cfg["causal"], tau,
                                         want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_prefill(q[:, :, q0:], k, v, cfg["causal"], tau, o.cpu().numpy(),
                                    lse.cpu().numpy(), mask.cpu().numpy(), q0=q0)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("name,cfg,taus", DECODE, ids=[c[0] for c in DECODE])
def test_decode_random_shape(name, cfg, taus):
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_decode(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    for tau in taus:
        print(f"[random] {name} tau={tau}", flush=True)
        o, lse, mask = lib.decode(dq, dk, dv, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, k, v, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy())
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def _quantized_case(width, name, cfg, taus, sas=0):
    import torch
    import long_context_tiled_amd as lib
    codec = {4: kvq4, 2: kvq2}[width]
    quantize = {4: lib.quantize_q4, 2: lib.quantize_q2}[width]
    decode = {4: lib.decode_q4, 2: lib.decode_q2}[width]
    q, k, v = synth.make_decode(cfg)
    L = k.shape[2]
    Hkv = k.shape[1]
    print(f"[random] q{width} {name}: quantise", flush=True)
    cache = quantize(_dev(k), _dev(v))
    torch.cuda.synchronize()
    enc = codec.encode(synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v))
    got = {n: t.cpu().numpy() for n, t in cache.items()}
    for n in ("kq", "kp", "vq", "vp"):
        g = got[n].view(np.uint32) if n in ("kp", "vp") else got[n]
        assert np.array_equal(g, enc[n]), f"{n} differs from the oracle's encoding"

    def kv_for(b, g):
        return (codec.decode_k(enc["kq"][b, g], enc["kp"][b, g]),
                codec.decode_v(enc["vq"][b, g], enc["vp"][b, g], L))
    dq = _dev(q)
    for tau in taus:
        print(f"[random] q{width} {name} tau={tau}", flush=True)
        o, lse, mask = decode(dq, cache, L, tau, want_mask=True, sas=sas)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), kv_for=kv_for, Hkv=Hkv, sas=sas)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("name,cfg,taus", DECODE_Q4, ids=[c[0] for c in DECODE_Q4])
def test_decode_q4_random_shape(name, cfg, taus):
    _quantized_case(4, name, cfg, taus)


@pytest.mark.parametrize("name,cfg,taus", DECODE_Q2, ids=[c[0] for c in DECODE_Q2])
def test_decode_q2_random_shape(name, cfg, taus):
    _quantized_case(2, name, cfg, taus)


@pytest.mark.parametrize("name,cfg,taus", DECODE_SAS, ids=[c[0] for c in DECODE_SAS])
def test_decode_sas_random_shape(name, cfg, taus):
    """SAS decodes on random shapes: the bf16 cache for every case, then the
    4-bit or 2-bit cache by turns; degree 2 or 3 by turns."""
    import torch
    import long_context_tiled_amd as lib
    degree = 2 + cfg["id"] % 2
    q, k, v = synth.make_decode(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    for tau in taus[:2]:
        print(f"[random] sas{degree} {name} tau={tau}", flush=True)
        o, lse, mask = lib.decode(dq, dk, dv, tau, want_mask=True, sas=degree)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, k, v, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), sas=degree)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
    _quantized_case(4 if cfg["id"] % 4 < 2 else 2, name, cfg, taus[:1], sas=degree)


PREFILL8 = PREFILL[1::2]      # 12 of the shapes, each run in one 8-bit format
_FORMATS8 = ("qk_fp8", "qk_int8", "pv8_qk_bf16", "pv8_qk_fp8")


@pytest.mark.parametrize("name,cfg,taus", PREFILL8, ids=[c[0] for c in PREFILL8])
def test_prefill_8bit_random_shape(name, cfg, taus):
    """The 8-bit prefills on random shapes, the format by turns: fp8 or int8
    QK^T against the exact oracle on the dequantised Q and K; fp8 P.V (QK^T
    in bf16 or fp8) against the 8-bit P.V oracle with its rounding slack."""
    import torch
    import long_context_tiled_amd as lib
    from oracle import fp8, int8
    fmt = _FORMATS8[(cfg["id"] // 2) % 4]
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    qk_enc = int8 if fmt == "qk_int8" else fp8
    qf = kf = None
    if fmt != "pv8_qk_bf16":
        qc, qs = qk_enc.quantize(synth.bf16_bits_to_f32(q))
        kc, ks = qk_enc.quantize(synth.bf16_bits_to_f32(k))
        qf, kf = qk_enc.dequantize(qc, qs), qk_enc.dequantize(kc, ks)
    blocks = q.shape[0] * q.shape[1] * ((q.shape[2] + 63) // 64)
    for tau in taus:
        print(f"[random] {fmt} {name} tau={tau}", flush=True)
        if fmt.startswith("qk_"):
            o, lse, mask, _ = lib.prefill_qk8(dq, dk, dv, cfg["causal"], tau, want_mask=True,
                                              int8=fmt == "qk_int8")
            kw = {}
        else:
            qk8 = fmt == "pv8_qk_fp8"
            o, lse, mask, _ = lib.prefill_pv8(dq, dk, dv, cfg["causal"], tau, qk8=qk8,
                                              want_mask=True)
            kw = dict(pv8=True, score_err_rel=2.0 ** -11 if qk8 else 2.0 ** -17, lin_err=qk8)
        torch.cuda.synchronize()
        rep = _parity.check_prefill(q, k, v, cfg["causal"], tau, o.cpu().numpy(),
                                    lse.cpu().numpy(), mask.cpu().numpy(), qf=qf, kf=kf, **kw)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
        assert rep.ambiguous <= max(1, blocks // 20), str(rep)
