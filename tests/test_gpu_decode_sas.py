"""GPU parity of attn_decode_sas (the decode with the SAS exponential)
against the SAS decode oracle: skip masks as for the exact decode (and equal
to the exact decode's), O within 1e-2 and LSE within 1e-3 beyond the
oracle's bound for arguments lying on a step of SAS."""
import math

import numpy as np
import pytest

import synth
from tests import _parity

pytestmark = pytest.mark.gpu
INF = math.inf


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _cfg(**kw):
    base = dict(kind="decode", B=2, Hq=8, Hkv=2, L=10000, d=128, sinks=True, window=True)
    base.update(kw)
    return base


CASES = [
    ("gqa4_ragged_3splits", _cfg(id=110), (INF, 4.0)),
    ("g1_d64_one_split", _cfg(B=1, Hq=2, Hkv=2, L=4096, d=64, id=111), (INF, 2.0)),
    ("g8_split_edge", _cfg(B=1, Hq=8, Hkv=1, L=4097, id=112), (INF, 0.0)),
    ("g16_short", _cfg(B=1, Hq=16, Hkv=1, L=65, id=113, sinks=False), (INF, 3.0)),
    ("g3_d64_plain", _cfg(B=3, Hq=6, Hkv=2, L=12345, d=64, id=114, sinks=False, window=False),
     (INF, 1.0)),
]


@pytest.mark.parametrize("degree", [2, 3])
@pytest.mark.parametrize("name,cfg,taus", CASES, ids=[c[0] for c in CASES])
def test_decode_sas_small(name, cfg, taus, degree):
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_decode(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    for tau in taus:
        print(f"[sas] {name} degree={degree} tau={tau}", flush=True)
        o, lse, mask = lib.decode(dq, dk, dv, tau, want_mask=True, sas=degree)
        _, _, mask0 = lib.decode(dq, dk, dv, tau, want_mask=True)
        torch.cuda.synchronize()
        assert torch.equal(mask, mask0), "SAS must not change the skip decisions"
        rep = _parity.check_decode(q, k, v, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), sas=degree)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_degree_zero_is_the_exact_decode():
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_decode(_cfg(id=115))
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    print("[sas] degree 0 against attn_decode", flush=True)
    a = lib.decode(dq, dk, dv, 4.0, want_mask=True)
    b = lib.decode(dq, dk, dv, 4.0, want_mask=True, sas=0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bad_degree_is_rejected():
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_decode(_cfg(B=1, Hq=2, Hkv=1, L=100, id=116))
    with pytest.raises(lib.SkipAttnError) as e:
        lib.decode(_dev(q), _dev(k), _dev(v), INF, sas=4)
    assert e.value.code == lib.EINVAL
    torch.cuda.synchronize()


@pytest.mark.parametrize("degree", [2, 3])
def test_decode_sas_workload_sampled(degree):
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("decode_128k")
    print(f"[sas] generating decode_128k (degree {degree})", flush=True)
    q, k, v = synth.make_decode(cfg)
    B, Hq, d = q.shape
    rng = np.random.default_rng(7 + degree)
    heads = sorted({(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(6)}
                   | {(0, 0), (B - 1, Hq - 1)})
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    for tau in (INF, cfg["taus"][-1]):
        print(f"[sas] decode_128k degree={degree} tau={tau}", flush=True)
        o, lse, mask = lib.decode(dq, dk, dv, tau, want_mask=True, sas=degree)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, k, v, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), heads=heads, sas=degree)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
        del o, lse, mask


QCASES = [
    ("q_gqa4_ragged", _cfg(id=120), (INF, 4.0)),
    ("q_g8_d64_edge", _cfg(B=1, Hq=8, Hkv=1, L=4097, d=64, id=121), (INF, 2.0)),
    ("q_g16_plain", _cfg(B=1, Hq=16, Hkv=1, L=9000, id=122, sinks=False, window=False),
     (INF,)),
]


@pytest.mark.parametrize("width", [4, 2])
@pytest.mark.parametrize("degree", [2, 3])
@pytest.mark.parametrize("name,cfg,taus", QCASES, ids=[c[0] for c in QCASES])
def test_decode_quantized_sas(name, cfg, taus, degree, width):
    """The quantised cache and SAS together: against the SAS oracle on the
    oracle's dequantised cache."""
    import torch
    import long_context_tiled_amd as lib
    from oracle import kvq2, kvq4
    codec = {4: kvq4, 2: kvq2}[width]
    quantize = {4: lib.quantize_q4, 2: lib.quantize_q2}[width]
    decode = {4: lib.decode_q4, 2: lib.decode_q2}[width]
    q, k, v = synth.make_decode(cfg)
    Hkv, L = k.shape[1], k.shape[2]
    print(f"[sas] q{width} {name}: quantise", flush=True)
    cache = quantize(_dev(k), _dev(v))
    enc = codec.encode(synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v))

    def kv_for(b, g):
        return (codec.decode_k(enc["kq"][b, g], enc["kp"][b, g]),
                codec.decode_v(enc["vq"][b, g], enc["vp"][b, g], L))
    dq = _dev(q)
    for tau in taus:
        print(f"[sas] q{width} {name} degree={degree} tau={tau}", flush=True)
        o, lse, mask = decode(dq, cache, L, tau, want_mask=True, sas=degree)
        _, _, mask0 = decode(dq, cache, L, tau, want_mask=True)
        torch.cuda.synchronize()
        assert torch.equal(mask, mask0), "SAS must not change the skip decisions"
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), kv_for=kv_for, Hkv=Hkv, sas=degree)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
