"""GPU parity of two boundary generalisations, against the fp64 oracle:

* decode with more than 16 query heads per KV head (one wave per slice of
  16 heads of a group; every head still decides on its own, per split);
* caches allocated for `cap` keys of which only the first L (N) exist: the
  bf16 decode, the 4-bit and 2-bit decodes over a cache appended chunk by
  chunk, and a chunked prefill into a preallocated cache. Rows past the
  attended length hold NaN (bf16) or all-ones bytes (codes and parameter
  words), so any read of them would show in the outputs.
"""
import math

import numpy as np
import pytest

import synth
from oracle import kvq2, kvq4
from tests import _parity

pytestmark = pytest.mark.gpu
INF = math.inf
NAN_BF16 = np.int16(0x7FC0)


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _np(t):
    return t.cpu().numpy()


WIDE = [  # (name, cfg): query heads per KV head beyond 16, ragged last slice
    ("g20", dict(kind="decode", id=120, B=1, Hq=40, Hkv=2, L=5000, d=128, sinks=True,
                 window=True)),
    ("g32_d64", dict(kind="decode", id=121, B=2, Hq=32, Hkv=1, L=4200, d=64, sinks=True,
                     window=True)),
]


@pytest.mark.parametrize("name,cfg", WIDE, ids=[w[0] for w in WIDE])
def test_decode_more_than_16_heads_per_group(name, cfg):
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_decode(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    L, Hkv = k.shape[2], k.shape[1]
    kf, vf = synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v)
    enc4, enc2 = kvq4.encode(kf, vf), kvq2.encode(kf, vf)
    c4, c2 = lib.quantize_q4(dk, dv), lib.quantize_q2(dk, dv)
    kv4 = lambda b, g: (kvq4.decode_k(enc4["kq"][b, g], enc4["kp"][b, g]),
                        kvq4.decode_v(enc4["vq"][b, g], enc4["vp"][b, g], L))
    kv2 = lambda b, g: (kvq2.decode_k(enc2["kq"][b, g], enc2["kp"][b, g]),
                        kvq2.decode_v(enc2["vq"][b, g], enc2["vp"][b, g], L))
    for tau in (INF, 4.0):
        print(f"[wide] {name} bf16 tau={tau}", flush=True)
        o, lse, m = lib.decode(dq, dk, dv, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, k, v, tau, _np(o), _np(lse), _np(m))
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
        for bits, cache, kv in ((4, c4, kv4), (2, c2, kv2)):
            print(f"[wide] {name} q{bits} tau={tau}", flush=True)
            fn = lib.decode_q4 if bits == 4 else lib.decode_q2
            o, lse, m = fn(dq, cache, L, tau, want_mask=True)
            torch.cuda.synchronize()
            rep = _parity.check_decode(q, None, None, tau, _np(o), _np(lse), _np(m),
                                       kv_for=kv, Hkv=Hkv)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)


def test_decode_partly_filled_bf16_cache():
    import torch
    import long_context_tiled_amd as lib
    cfg = dict(kind="decode", id=122, B=2, Hq=16, Hkv=2, L=6000, d=128, sinks=True, window=True)
    q, k, v = synth.make_decode(cfg)
    n, cap = k.shape[2], 9000
    kc = np.full(k.shape[:2] + (cap, k.shape[3]), NAN_BF16, np.int16)
    vc = kc.copy()
    kc[:, :, :n], vc[:, :, :n] = k, v
    dq, dk, dv = _dev(q), _dev(kc), _dev(vc)
    for tau in (INF, 4.0):
        for sas in (0, 2):
            print(f"[cap] bf16 L={n} cap={cap} tau={tau} sas={sas}", flush=True)
            o, lse, m = lib.decode(dq, dk, dv, tau, want_mask=True, sas=sas, L=n)
            torch.cuda.synchronize()
            rep = _parity.check_decode(q, k, v, tau, _np(o), _np(lse), _np(m), sas=sas)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)


@pytest.mark.parametrize("bits", [4, 2])
def test_decode_appended_quantised_cache(bits):
    # a cache sized for cap keys, appended in chunks (the first on tile
    # boundaries, the last one ragged), decoded at each length reached
    import torch
    import long_context_tiled_amd as lib
    enc_mod = kvq4 if bits == 4 else kvq2
    cfg = dict(kind="decode", id=123, B=2, Hq=8, Hkv=2, L=7000, d=128, sinks=True, window=True)
    q, k, v = synth.make_decode(cfg)
    cap = 10000
    kc = np.full(k.shape[:2] + (cap, k.shape[3]), NAN_BF16, np.int16)
    vc = kc.copy()
    kc[:, :, :k.shape[2]], vc[:, :, :k.shape[2]] = k, v
    dq, dk, dv = _dev(q), _dev(kc), _dev(vc)
    empty = lib.empty_q4 if bits == 4 else lib.empty_q2
    cache = empty(2, 2, cap, 128, dk.device)
    for t in cache.values():
        t.fill_(-1)                                  # all-ones bytes: NaN parameters
    quant = lib.attn_kv_quantize_q4 if bits == 4 else lib.attn_kv_quantize_q2
    decode = lib.decode_q4 if bits == 4 else lib.decode_q2
    k0 = 0
    for k1 in (4096, 5000, 7000):
        quant(dk, dv, cache, key_range=(k0, k1))
        k0 = (k1 // 64) * 64                         # the next chunk rewrites a partial tile
        enc = enc_mod.encode(synth.bf16_bits_to_f32(k[:, :, :k1]),
                             synth.bf16_bits_to_f32(v[:, :, :k1]))

        def kv_for(b, g, enc=enc, k1=k1):
            return (enc_mod.decode_k(enc["kq"][b, g], enc["kp"][b, g]),
                    enc_mod.decode_v(enc["vq"][b, g], enc["vp"][b, g], k1))
        for tau in (INF, 4.0):
            print(f"[cap] q{bits} L={k1} cap={cap} tau={tau}", flush=True)
            o, lse, m = decode(dq, cache, k1, tau, want_mask=True)
            torch.cuda.synchronize()
            rep = _parity.check_decode(q, None, None, tau, _np(o), _np(lse), _np(m),
                                       kv_for=kv_for, Hkv=2)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)


def test_prefill_chunk_into_preallocated_cache():
    import torch
    import long_context_tiled_amd as lib
    cfg = dict(kind="prefill", id=124, B=1, Hq=8, Hkv=2, N=1536, d=128, causal=True,
               sinks=True, band=True)
    q, k, v = synth.make_prefill(cfg)
    cap = 4096
    kc = np.full(k.shape[:2] + (cap, k.shape[3]), NAN_BF16, np.int16)
    vc = kc.copy()
    dq = _dev(q)
    for N, q0 in ((1024, 512), (1536, 1024), (1536, 0)):
        kc[:, :, :N], vc[:, :, :N] = k[:, :, :N], v[:, :, :N]
        dk, dv = _dev(kc), _dev(vc)
        for tau in (INF, 4.0):
            print(f"[cap] prefill chunk N={N} q0={q0} cap={cap} tau={tau}", flush=True)
            o, lse, m = lib.prefill_chunk(dq[:, :, q0:N].contiguous(), dk, dv, True, tau,
                                          want_mask=True, N=N)
            torch.cuda.synchronize()
            # the same chunk over exactly N keys gives the same bits
            o2, lse2, m2 = lib.prefill_chunk(dq[:, :, q0:N].contiguous(), dk[:, :, :N].contiguous(),
                                             dv[:, :, :N].contiguous(), True, tau, want_mask=True)
            torch.cuda.synchronize()
            assert np.array_equal(_np(o), _np(o2)) and np.array_equal(_np(lse), _np(lse2))
            assert np.array_equal(_np(m), _np(m2))
            rep = _parity.check_prefill(q[:, :, q0:N], k[:, :, :N], v[:, :, :N], True, tau,
                                        _np(o), _np(lse), _np(m), q0=q0)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)
