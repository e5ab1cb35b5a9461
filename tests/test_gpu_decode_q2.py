"""GPU parity of the 2-bit KV cache: the quantiser against the oracle's
encoder bit for bit, and attn_decode_q2 against the fp64 decode oracle run
on the oracle's dequantised cache (same tolerances as the bf16 decode)."""
import math

import numpy as np
import pytest

import synth
from oracle import kvq2
from tests import _parity
from tests.test_gpu_decode_q4 import _assert_same_cache, _cfg, _dev, _host, _rand_kv

pytestmark = pytest.mark.gpu
INF = math.inf


def _oracle_kv(enc, L):
    def kv_for(b, g):
        return (kvq2.decode_k(enc["kq"][b, g], enc["kp"][b, g]),
                kvq2.decode_v(enc["vq"][b, g], enc["vp"][b, g], L))
    return kv_for


def _encode(k, v):
    return kvq2.encode(synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v))


QCASES = [  # (B, Hkv, L, d, seed, scale)
    (1, 1, 1, 128, 1, 1.0), (1, 2, 63, 64, 2, 1.0), (2, 1, 64, 128, 3, 1.0),
    (1, 3, 65, 64, 4, 30.0), (2, 2, 4097, 128, 5, 1.0), (1, 1, 1000, 128, 6, 1e-3),
    (1, 2, 300, 64, 7, 1e4),
]


@pytest.mark.parametrize("B,Hkv,L,d,seed,scale", QCASES)
def test_quantiser_bit_exact(B, Hkv, L, d, seed, scale):
    import torch
    import long_context_tiled_amd as lib
    k, v = _rand_kv(B, Hkv, L, d, seed, scale)
    k[0, 0, 0, :] = k[0, 0, 0, 0]                   # a constant K row
    v[0, 0, : min(L, 64), 0] = v[0, 0, 0, 0]         # a constant V block
    print(f"[q2] quantise B={B} Hkv={Hkv} L={L} d={d} seed={seed}", flush=True)
    got = _host(lib.quantize_q2(_dev(k), _dev(v)))
    torch.cuda.synchronize()
    _assert_same_cache(got, _encode(k, v))


def _on_ties(rng, shape):
    """bf16 blocks along the last axis whose codes sit on rounding ties: each
    block holds its minimum z and z + 3 s0 (s0 a power of two, so s = s0),
    and otherwise values z + (j + 1/2) s0, exact ties of (x - z) / s, a third
    of them moved one bf16 step up or down."""
    lead = shape[:-1] + (1,)
    s0 = 2.0 ** rng.integers(-8, 8, lead)
    z = -s0 * rng.integers(0, 4, lead)
    x = z + s0 * (rng.integers(0, 3, shape) + 0.5)
    x[..., 0:1], x[..., 1:2] = z, z + 3 * s0
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(bits), x.astype(np.float32))
    step = rng.integers(-1, 2, shape).astype(np.int32)
    step[..., :2] = 0
    return (bits.astype(np.int32) + step).astype(np.uint16)


def test_quantiser_bit_exact_on_ties():
    import torch
    import long_context_tiled_amd as lib
    rng = np.random.default_rng(12)
    B, Hkv, L, d = 2, 2, 192, 128
    k = _on_ties(rng, (B, Hkv, L, d))
    vt = _on_ties(rng, (B, Hkv, L // 64, d, 64))
    v = np.ascontiguousarray(vt.transpose(0, 1, 2, 4, 3).reshape(B, Hkv, L, d))
    print("[q2] quantise on ties", flush=True)
    got = _host(lib.quantize_q2(_dev(k), _dev(v)))
    torch.cuda.synchronize()
    _assert_same_cache(got, _encode(k, v), "ties")


def _decode_case(q, k, v, taus, name):
    import torch
    import long_context_tiled_amd as lib
    Hkv, L = k.shape[1], k.shape[2]
    print(f"[q2] {name}: quantise", flush=True)
    cache = lib.quantize_q2(_dev(k), _dev(v))
    enc = _encode(k, v)
    _assert_same_cache(_host(cache), enc, name)
    dq = _dev(q)
    for tau in taus:
        print(f"[q2] {name} tau={tau}", flush=True)
        o, lse, mask = lib.decode_q2(dq, cache, L, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), kv_for=_oracle_kv(enc, L), Hkv=Hkv)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


SMALL = [
    ("gqa4_ragged_3splits", _cfg(id=80), (INF, 8.0, 4.0, 1.0)),
    ("g1_d64_one_split", _cfg(B=1, Hq=2, Hkv=2, L=4096, d=64, id=81), (INF, 2.0)),
    ("g8_split_edge", _cfg(B=1, Hq=8, Hkv=1, L=4097, id=82), (INF, 4.0)),
    ("g16", _cfg(B=1, Hq=16, Hkv=1, L=9000, id=83), (INF, 3.0)),
    ("g3_d64", _cfg(B=3, Hq=6, Hkv=2, L=12345, d=64, id=84), (INF, 0.0, 2.0)),
    # two KV groups per wave: an odd last group without a partner, and G = 8
    # at d = 64 over two splits
    ("g5_hkv3_odd_pair", _cfg(B=2, Hq=15, Hkv=3, L=5000, id=85), (INF, 3.0)),
    ("g8_hkv4_d64", _cfg(B=1, Hq=32, Hkv=4, L=8192, d=64, id=86), (INF, 4.0)),
]


@pytest.mark.parametrize("name,cfg,taus", SMALL, ids=[s[0] for s in SMALL])
def test_decode_q2_small(name, cfg, taus):
    q, k, v = synth.make_decode(cfg)
    _decode_case(q, k, v, taus, name)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 4095, 4096, 4160, 8193])
def test_decode_q2_edge_lengths(L):
    q, k, v = synth.make_decode(_cfg(B=1, Hq=4, Hkv=1, L=L, id=90))
    _decode_case(q, k, v, (INF, 0.0, 3.0), f"edge L={L}")


def test_decode_q2_workload_sampled():
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("decode_128k")
    print("[q2] generating decode_128k", flush=True)
    q, k, v = synth.make_decode(cfg)
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    print("[q2] decode_128k: quantise", flush=True)
    cache = lib.quantize_q2(_dev(k), _dev(v))
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    heads = sorted({(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(8)}
                   | {(0, 0), (B - 1, Hq - 1)})
    groups = sorted({(b, h // G) for b, h in heads})
    enc = {}
    for b, g in groups:   # the cache of every sampled KV head, bit for bit
        e = _encode(k[b, g], v[b, g])
        got = {n: cache[n][b, g].cpu().numpy() for n in cache}
        got["kp"], got["vp"] = got["kp"].view(np.uint32), got["vp"].view(np.uint32)
        _assert_same_cache(got, e, f"b={b} g={g}")
        enc[(b, g)] = e

    def kv_for(b, g):
        e = enc[(b, g)]
        return kvq2.decode_k(e["kq"], e["kp"]), kvq2.decode_v(e["vq"], e["vp"], L)

    dq = _dev(q)
    prev = None
    for tau in cfg["taus"]:
        print(f"[q2] decode_128k tau={tau}", flush=True)
        o, lse, mask = lib.decode_q2(dq, cache, L, tau, want_mask=True)
        torch.cuda.synchronize()
        mask_np = mask.cpu().numpy()
        assert (mask_np[:, :, ::64] == 0).all()
        if prev is not None:
            assert ((prev == 1) <= (mask_np == 1)).all()
        prev = mask_np
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask_np, heads=heads, kv_for=kv_for, Hkv=Hkv)
        print(f"  skip_fraction={(mask_np == 1).mean():.4f} {rep}", flush=True)
        assert rep.ok(), str(rep)
        del o, lse, mask


def test_quantiser_key_ranges_compose():
    import torch
    import long_context_tiled_amd as lib
    k, v = _rand_kv(2, 2, 1000, 128, 22)
    dk, dv = _dev(k), _dev(v)
    whole = _host(lib.quantize_q2(dk, dv))
    for ranges in (((0, 512), (512, 1000)), ((0, 700), (640, 1000)), ((0, 64), (64, 65), (64, 1000))):
        print(f"[q2] ranges {ranges}", flush=True)
        cache = lib.empty_q2(2, 2, 1000, 128, dk.device)
        for i, (k0, k1) in enumerate(ranges):
            lib.attn_kv_quantize_q2(dk, dv, cache, key_range=(k0, k1))
            if i == 0:
                torch.cuda.synchronize()
                part = _host(cache)
                want = _encode(k[:, :, :k1], v[:, :, :k1])
                T1 = (k1 + 63) // 64
                got = dict(kq=part["kq"][:, :, :k1], kp=part["kp"][:, :, :k1],
                           vq=part["vq"][:, :, :T1], vp=part["vp"][:, :, :T1])
                _assert_same_cache(got, want, f"prefix {k1}")
        torch.cuda.synchronize()
        _assert_same_cache(_host(cache), whole, str(ranges))
