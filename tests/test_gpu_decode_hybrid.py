"""GPU parity of the hybrid 2/4-bit KV cache (one width per KV head): the
quantiser against the oracle's encoder bit for bit, and attn_decode_hybrid
against the fp64 decode oracle run on the oracle's dequantised cache (each
head at its own width; same tolerances as the single-width decodes)."""
import math

import numpy as np
import pytest

import synth
from oracle import kvq_hybrid
from tests import _parity
from tests.test_gpu_decode_q4 import _assert_same_cache, _cfg, _dev, _host, _rand_kv

pytestmark = pytest.mark.gpu
INF = math.inf


def _encode(k, v, bits):
    return kvq_hybrid.encode(synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v), bits)


def _assert_same_hybrid(cache, enc, where=""):
    for w, key in ((4, "q4"), (2, "q2")):
        if enc[w] is None:
            assert cache[key] is None, (where, key)
        else:
            _assert_same_cache(_host(cache[key]), enc[w], f"{where} {key}")


def _kv_for(enc, bits, L):
    K, V = kvq_hybrid.decode_kv(enc, bits, L)
    return lambda b, g: (K[b, g], V[b, g])


QCASES = [  # (B, L, d, bits, seed)
    (1, 65, 64, (4, 2), 1), (2, 300, 128, (2, 4, 2), 2), (1, 4097, 128, (2, 2, 4, 4, 2), 3),
    (2, 1000, 64, (4,), 4), (1, 129, 128, (2,), 5),
]


@pytest.mark.parametrize("B,L,d,bits,seed", QCASES)
def test_hybrid_quantiser_bit_exact(B, L, d, bits, seed):
    import torch
    import long_context_tiled_amd as lib
    k, v = _rand_kv(B, len(bits), L, d, seed)
    print(f"[hy] quantise B={B} L={L} d={d} bits={bits}", flush=True)
    cache = lib.quantize_hybrid(_dev(k), _dev(v), bits)
    torch.cuda.synchronize()
    _assert_same_hybrid(cache, _encode(k, v, bits))


def test_hybrid_quantiser_key_ranges_compose():
    import torch
    import long_context_tiled_amd as lib
    bits = (2, 4, 4, 2)
    k, v = _rand_kv(2, 4, 1000, 128, 9)
    dk, dv = _dev(k), _dev(v)
    want = _encode(k, v, bits)
    for ranges in (((0, 512), (512, 1000)), ((0, 64), (64, 65), (64, 1000))):
        print(f"[hy] ranges {ranges}", flush=True)
        cache = lib.empty_hybrid(bits, 2, 1000, 128, dk.device)
        for k0, k1 in ranges:
            lib.attn_kv_quantize_hybrid(dk, dv, cache, key_range=(k0, k1))
        torch.cuda.synchronize()
        _assert_same_hybrid(cache, want, str(ranges))


def _decode_case(q, k, v, bits, taus, name, sas=0):
    import torch
    import long_context_tiled_amd as lib
    Hkv, L = k.shape[1], k.shape[2]
    print(f"[hy] {name}: quantise bits={bits}", flush=True)
    cache = lib.quantize_hybrid(_dev(k), _dev(v), bits)
    enc = _encode(k, v, bits)
    _assert_same_hybrid(cache, enc, name)
    kv_for = _kv_for(enc, bits, L)
    dq = _dev(q)
    for tau in taus:
        print(f"[hy] {name} tau={tau} sas={sas}", flush=True)
        o, lse, mask = lib.decode_hybrid(dq, cache, L, tau, want_mask=True, sas=sas)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), kv_for=kv_for, Hkv=Hkv, sas=sas)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


SMALL = [
    # G = 4 (2-bit heads in pairs, one odd last pair), three splits, ragged
    ("g4_mixed_ragged", _cfg(B=2, Hq=20, Hkv=5, L=9000, id=120), (2, 4, 2, 2, 4), (INF, 8.0, 3.0)),
    # G = 8 with the widths alternating, as in decode_128k's head count
    ("g8_alternating", _cfg(B=2, Hq=64, Hkv=8, L=5000, id=121), (4, 2) * 4, (INF, 4.0)),
    # G = 16: the 2-bit heads take the one-group kernel
    ("g16_d64", _cfg(B=1, Hq=48, Hkv=3, L=4097, d=64, id=122), (4, 2, 2), (INF, 2.0)),
    # a single head of each width, and every head at one width
    ("one_each", _cfg(B=3, Hq=4, Hkv=2, L=700, id=123), (2, 4), (INF, 0.0, 3.0)),
    ("all_2", _cfg(B=1, Hq=8, Hkv=2, L=4160, id=124), (2, 2), (INF, 4.0)),
    ("all_4", _cfg(B=1, Hq=8, Hkv=2, L=4160, id=125), (4, 4), (INF, 4.0)),
]


@pytest.mark.parametrize("name,cfg,bits,taus", SMALL, ids=[s[0] for s in SMALL])
def test_decode_hybrid_small(name, cfg, bits, taus):
    q, k, v = synth.make_decode(cfg)
    _decode_case(q, k, v, bits, taus, name)


@pytest.mark.parametrize("degree", [2, 3])
def test_decode_hybrid_sas(degree):
    q, k, v = synth.make_decode(_cfg(B=2, Hq=24, Hkv=3, L=6000, id=126))
    _decode_case(q, k, v, (4, 2, 2), (INF, 4.0), f"sas{degree}", sas=degree)


def test_decode_hybrid_capacity_beyond_length():
    """Arrays sized for more keys than attended, poisoned past the written
    keys: the decode of the first L keys reads none of them."""
    import torch
    import long_context_tiled_amd as lib
    cap, L, bits = 8192, 5000, (2, 4, 4, 2)
    q, k, v = synth.make_decode(_cfg(B=2, Hq=16, Hkv=4, L=cap, id=127))
    cache = lib.empty_hybrid(bits, 2, cap, 128, "cuda")
    for key in ("q4", "q2"):
        for t in cache[key].values():
            t.fill_(255 if t.dtype == torch.uint8 else -1)
    dk, dv = _dev(k), _dev(v)
    print("[hy] capacity: quantise the first L keys", flush=True)
    lib.attn_kv_quantize_hybrid(dk, dv, cache, key_range=(0, L))
    enc = _encode(k[:, :, :L], v[:, :, :L], bits)
    kv_for = _kv_for(enc, bits, L)
    for tau in (INF, 4.0):
        print(f"[hy] capacity tau={tau}", flush=True)
        o, lse, mask = lib.decode_hybrid(_dev(q), cache, L, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), kv_for=kv_for, Hkv=4)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_decode_hybrid_workload_sampled():
    """decode_128k with its eight KV heads alternating 4 and 2 bits: every
    sampled head's codes bit for bit, and decode parity on sampled heads."""
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("decode_128k")
    print("[hy] generating decode_128k", flush=True)
    q, k, v = synth.make_decode(cfg)
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    bits = (4, 2) * (Hkv // 2)
    print("[hy] decode_128k: quantise", flush=True)
    cache = lib.quantize_hybrid(_dev(k), _dev(v), bits)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    heads = sorted({(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(8)}
                   | {(0, 0), (0, G), (B - 1, Hq - 1)})
    groups = sorted({(b, h // G) for b, h in heads})
    kv = {}
    for b, g in groups:   # every sampled KV head's codes, bit for bit
        w = bits[g]
        i = kvq_hybrid.heads_of(bits, w).index(g)
        one = _encode(k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], (w,))
        sub = cache["q4" if w == 4 else "q2"]
        got = {n: t[b:b + 1, i:i + 1] for n, t in sub.items()}
        _assert_same_cache(_host(got), one[w], f"b={b} g={g}")
        K, V = kvq_hybrid.decode_kv(one, (w,), L)
        kv[(b, g)] = (K[0, 0], V[0, 0])
    dq = _dev(q)
    for tau in cfg["taus"]:
        print(f"[hy] decode_128k tau={tau}", flush=True)
        o, lse, mask = lib.decode_hybrid(dq, cache, L, tau, want_mask=True)
        torch.cuda.synchronize()
        mask_np = mask.cpu().numpy()
        assert (mask_np[:, :, ::64] == 0).all()
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask_np, heads=heads, kv_for=lambda b, g: kv[(b, g)], Hkv=Hkv)
        print(f"  skip_fraction={(mask_np == 1).mean():.4f} {rep}", flush=True)
        assert rep.ok(), str(rep)
        del o, lse, mask
