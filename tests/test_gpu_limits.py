"""GPU parity at the largest head the library accepts: one K/V head of
2^31 - 2^16 bytes (L = 8,388,352 keys at d = 128), where every 32-bit
buffer offset of the kernels is near its limit. The bf16 decode, the 4-bit
decode and a 64-query causal prefill chunk at the end of the keys are
checked against the fp64 oracle. Host memory: about 25 GB."""
import math

import numpy as np
import pytest

import synth
from oracle import kvq4
from tests import _parity

pytestmark = pytest.mark.gpu
INF = math.inf
D = 128
L_MAX = ((1 << 31) - (1 << 16)) // (2 * D)


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.fixture(scope="module")
def kv():
    rng = np.random.default_rng(2026)
    print(f"[limits] generating K, V with L={L_MAX}", flush=True)
    k = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, L_MAX, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, L_MAX, D), dtype=np.float32))
    # a few strong keys spread over the length (sinks deep inside the cache)
    for pos in (5, L_MAX // 2, L_MAX - 7):
        k[0, 0, pos] = synth.f32_to_bf16_bits(np.full(D, 0.9, np.float32))
    return k, v


def _q(rng, shape):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) + 0.8).astype(np.float32))


def test_decode_at_max_head(kv):
    import torch
    import long_context_tiled_amd as lib
    k, v = kv
    q = _q(np.random.default_rng(1), (1, 2, D))
    dk, dv = _dev(k), _dev(v)
    for tau in (INF, 4.0):
        print(f"[limits] decode L={L_MAX} tau={tau}", flush=True)
        o, lse, mask = lib.decode(_dev(q), dk, dv, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, k, v, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy())
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_decode_q4_at_max_head(kv):
    import torch
    import long_context_tiled_amd as lib
    k, v = kv
    q = _q(np.random.default_rng(2), (1, 2, D))
    print(f"[limits] quantise L={L_MAX}", flush=True)
    cache = lib.quantize_q4(_dev(k), _dev(v))
    torch.cuda.synchronize()
    enc = kvq4.encode(synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v))
    for n in ("kq", "kp", "vq", "vp"):
        got = cache[n].cpu().numpy().view(enc[n].dtype)
        assert np.array_equal(got, enc[n]), n

    def kv_for(b, g):
        return kvq4.decode_k(enc["kq"][b, g], enc["kp"][b, g]), kvq4.decode_v(
            enc["vq"][b, g], enc["vp"][b, g], L_MAX)

    for tau in (INF, 4.0):
        print(f"[limits] decode_q4 L={L_MAX} tau={tau}", flush=True)
        o, lse, mask = lib.decode_q4(_dev(q), cache, L_MAX, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_decode(q, None, None, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask.cpu().numpy(), kv_for=kv_for, Hkv=1)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_prefill_chunk_at_max_head(kv):
    import torch
    import long_context_tiled_amd as lib
    k, v = kv
    q = _q(np.random.default_rng(3), (1, 1, 64, D))
    q0 = L_MAX - 64
    for tau in (INF, 4.0):
        print(f"[limits] prefill chunk of 64 at the end of N={L_MAX} tau={tau}", flush=True)
        o, lse, mask = lib.prefill_chunk(_dev(q), _dev(k), _dev(v), True, tau, want_mask=True)
        torch.cuda.synchronize()
        rep = _parity.check_prefill(q, k, v, True, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                    mask.cpu().numpy(), [(0, 0, 0)], q0=q0)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
