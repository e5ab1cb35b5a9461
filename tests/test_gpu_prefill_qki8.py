"""GPU parity of the prefill with block-quantised symmetric int8 QK^T
(attn_prefill_qki8): the quantiser's codes and tile scales bit for bit
against the oracle's encoder (oracle/int8.py), and the outputs and skip
masks against the fp64 prefill oracle run on the oracle's dequantised Q and
K (V as given), with the tolerances of the bf16 prefill: the int8 products
are exact in int32, so the kernel's scores differ from the oracle's only by
the fp32 rounding of the scales."""
import math

import numpy as np
import pytest

import synth
from oracle import int8
from tests import _parity

pytestmark = pytest.mark.gpu
INF = math.inf


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _np(t):
    return t.cpu().numpy()


def _parts(ws, B, Hq, Hkv, N, d):
    import long_context_tiled_amd as lib
    parts = {n: _np(t) for n, t in lib.qk8_workspace_parts(ws, B, Hq, Hkv, N, d).items()}
    parts["qc"] = parts["qc"].view(np.int8)
    parts["kc"] = parts["kc"].view(np.int8)
    return parts


def _run(q, k, v, causal, tau):
    import torch
    import long_context_tiled_amd as lib
    o, lse, mask, ws = lib.prefill_qk8(_dev(q), _dev(k), _dev(v), causal, tau, want_mask=True,
                                       int8=True)
    torch.cuda.synchronize()
    B, Hq, N, d = q.shape
    return _np(o), _np(lse), _np(mask), _parts(ws, B, Hq, k.shape[1], N, d)


def _encode(q, k):
    qc, qs = int8.quantize(synth.bf16_bits_to_f32(q))
    kc, ks = int8.quantize(synth.bf16_bits_to_f32(k))
    return qc, qs, kc, ks


def _check_codes(parts, qc, qs, kc, ks):
    for name, want in (("qc", qc), ("kc", kc)):
        got = parts[name]
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name}: {len(bad)} codes differ, first {bad[:3].tolist()}"
    for name, want in (("qs", qs), ("ks", ks)):
        assert np.array_equal(parts[name].view(np.uint32), want.view(np.uint32)), name


CASES = [  # (name, cfg)
    ("tiny_full", dict(kind="prefill", id=160, B=1, Hq=2, Hkv=2, N=256, d=64, causal=False,
                       sinks=False, band=False)),
    ("gqa4_ragged_causal", dict(kind="prefill", id=161, B=1, Hq=8, Hkv=2, N=1000, d=128,
                                causal=True, sinks=True, band=True)),
    ("b2_g1_d64_causal", dict(kind="prefill", id=162, B=2, Hq=2, Hkv=2, N=700, d=64, causal=True,
                              sinks=True, band=False)),
    ("g8_full_ragged", dict(kind="prefill", id=163, B=1, Hq=8, Hkv=1, N=333, d=128,
                            causal=False, sinks=True, band=True)),
    ("g3_one_tile", dict(kind="prefill", id=164, B=1, Hq=3, Hkv=1, N=64, d=128, causal=True,
                         sinks=True, band=False)),
    ("g2_short", dict(kind="prefill", id=165, B=1, Hq=4, Hkv=2, N=65, d=128, causal=True,
                      sinks=True, band=False)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_qki8_prefill_against_oracle(name, cfg):
    q, k, v = synth.make_prefill(cfg)
    causal = cfg["causal"]
    qc, qs, kc, ks = _encode(q, k)
    qf, kf = int8.dequantize(qc, qs), int8.dequantize(kc, ks)
    for tau in (INF, 4.0, 1.0):
        print(f"[qki8] {name} tau={tau}", flush=True)
        o, lse, mask, parts = _run(q, k, v, causal, tau)
        _check_codes(parts, qc, qs, kc, ks)
        rep = _parity.check_prefill(q, k, v, causal, tau, o, lse, mask, qf=qf, kf=kf)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_qki8_quantiser_ties_and_zero_tiles():
    # tiles whose largest |x| is 127 (scale 1): values halfway between codes
    # (ties to even), negatives, and a tile of zeros (scale 1, codes 0);
    # bit-exact against the oracle's encoder
    B, H, N, d = 1, 2, 192, 64
    rng = np.random.default_rng(11)
    vals = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 0.0, 7.0, 0.25, -3.75],
                    np.float32)
    x = rng.choice(vals, (B, H, N, d)).astype(np.float32)
    x[..., 0:64:7, 0] = 127.0
    x[..., 64:128, :] = 0.0                                   # a zero tile
    x[..., 128:192:5, 3] = -127.0
    bits = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(bits), x)
    v = synth.f32_to_bf16_bits(rng.normal(size=(B, H, N, d)).astype(np.float32))
    o, lse, mask, parts = _run(bits, bits, v, True, INF)
    qc, qs, kc, ks = _encode(bits, bits)
    assert float(qs[0, 0, 0]) == 1.0 and float(qs[0, 0, 1]) == 1.0 and not qc[0, 0, 64:128].any()
    assert qc[0, 0, 0, 0] == 127 and np.isin(qc[0, 0, :64][x[0, 0, :64] == 2.5], [2]).all()
    _check_codes(parts, qc, qs, kc, ks)


@pytest.mark.parametrize("name,count", [("prefill_8k", 64), ("prefill_128k", 12)])
def test_qki8_workload_sampled(name, count):
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload(name)
    print(f"[qki8] generating {name}", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nt = (N + 63) // 64
    blocks = _parity.sample_blocks(B, Hq, nt, True, count, seed=len(name) + 3)
    ws = torch.empty(lib.attn_prefill_qk8_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8,
                     device="cuda")
    qf = kf = None
    for tau in cfg["taus"]:
        print(f"[qki8] {name} tau={tau}", flush=True)
        o, lse, mask, _ = lib.prefill_qk8(dq, dk, dv, True, tau, want_mask=True, workspace=ws,
                                          int8=True)
        torch.cuda.synchronize()
        if qf is None:
            parts = _parts(ws, B, Hq, Hkv, N, d)
            qc, qs, kc, ks = parts["qc"], parts["qs"], parts["kc"], parts["ks"]
            # codes and scales of the sampled heads' tiles against the encoder
            for b, h in sorted({(b, h) for b, h, _ in blocks}):
                wc, wsc = int8.quantize(synth.bf16_bits_to_f32(q[b, h]))
                assert np.array_equal(qc[b, h], wc) and np.array_equal(qs[b, h], wsc)
            for g in range(Hkv):
                wc, wsc = int8.quantize(synth.bf16_bits_to_f32(k[0, g]))
                assert np.array_equal(kc[0, g], wc) and np.array_equal(ks[0, g], wsc)
            qf = int8.dequantize(qc, qs)
            kf = int8.dequantize(kc, ks)
        mask_np = _np(mask)
        tri = np.triu(np.ones((nt, nt), bool), 1)
        assert (mask_np[..., tri] == 2).all() and not (mask_np[..., ~tri] == 2).any()
        rows = sorted({(b, h) for b, h, _ in blocks})
        o_rows = {bh: _np(o[bh[0], bh[1]]) for bh in rows}
        lse_np = _np(lse)
        chk = _parity.PrefillChecker(q, k, v, True, qf=qf, kf=kf)
        rep = _parity.Report()
        for b, h, qb in sorted(blocks, key=lambda x: (x[0], x[1] // (Hq // Hkv), x[1])):
            r0, r1 = qb * 64, min(N, qb * 64 + 64)
            rep.merge(chk.check_block(b, h, qb, tau, o_rows[(b, h)][r0:r1], lse_np[b, h, r0:r1],
                                      mask_np[b, h, qb]))
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
        del o, lse, mask
