"""GPU parity of the prefill with the P.V product on 8-bit operands
(attn_prefill_pv8), QK^T in bf16 or on fp8 codes: the V quantiser's code
blocks and scales bit for bit against the oracle (oracle/fp8pv.py), and the
outputs and skip masks against the 8-bit P.V oracle on the oracle's codes,
with the tolerances of the bf16 prefill beyond a per-row slack: the
kernel's scores may sit off the oracle's by the accumulation error of its
QK^T product (bound below), which moves O and LSE to first order and lets
probabilities close to an E4M3 rounding point round either way; the
oracle bounds both per row (oracle/fp8pv.py, tests/_parity.py)."""
import math

import numpy as np
import pytest

import synth
from oracle import fp8, fp8pv
from tests import _parity

pytestmark = pytest.mark.gpu
INF = math.inf
# kernel score error bounds, relative to sum |q_i k_i| / sqrt(d): fp32
# accumulation of up to 128 bf16 products (2^-17); the fp8 MFMA's inexact
# sums (measured up to 2^-12.2 of that sum; 2^-11 taken). Both set which
# probabilities may round either way (the oracle's slack adds what that
# moves O); only the fp8 one also widens O and LSE to first order (bf16
# scores are as exact as the bf16 prefill's own tolerances assume, so with
# bf16 QK^T the P.V product is held to them beyond its roundings).
ERR_BF16, ERR_FP8 = 2.0 ** -17, 2.0 ** -11


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _np(t):
    return t.cpu().numpy()


def _run(q, k, v, causal, tau, qk8):
    import torch
    import long_context_tiled_amd as lib
    o, lse, mask, ws = lib.prefill_pv8(_dev(q), _dev(k), _dev(v), causal, tau, qk8=qk8,
                                       want_mask=True)
    torch.cuda.synchronize()
    B, Hq, N, d = q.shape
    parts = lib.pv8_workspace_parts(ws, B, Hq, k.shape[1], N, d, qk8)
    return _np(o), _np(lse), _np(mask), {n: _np(t) for n, t in parts.items()}


def _check_vcodes(parts, v):
    B, Hkv = v.shape[:2]
    for b in range(B):
        for g in range(Hkv):
            codes, s = fp8pv.quantize_v(synth.bf16_bits_to_f32(v[b, g]))
            want = fp8pv.v_layout(codes)
            got = parts["vc"][b, g]
            bad = np.argwhere(got != want)
            assert bad.size == 0, f"V codes of b={b} g={g}: {len(bad)} differ, first {bad[:3].tolist()}"
            assert parts["vs"][b, g].view(np.uint32) == np.float32(s).view(np.uint32), (b, g)


def _qk(q, k, qk8):
    if not qk8:
        return None, None
    qc, qs = fp8.quantize(synth.bf16_bits_to_f32(q))
    kc, ks = fp8.quantize(synth.bf16_bits_to_f32(k))
    return fp8.dequantize(qc, qs), fp8.dequantize(kc, ks)


CASES = [  # (name, cfg)
    ("tiny_full", dict(kind="prefill", id=150, B=1, Hq=2, Hkv=2, N=256, d=64, causal=False,
                       sinks=False, band=False)),
    ("gqa4_ragged_causal", dict(kind="prefill", id=151, B=1, Hq=8, Hkv=2, N=1000, d=128,
                                causal=True, sinks=True, band=True)),
    ("b2_g1_d64_causal", dict(kind="prefill", id=152, B=2, Hq=2, Hkv=2, N=700, d=64, causal=True,
                              sinks=True, band=False)),
    ("g8_full_ragged", dict(kind="prefill", id=153, B=1, Hq=8, Hkv=1, N=333, d=128,
                            causal=False, sinks=True, band=True)),
    ("g3_one_tile", dict(kind="prefill", id=154, B=1, Hq=3, Hkv=1, N=64, d=128, causal=True,
                         sinks=True, band=False)),
    ("g2_short_d64", dict(kind="prefill", id=155, B=1, Hq=4, Hkv=2, N=65, d=64, causal=True,
                          sinks=True, band=False)),
]


@pytest.mark.parametrize("qk8", [False, True], ids=["qk_bf16", "qk_fp8"])
@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_pv8_prefill_against_oracle(name, cfg, qk8):
    q, k, v = synth.make_prefill(cfg)
    causal = cfg["causal"]
    qf, kf = _qk(q, k, qk8)
    blocks = 0
    for tau in (INF, 4.0, 1.0):
        print(f"[pv8] {name} qk8={qk8} tau={tau}", flush=True)
        o, lse, mask, parts = _run(q, k, v, causal, tau, qk8)
        _check_vcodes(parts, v)
        rep = _parity.check_prefill(q, k, v, causal, tau, o, lse, mask, qf=qf, kf=kf, pv8=True,
                                    score_err_rel=ERR_FP8 if qk8 else ERR_BF16, lin_err=qk8)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
        blocks += q.shape[0] * q.shape[1] * ((q.shape[2] + 63) // 64)
        assert rep.ambiguous <= max(1, blocks // 20), str(rep)


def test_pv8_zero_head_and_extreme_v():
    # one KV head of zeros (scale 1, every code 0), one whose largest |v| is
    # an exact 448 multiple (codes on the grid), and large-magnitude values
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 128
    rng = np.random.default_rng(5)
    q = synth.f32_to_bf16_bits(rng.normal(size=(B, Hq, N, d)).astype(np.float32))
    k = synth.f32_to_bf16_bits(rng.normal(size=(B, Hkv, N, d)).astype(np.float32))
    vf = rng.normal(size=(B, Hkv, N, d)).astype(np.float32) * 300.0
    vf[0, 0] = 0.0
    vf[0, 1, 17, 5] = 448.0 * 4
    v = synth.f32_to_bf16_bits(vf)
    o, lse, mask, parts = _run(q, k, v, True, INF, False)
    _check_vcodes(parts, v)
    assert float(parts["vs"][0, 0]) == 1.0 and not parts["vc"][0, 0].any()
    assert np.all(o[0, :2] == 0.0)
    # |v| up to ~1800: O's absolute tolerance (1e-2) is then a 1e-5 relative
    # one, so the bf16 scores' fp32 error counts to first order here
    rep = _parity.check_prefill(q, k, v, True, INF, o, lse, mask, pv8=True,
                                score_err_rel=ERR_BF16, lin_err=True)
    print(f"  {rep}", flush=True)
    assert rep.ok(), str(rep)


@pytest.mark.parametrize("qk8", [False, True], ids=["qk_bf16", "qk_fp8"])
@pytest.mark.parametrize("name,count", [("prefill_8k", 48), ("prefill_128k", 8)])
def test_pv8_workload_sampled(name, count, qk8):
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload(name)
    print(f"[pv8] generating {name}", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nt = (N + 63) // 64
    blocks = _parity.sample_blocks(B, Hq, nt, True, count, seed=len(name) + 7)
    ws = torch.empty(lib.attn_prefill_pv8_workspace_bytes(B, Hq, Hkv, N, d, qk8),
                     dtype=torch.uint8, device="cuda")
    qf = kf = None
    checked = False
    for tau in cfg["taus"]:
        print(f"[pv8] {name} qk8={qk8} tau={tau}", flush=True)
        o, lse, mask, _ = lib.prefill_pv8(dq, dk, dv, True, tau, qk8=qk8, want_mask=True,
                                          workspace=ws)
        torch.cuda.synchronize()
        if not checked:
            parts = {n: _np(t) for n, t in
                     lib.pv8_workspace_parts(ws, B, Hq, Hkv, N, d, qk8).items()}
            _check_vcodes(parts, v)
            if qk8:
                qf = fp8.dequantize(parts["qc"], parts["qs"])
                kf = fp8.dequantize(parts["kc"], parts["ks"])
                for g in range(Hkv):
                    wc, wsc = fp8.quantize(synth.bf16_bits_to_f32(k[0, g]))
                    assert np.array_equal(parts["kc"][0, g], wc)
            checked = True
        mask_np = _np(mask)
        tri = np.triu(np.ones((nt, nt), bool), 1)
        assert (mask_np[..., tri] == 2).all() and not (mask_np[..., ~tri] == 2).any()
        rows = sorted({(b, h) for b, h, _ in blocks})
        o_rows = {bh: _np(o[bh[0], bh[1]]) for bh in rows}
        lse_np = _np(lse)
        chk = _parity.PrefillChecker(q, k, v, True, qf=qf, kf=kf, pv8=True,
                                     score_err_rel=ERR_FP8 if qk8 else ERR_BF16, lin_err=qk8)
        rep = _parity.Report()
        for b, h, qb in sorted(blocks, key=lambda x: (x[0], x[1] // (Hq // Hkv), x[1])):
            r0, r1 = qb * 64, min(N, qb * 64 + 64)
            rep.merge(chk.check_block(b, h, qb, tau, o_rows[(b, h)][r0:r1], lse_np[b, h, r0:r1],
                                      mask_np[b, h, qb]))
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
        assert rep.ambiguous <= max(1, count // 10), str(rep)
        del o, lse, mask
