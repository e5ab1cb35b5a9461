"""Skip masks at full size against the fp64 oracle's decisions, beyond the
sampled blocks of the workload tests:

* decode_128k: every query head at every tau - mask, O and LSE;
* prefill_8k: every query block of every head at every tau - mask, O and
  LSE;
* prefill_32k and prefill_128k: every query block of one whole head at
  every tau - the mask (the oracle's decisions alone: scores and tile
  maxima once per block, the rule per tau).

Masks must agree bit for bit except on tiles whose oracle margin is within
1e-3 logits of the threshold; those are counted and printed (and, where O
and LSE are compared, the oracle re-evaluates the block under the GPU's
decision). The oracle work is spread over host threads.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from tests import _parity

pytestmark = pytest.mark.gpu


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def test_decode_128k_every_head():
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("decode_128k")
    print("[full] generating decode_128k", flush=True)
    q, k, v = synth.make_decode(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = {}
    for tau in cfg["taus"]:
        o, lse, mask = lib.decode(dq, dk, dv, tau, want_mask=True)
        torch.cuda.synchronize()
        out[tau] = (o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy())
    del dq, dk, dv
    torch.cuda.empty_cache()

    def group(bg):
        b, g = bg
        kv = (synth.bf16_bits_to_f64(k[b, g]), synth.bf16_bits_to_f64(v[b, g]))
        heads = [(b, h) for h in range(g * G, (g + 1) * G)]
        reps = {}
        for tau, (o, lse, mask) in out.items():
            reps[tau] = _parity.check_decode(q, None, None, tau, o, lse, mask, heads=heads,
                                             kv_for=lambda *_: kv, Hkv=Hkv)
        return reps

    total = {tau: _parity.Report() for tau in out}
    with _one_blas_thread(), ThreadPoolExecutor(_threads()) as ex:
        for i, reps in enumerate(ex.map(group, [(b, g) for b in range(B) for g in range(Hkv)])):
            for tau, r in reps.items():
                total[tau].merge(r)
            if i % 32 == 31:
                print(f"[full] decode_128k {i + 1} of {B * Hkv} KV heads checked", flush=True)
    for tau, rep in total.items():
        print(f"[full] decode_128k tau={tau} heads={B * Hq} {rep}", flush=True)
        assert rep.tiles == B * Hq * (k.shape[2] // 64)
        assert rep.ok(), str(rep)


def test_prefill_8k_every_block():
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("prefill_8k")
    print("[full] generating prefill_8k", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    nt = (N + 63) // 64
    out = {}
    for tau in cfg["taus"]:
        o, lse, mask = lib.prefill(dq, dk, dv, True, tau, want_mask=True)
        torch.cuda.synchronize()
        out[tau] = (o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy())
        del o, lse, mask
    del dq, dk, dv
    torch.cuda.empty_cache()

    def head(bh):
        b, h = bh
        chk = _parity.PrefillChecker(q, k, v, True)
        reps = {}
        for tau, (o, lse, mask) in out.items():
            rep = _parity.Report()
            for qb0 in range(0, nt, 16):
                qb1 = min(nt, qb0 + 16)
                r0, r1 = qb0 * 64, min(N, qb1 * 64)
                rep.merge(chk.check_blocks(b, h, qb0, qb1, tau, o[b, h, r0:r1],
                                           lse[b, h, r0:r1], mask[b, h, qb0:qb1]))
            reps[tau] = rep
        return reps

    total = {tau: _parity.Report() for tau in out}
    with _one_blas_thread(), ThreadPoolExecutor(_threads()) as ex:
        for i, reps in enumerate(ex.map(head, [(b, h) for b in range(B) for h in range(Hq)])):
            for tau, r in reps.items():
                total[tau].merge(r)
            if i % 8 == 7:
                print(f"[full] prefill_8k {i + 1} of {B * Hq} heads checked", flush=True)
    for tau, rep in total.items():
        print(f"[full] prefill_8k tau={tau} blocks={B * Hq * nt} {rep}", flush=True)
        assert rep.tiles == B * Hq * nt * (nt + 1) // 2
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("name,h", [("prefill_32k", 37), ("prefill_128k", 5)])
def test_prefill_one_whole_head_masks(name, h):
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload(name)
    print(f"[full] generating {name}", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    nt = (N + 63) // 64
    taus = tuple(cfg["taus"])
    gpu = {}
    for tau in taus:
        _, _, mask = lib.prefill(dq, dk, dv, True, tau, want_mask=True)
        torch.cuda.synchronize()
        gpu[tau] = mask[0, h].cpu().numpy()
        del mask
    del dq, dk, dv
    torch.cuda.empty_cache()
    kf = synth.bf16_bits_to_f64(k[0, h // G])
    step = 16                                     # query blocks per oracle call

    def chunk(qb0):
        # causal: the rows of blocks qb0 .. qb1 - 1 see no key past qb1 * 64,
        # so the oracle runs on those keys (its decisions for the tiles it
        # visits are the same; the GPU must mark every later tile not visited)
        qb1 = min(nt, qb0 + step)
        rows = synth.bf16_bits_to_f64(q[0, h, qb0 * 64:min(N, qb1 * 64)])
        return qb0, oracle.prefill_decisions(rows, kf[:qb1 * 64], qb0, True, taus)

    stats = {tau: [0, 0, 0, 0] for tau in taus}  # tiles, skipped, ambiguous, hard
    bad = []
    with _one_blas_thread(), ThreadPoolExecutor(_threads()) as ex:
        for i, (qb0, res) in enumerate(ex.map(chunk, range(0, nt, step))):
            for tau, (dec, margin) in res.items():
                got = gpu[tau][qb0:qb0 + dec.shape[0]]
                assert (got[:, dec.shape[1]:] == oracle.NOT_VISITED).all(), qb0
                got = got[:, :dec.shape[1]]
                vis = dec != oracle.NOT_VISITED
                assert np.array_equal(got[~vis], dec[~vis]), f"not-visited marks at qb {qb0}"
                diff = (got != dec) & vis
                amb = diff & (np.abs(margin) < _parity.MARGIN_EPS)
                st = stats[tau]
                st[0] += int(vis.sum())
                st[1] += int((got[vis] == oracle.SKIPPED).sum())
                st[2] += int(amb.sum())
                st[3] += int((diff & ~amb).sum())
                if (diff & ~amb).any() and len(bad) < 4:
                    bad.append((tau, qb0, np.argwhere(diff & ~amb)[:3].tolist()))
            if i % 128 == 127:
                print(f"[full] {name} head {h}: {(i + 1) * step} of {nt} query blocks", flush=True)
    for tau, (tiles, skipped, amb, hard) in stats.items():
        print(f"[full] {name} head {h} tau={tau} tiles={tiles} skipped={skipped} "
              f"ambiguous={amb} hard_mismatch={hard}", flush=True)
        assert tiles == nt * (nt + 1) // 2
        assert hard == 0, bad


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_prefill_8k_qk8_every_block(fmt):
    # the 8-bit QK^T prefill (fp8 E4M3 or int8 codes) over every query block
    # of prefill_8k at every tau, against the oracle on the dequantised Q and K
    import torch
    import long_context_tiled_amd as lib
    from oracle import fp8, int8
    enc = int8 if fmt == "int8" else fp8
    cfg = synth.workload("prefill_8k")
    print(f"[full] generating prefill_8k (qk8 {fmt})", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nt = (N + 63) // 64
    ws = torch.empty(lib.attn_prefill_qk8_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8,
                     device="cuda")
    out = {}
    for tau in cfg["taus"]:
        o, lse, mask, _ = lib.prefill_qk8(dq, dk, dv, True, tau, want_mask=True, workspace=ws,
                                          int8=fmt == "int8")
        torch.cuda.synchronize()
        out[tau] = (o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy())
        del o, lse, mask
    parts = {n: t.cpu().numpy() for n, t in lib.qk8_workspace_parts(ws, B, Hq, Hkv, N, d).items()}
    del dq, dk, dv, ws
    torch.cuda.empty_cache()
    qc, qs = enc.quantize(synth.bf16_bits_to_f32(q))
    kc, ks = enc.quantize(synth.bf16_bits_to_f32(k))
    assert np.array_equal(parts["qc"].view(qc.dtype), qc)
    assert np.array_equal(parts["kc"].view(kc.dtype), kc)
    assert np.array_equal(parts["qs"], qs) and np.array_equal(parts["ks"], ks)
    qf, kf = enc.dequantize(qc, qs), enc.dequantize(kc, ks)

    def head(bh):
        b, h = bh
        chk = _parity.PrefillChecker(q, k, v, True, qf=qf, kf=kf)
        reps = {}
        for tau, (o, lse, mask) in out.items():
            rep = _parity.Report()
            for qb0 in range(0, nt, 16):
                qb1 = min(nt, qb0 + 16)
                r0, r1 = qb0 * 64, min(N, qb1 * 64)
                rep.merge(chk.check_blocks(b, h, qb0, qb1, tau, o[b, h, r0:r1],
                                           lse[b, h, r0:r1], mask[b, h, qb0:qb1]))
            reps[tau] = rep
        return reps

    total = {tau: _parity.Report() for tau in out}
    with _one_blas_thread(), ThreadPoolExecutor(_threads()) as ex:
        for i, reps in enumerate(ex.map(head, [(b, h) for b in range(B) for h in range(Hq)])):
            for tau, r in reps.items():
                total[tau].merge(r)
            if i % 8 == 7:
                print(f"[full] prefill_8k qk8 {fmt} {i + 1} of {B * Hq} heads checked",
                      flush=True)
    for tau, rep in total.items():
        print(f"[full] prefill_8k qk8 {fmt} tau={tau} blocks={B * Hq * nt} {rep}", flush=True)
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("qk8", [False, True], ids=["qk_bf16", "qk_fp8"])
def test_prefill_8k_pv8_every_block(qk8):
    # the prefill with the P.V product on fp8 (QK^T in bf16, or fp8 too) over
    # every query block of one query head per KV head of prefill_8k (8 of 32
    # heads, each KV head's code blocks in use) at every tau, against the
    # 8-bit P.V oracle on the oracle's codes: probabilities within the score
    # error of an E4M3 rounding point may round either way; with fp8 QK^T the
    # MFMA's accumulation error also widens O and LSE to first order
    import torch
    import long_context_tiled_amd as lib
    from oracle import fp8
    cfg = synth.workload("prefill_8k")
    print(f"[full] generating prefill_8k (pv8, qk8={qk8})", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nt = (N + 63) // 64
    ws = torch.empty(lib.attn_prefill_pv8_workspace_bytes(B, Hq, Hkv, N, d, qk8),
                     dtype=torch.uint8, device="cuda")
    out = {}
    for tau in cfg["taus"]:
        o, lse, mask, _ = lib.prefill_pv8(dq, dk, dv, True, tau, qk8=qk8, want_mask=True,
                                          workspace=ws)
        torch.cuda.synchronize()
        out[tau] = (o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy())
        del o, lse, mask
    parts = {n: t.cpu().numpy()
             for n, t in lib.pv8_workspace_parts(ws, B, Hq, Hkv, N, d, qk8).items()}
    del dq, dk, dv, ws
    torch.cuda.empty_cache()
    qf = kf = None
    if qk8:
        qc, qs = fp8.quantize(synth.bf16_bits_to_f32(q))
        kc, ks = fp8.quantize(synth.bf16_bits_to_f32(k))
        assert np.array_equal(parts["qc"], qc) and np.array_equal(parts["kc"], kc)
        qf, kf = fp8.dequantize(qc, qs), fp8.dequantize(kc, ks)

    def head(bh):
        b, h = bh
        chk = _parity.PrefillChecker(q, k, v, True, qf=qf, kf=kf, pv8=True,
                                     score_err_rel=2.0 ** -11 if qk8 else 2.0 ** -17,
                                     lin_err=qk8)
        reps = {}
        for tau, (o, lse, mask) in out.items():
            rep = _parity.Report()
            for qb in range(nt):
                r0, r1 = qb * 64, min(N, qb * 64 + 64)
                rep.merge(chk.check_block(b, h, qb, tau, o[b, h, r0:r1], lse[b, h, r0:r1],
                                          mask[b, h, qb]))
            reps[tau] = rep
        return reps

    G = Hq // Hkv
    heads = [(b, g * G + g % G) for b in range(B) for g in range(Hkv)]
    total = {tau: _parity.Report() for tau in out}
    with _one_blas_thread(), ThreadPoolExecutor(_threads()) as ex:
        for i, reps in enumerate(ex.map(head, heads)):
            for tau, r in reps.items():
                total[tau].merge(r)
            print(f"[full] prefill_8k pv8 qk8={qk8} {i + 1} of {len(heads)} heads checked",
                  flush=True)
    for tau, rep in total.items():
        print(f"[full] prefill_8k pv8 qk8={qk8} tau={tau} blocks={len(heads) * nt} {rep}",
              flush=True)
        assert rep.ok(), str(rep)
        assert rep.ambiguous <= len(heads) * nt // 100, str(rep)
