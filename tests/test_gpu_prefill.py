"""GPU parity of attn_prefill against the fp64 oracle (through the C ABI)."""
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


def _run(q, k, v, causal, tau):
    import torch
    import long_context_tiled_amd as lib
    o, lse, mask = lib.prefill(_dev(q), _dev(k), _dev(v), causal, tau, want_mask=True)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy()


def _case(**kw):
    base = dict(kind="prefill", B=1, Hq=2, Hkv=2, N=256, d=64, causal=False,
                sinks=False, band=False)
    base.update(kw)
    return base


SMALL = [
    ("tiny", synth.workload("tiny"), (INF, 4.0)),
    ("tiny_sinks", _case(sinks=True, id=10), (INF, 4.0, 1.0)),
    ("gqa_causal_1k", _case(B=2, Hq=8, Hkv=2, N=1024, d=128, causal=True, sinks=True,
                            band=True, id=11), (INF, 8.0, 4.0, 2.0)),
    ("ragged_causal_g3", _case(Hq=6, Hkv=2, N=1000, d=128, causal=True, sinks=True,
                               id=12), (INF, 4.0)),
    ("ragged_full_g2_d64", _case(Hq=4, Hkv=2, N=300, d=64, sinks=True, id=13), (INF, 2.0)),
    ("g1_causal_d64", _case(Hq=3, Hkv=3, N=777, d=64, causal=True, sinks=True, band=True,
                            id=14), (INF, 3.0)),
    ("g8_causal_d128", _case(Hq=8, Hkv=1, N=2048, d=128, causal=True, sinks=True,
                             band=True, id=15), (INF, 12.0, 4.0)),
]


@pytest.mark.parametrize("name,cfg,taus", SMALL, ids=[s[0] for s in SMALL])
def test_prefill_small_full(name, cfg, taus):
    q, k, v = synth.make_prefill(cfg)
    for tau in taus:
        print(f"[prefill] {name} tau={tau}", flush=True)
        o, lse, mask = _run(q, k, v, cfg["causal"], tau)
        rep = _parity.check_prefill(q, k, v, cfg["causal"], tau, o, lse, mask)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_edge_lengths(N, causal):
    cfg = _case(Hq=4, Hkv=1, N=N, d=128, causal=causal, sinks=True, id=20 + N)
    q, k, v = synth.make_prefill(cfg)
    for tau in (INF, 0.0, 2.0):
        print(f"[prefill] edge N={N} causal={causal} tau={tau}", flush=True)
        o, lse, mask = _run(q, k, v, causal, tau)
        rep = _parity.check_prefill(q, k, v, causal, tau, o, lse, mask)
        assert rep.ok(), str(rep)


def test_prefill_empty_is_noop():
    import torch
    import long_context_tiled_amd as lib
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 1, 16, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((0, 2, 16, 64), dtype=torch.float32, device="cuda")
    lse = torch.zeros((0, 2, 16), dtype=torch.float32, device="cuda")
    # torch gives empty tensors a non-null, aligned pointer or null; pass a
    # real buffer so the pointer checks see valid addresses
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    rc = lib.load().attn_prefill(buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                 buf.data_ptr(), buf.data_ptr(), 0, 2, 1, 16, 64, 1,
                                 1.0, None, None)
    assert rc == 0
    rc = lib.load().attn_prefill(buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                 buf.data_ptr(), buf.data_ptr(), 1, 2, 1, 0, 64, 1,
                                 1.0, None, None)
    assert rc == 0
    torch.cuda.synchronize()
    del q, k, o, lse


def test_prefill_deterministic():
    cfg = _case(Hq=8, Hkv=2, N=512, d=128, causal=True, sinks=True, id=30)
    q, k, v = synth.make_prefill(cfg)
    a = _run(q, k, v, True, 4.0)
    b = _run(q, k, v, True, 4.0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_without_mask_matches(causal):
    """Without a skip-mask buffer the kernel keeps a tile's copies in flight
    across the barrier (with one it waits for all stores); O and LSE must be
    bit-identical either way, and match the oracle."""
    import torch
    import long_context_tiled_amd as lib
    cfg = _case(Hq=8, Hkv=2, N=1000, d=128, causal=causal, sinks=True, band=True, id=32)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    o1, l1, m1 = lib.prefill(dq, dk, dv, causal, 4.0, want_mask=True)
    o2, l2, _ = lib.prefill(dq, dk, dv, causal, 4.0, want_mask=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
    rep = _parity.check_prefill(q, k, v, causal, 4.0, o2.cpu().numpy(), l2.cpu().numpy(),
                                m1.cpu().numpy())
    assert rep.ok(), str(rep)


def test_prefill_reading_p_has_no_skips():
    """Under the literal amplitude reading the structure adds < 1 logit, so
    no tile can be skipped at tau >= 2: every sweep equals dense."""
    cfg = _case(Hq=8, Hkv=2, N=1024, d=128, causal=True, sinks=True, band=True, id=31)
    q, k, v = synth.make_prefill(cfg, reading="P")
    o, lse, mask = _run(q, k, v, True, 4.0)
    assert not (mask == 1).any()
    rep = _parity.check_prefill(q, k, v, True, 4.0, o, lse, mask)
    assert rep.ok(), str(rep)


# ---- the workloads at full size: sampled blocks, properties at every block

FULL = [("prefill_8k", 48), ("prefill_32k", 24), ("prefill_128k", 12)]


@pytest.mark.parametrize("name,count", FULL, ids=[f[0] for f in FULL])
def test_prefill_workload_sampled(name, count):
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload(name)
    print(f"[prefill] generating {name}", flush=True)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    nt = (N + 63) // 64
    blocks = _parity.sample_blocks(B, Hq, nt, True, count, seed=len(name))
    prev = None
    for tau in cfg["taus"]:
        print(f"[prefill] {name} tau={tau}", flush=True)
        o, lse, mask = lib.prefill(dq, dk, dv, True, tau, want_mask=True)
        torch.cuda.synchronize()
        mask_np = mask.cpu().numpy()
        # every tile above the diagonal is marked not-visited, none below
        tri = np.triu(np.ones((nt, nt), bool), 1)
        assert (mask_np[..., tri] == 2).all() and not (mask_np[..., ~tri] == 2).any()
        if prev is not None:  # skip(tau1) is contained in skip(tau2) for tau1 > tau2
            assert ((prev == 1) <= (mask_np == 1)).all()
        prev = mask_np
        rows = sorted({(b, h) for b, h, _ in blocks})
        o_rows = {bh: o[bh[0], bh[1]].cpu().numpy() for bh in rows}
        lse_np = lse.cpu().numpy()
        assert np.isfinite(lse_np).all()
        chk = _parity.PrefillChecker(q, k, v, True)
        rep = _parity.Report()
        for b, h, qb in sorted(blocks, key=lambda x: (x[0], x[1] // (Hq // k.shape[1]), x[1])):
            r0, r1 = qb * 64, min(N, qb * 64 + 64)
            rep.merge(chk.check_block(b, h, qb, tau, o_rows[(b, h)][r0:r1],
                                      lse_np[b, h, r0:r1], mask_np[b, h, qb]))
        frac = float((mask_np == 1).sum()) / float((mask_np != 2).sum())
        print(f"  skip_fraction={frac:.4f} {rep}", flush=True)
        assert rep.ok(), str(rep)
        del o, lse, mask


def test_prefill_work_queue_reuse_and_streams():
    """The persistent grid takes work items from a per-call device counter
    pair that the call's last workgroup returns to zero. More calls than
    there are counter slots, alternating between two streams with outputs
    pre-filled with NaN, must each reproduce the first call's bytes (a lost
    or doubly taken item would leave NaN or differ)."""
    import torch
    import long_context_tiled_amd as lib
    # 2 x 4 KV groups x 64 query tiles = 512 work items, more than the CUs
    cfg = _case(B=2, Hq=16, Hkv=4, N=4096, d=128, causal=True, sinks=True, band=True,
                id=16)
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, d = q.shape
    o_ref = torch.empty((B, Hq, N, d), dtype=torch.float32, device="cuda")
    l_ref = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    lib.attn_prefill(dq, dk, dv, o_ref, l_ref, True, 4.0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(torch.empty_like(o_ref), torch.empty_like(l_ref)) for _ in streams]
    bad = []
    for i in range(1100):
        s = i % 2
        o, l = outs[s]
        with torch.cuda.stream(streams[s]):
            o.fill_(math.nan)
            l.fill_(math.nan)
            lib.attn_prefill(dq, dk, dv, o, l, True, 4.0)
        if i % 2 == 1 or i == 1099:
            torch.cuda.synchronize()
            for j in ((0, 1) if i % 2 == 1 else (0,)):
                oj, lj = outs[j]
                if not (torch.equal(oj, o_ref) and torch.equal(lj, l_ref)):
                    bad.append(i - (i % 2) + j)
    print(f"[prefill] 1100 calls on two streams: {len(bad)} differ", flush=True)
    assert not bad, bad[:10]
