"""GPU parity of attn_prefill_chunk: a chunk of Nq queries at the end of N
positions. A causal chunk starting on a tile boundary must reproduce the
corresponding rows of the full prefill bit for bit (same tiles, same
order) and match the fp64 oracle; a non-causal chunk may start anywhere and
is checked against the oracle on its own 64-row tiles."""
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


def _np(t):
    return t.cpu().numpy()


CASES = [  # (name, cfg, q0 list)
    ("gqa4_ragged", dict(kind="prefill", id=90, B=1, Hq=8, Hkv=2, N=1000, d=128, causal=True,
                         sinks=True, band=True), (0, 64, 512, 960)),
    ("d64_g1", dict(kind="prefill", id=91, B=2, Hq=2, Hkv=2, N=700, d=64, causal=True,
                    sinks=True, band=False), (128, 640)),
    ("g16", dict(kind="prefill", id=92, B=1, Hq=16, Hkv=1, N=2048, d=128, causal=True,
                 sinks=True, band=True), (1024, 1984)),
]


@pytest.mark.parametrize("name,cfg,q0s", CASES, ids=[c[0] for c in CASES])
def test_causal_chunk_is_rows_of_full_prefill(name, cfg, q0s):
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    N = q.shape[2]
    for tau in (INF, 4.0):
        print(f"[chunk] {name} full tau={tau}", flush=True)
        fo, fl, fm = lib.prefill(dq, dk, dv, True, tau, want_mask=True)
        torch.cuda.synchronize()
        fo, fl, fm = _np(fo), _np(fl), _np(fm)
        for q0 in q0s:
            print(f"[chunk] {name} q0={q0} tau={tau}", flush=True)
            co, cl, cm = lib.prefill_chunk(_dev(q[:, :, q0:]), dk, dv, True, tau, want_mask=True)
            torch.cuda.synchronize()
            co, cl, cm = _np(co), _np(cl), _np(cm)
            assert np.array_equal(co, fo[:, :, q0:]), "O differs from the full prefill's rows"
            assert np.array_equal(cl, fl[:, :, q0:]), "LSE differs from the full prefill's rows"
            assert np.array_equal(cm, fm[:, :, q0 // 64:]), "mask differs"
            B, Hq = q.shape[:2]
            nqb = (N - q0 + 63) // 64
            blocks = _parity.sample_blocks(B, Hq, nqb, True, min(12, B * Hq * nqb), seed=q0)
            rep = _parity.check_prefill(q[:, :, q0:], k, v, True, tau, co, cl, cm, blocks, q0=q0)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)


def test_noncausal_chunk_any_start():
    import torch
    import long_context_tiled_amd as lib
    cfg = dict(kind="prefill", id=93, B=1, Hq=4, Hkv=2, N=900, d=128, causal=False,
               sinks=True, band=False)
    q, k, v = synth.make_prefill(cfg)
    dk, dv = _dev(k), _dev(v)
    full = lib.prefill(_dev(q), dk, dv, False, INF)
    torch.cuda.synchronize()
    for q0 in (0, 100, 899):
        for tau in (INF, 3.0):
            print(f"[chunk] non-causal q0={q0} tau={tau}", flush=True)
            co, cl, cm = lib.prefill_chunk(_dev(q[:, :, q0:]), dk, dv, False, tau, want_mask=True)
            torch.cuda.synchronize()
            co, cl, cm = _np(co), _np(cl), _np(cm)
            if tau == INF:   # each row's result does not depend on its tile
                assert np.array_equal(co, _np(full[0])[:, :, q0:])
                assert np.array_equal(cl, _np(full[1])[:, :, q0:])
            rep = _parity.check_prefill(q[:, :, q0:], k, v, False, tau, co, cl, cm, None, q0=q0)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)


def test_chunk_rejects_unaligned_causal_start():
    import long_context_tiled_amd as lib
    q, k, v = synth.make_prefill(dict(kind="prefill", id=94, B=1, Hq=2, Hkv=2, N=256, d=64,
                                      causal=True, sinks=False, band=False))
    with pytest.raises(lib.SkipAttnError) as e:
        lib.prefill_chunk(_dev(q[:, :, 10:]), _dev(k), _dev(v), True, INF)
    assert e.value.code == lib.EUNSUPPORTED
