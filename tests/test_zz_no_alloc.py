"""attn_decode_noalloc, the decode entry point that allocates nothing (its
per-split partials live in the library's device scratch), against
attn_decode with a caller workspace on the same inputs: outputs, LSEs and
skip masks identical bit for bit, on calls in a row of decreasing size (the
scratch keeps the previous call's contents), plus the fp64 oracle on a
sample of heads."""
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


CASES = [  # largest first: every later call reuses a scratch holding more
    dict(kind="decode", id=130, B=4, Hq=16, Hkv=2, L=20000, d=128, sinks=True, window=True),
    dict(kind="decode", id=131, B=2, Hq=8, Hkv=8, L=3000, d=64, sinks=True, window=True),
    dict(kind="decode", id=132, B=1, Hq=4, Hkv=1, L=70, d=128, sinks=True, window=False),
]


def test_noalloc_decode_matches_workspace_decode():
    import torch
    import long_context_tiled_amd as lib
    for i, cfg in enumerate(CASES):
        q, k, v = synth.make_decode(cfg)
        dq, dk, dv = _dev(q), _dev(k), _dev(v)
        B, Hq, d = q.shape
        nt = (k.shape[2] + 63) // 64
        for tau in (INF, 4.0):
            print(f"[noalloc] call {i} B={B} Hq={Hq} L={k.shape[2]} d={d} tau={tau}", flush=True)
            o1, l1, m1 = lib.decode(dq, dk, dv, tau, want_mask=True)
            o2 = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
            l2 = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
            m2 = torch.full((B, Hq, nt), 7, dtype=torch.uint8, device="cuda")
            lib.attn_decode_noalloc(dq, dk, dv, o2, l2, tau, m2)
            torch.cuda.synchronize()
            o1, l1, m1 = o1.cpu().numpy(), l1.cpu().numpy(), m1.cpu().numpy()
            o2, l2, m2 = o2.cpu().numpy(), l2.cpu().numpy(), m2.cpu().numpy()
            assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), "O differs"
            assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), "LSE differs"
            assert np.array_equal(m1, m2), "mask differs"
            heads = [(b, h) for b in range(B) for h in range(Hq)][:: max(1, B * Hq // 8)]
            rep = _parity.check_decode(q, k, v, tau, o2, l2, m2, heads=heads)
            print(f"  {rep}", flush=True)
            assert rep.ok(), str(rep)


def test_noalloc_decode_rejects_more_than_the_scratch():
    import torch
    import long_context_tiled_amd as lib
    # partials of B = 1, Hq = 2048, L = 131072, d = 128: 34.6 MB > 32 MiB
    q = torch.zeros((1, 2048, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((1, 2048, 128), dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, 2048), dtype=torch.float32, device="cuda")
    so = lib.load()
    rc = so.attn_decode_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), 1, 2048, 1, 131072, 128, INF, None, None)
    assert rc == lib.EWORKSPACE and "scratch" in lib.attn_last_error()
