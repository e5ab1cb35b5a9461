"""GPU parity of attn_decode (split-K + LSE merge) against the fp64 oracle."""
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


def _run(q, k, v, tau):
    import torch
    import long_context_tiled_amd as lib
    o, lse, mask = lib.decode(_dev(q), _dev(k), _dev(v), tau, want_mask=True)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy()


def _case(**kw):
    base = dict(kind="decode", B=2, Hq=8, Hkv=2, L=10000, d=128, sinks=True,
                window=True)
    base.update(kw)
    return base


SMALL = [
    ("gqa4_ragged_3splits", _case(id=40), (INF, 8.0, 4.0, 1.0)),
    ("g1_d64_one_split", _case(B=1, Hq=2, Hkv=2, L=4096, d=64, id=41), (INF, 2.0)),
    ("g8_split_edge", _case(B=1, Hq=8, Hkv=1, L=4097, id=42), (INF, 4.0)),
    ("g16", _case(B=1, Hq=16, Hkv=1, L=9000, id=43), (INF, 3.0)),
    ("g3_d64", _case(B=3, Hq=6, Hkv=2, L=12345, d=64, id=44), (INF, 0.0, 2.0)),
]


@pytest.mark.parametrize("name,cfg,taus", SMALL, ids=[s[0] for s in SMALL])
def test_decode_small_full(name, cfg, taus):
    q, k, v = synth.make_decode(cfg)
    for tau in taus:
        print(f"[decode] {name} tau={tau}", flush=True)
        o, lse, mask = _run(q, k, v, tau)
        rep = _parity.check_decode(q, k, v, tau, o, lse, mask)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 4095, 4096, 4160, 8193])
def test_decode_edge_lengths(L):
    cfg = _case(B=1, Hq=4, Hkv=1, L=L, id=50)
    q, k, v = synth.make_decode(cfg)
    for tau in (INF, 0.0, 3.0):
        print(f"[decode] edge L={L} tau={tau}", flush=True)
        o, lse, mask = _run(q, k, v, tau)
        rep = _parity.check_decode(q, k, v, tau, o, lse, mask)
        assert rep.ok(), str(rep)


def test_decode_rejects_bad_workspace_and_head_dim():
    import torch
    import long_context_tiled_amd as lib
    q = torch.zeros((1, 32, 96), dtype=torch.bfloat16, device="cuda")
    k96 = torch.zeros((1, 1, 128, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.SkipAttnError) as e:
        lib.decode(q, k96, k96, 1.0)
    assert e.value.code == lib.EINVAL
    k = torch.zeros((1, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((1, 8, 128), dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, 8), dtype=torch.float32, device="cuda")
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.SkipAttnError) as e:
        lib.attn_decode(q, k, k, o, lse, 1.0, ws)
    assert e.value.code == lib.EWORKSPACE


def test_decode_workload_sampled():
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("decode_128k")
    print("[decode] generating decode_128k", flush=True)
    q, k, v = synth.make_decode(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, d = q.shape
    rng = np.random.default_rng(4)
    heads = sorted({(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(12)}
                   | {(0, 0), (B - 1, Hq - 1)})
    prev = None
    for tau in cfg["taus"]:
        print(f"[decode] decode_128k tau={tau}", flush=True)
        o, lse, mask = lib.decode(dq, dk, dv, tau, want_mask=True)
        torch.cuda.synchronize()
        mask_np = mask.cpu().numpy()
        # the first tile of every split is always kept
        assert (mask_np[:, :, ::64] == 0).all()
        if prev is not None:
            assert ((prev == 1) <= (mask_np == 1)).all()
        prev = mask_np
        rep = _parity.check_decode(q, k, v, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                   mask_np, heads=heads)
        print(f"  skip_fraction={(mask_np == 1).mean():.4f} {rep}", flush=True)
        assert rep.ok(), str(rep)
        del o, lse, mask
