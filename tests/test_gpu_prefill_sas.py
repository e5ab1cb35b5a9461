"""GPU parity of attn_prefill_sas (the prefill with the SAS exponential)
against the SAS prefill oracle (oracle/sas.py), through the C ABI: skip
masks bit-exact (the exact rule's decisions), O and LSE within the prefill
tolerances beyond the slack of SAS arguments at its steps."""
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


def _case(**kw):
    base = dict(kind="prefill", B=1, Hq=2, Hkv=2, N=256, d=64, causal=False,
                sinks=False, band=False)
    base.update(kw)
    return base


SMALL = [
    ("tiny_sinks", _case(sinks=True, id=10), (INF, 4.0, 1.0)),
    ("gqa_causal_1k", _case(B=2, Hq=8, Hkv=2, N=1024, d=128, causal=True, sinks=True,
                            band=True, id=11), (INF, 8.0, 2.0)),
    ("ragged_causal_g3", _case(Hq=6, Hkv=2, N=1000, d=128, causal=True, sinks=True, id=12),
     (INF, 4.0)),
    ("ragged_full_g2_d64", _case(Hq=4, Hkv=2, N=300, d=64, sinks=True, id=13), (INF, 2.0)),
    ("g1_causal_d64_band", _case(Hq=3, Hkv=3, N=777, d=64, causal=True, sinks=True, band=True,
                                 id=14), (INF, 3.0)),
    # no sinks: row maxima rise over many tiles, so the rescale factor runs often
    ("g8_causal_rising", _case(Hq=8, Hkv=1, N=2048, d=128, causal=True, band=True, id=15),
     (INF, 4.0)),
]


@pytest.mark.parametrize("degree", [2, 3])
@pytest.mark.parametrize("name,cfg,taus", SMALL, ids=[s[0] for s in SMALL])
def test_prefill_sas_small(name, cfg, taus, degree):
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    for tau in taus:
        print(f"[prefill_sas] {name} degree={degree} tau={tau}", flush=True)
        o, lse, mask = lib.prefill(dq, dk, dv, cfg["causal"], tau, want_mask=True, sas=degree)
        torch.cuda.synchronize()
        rep = _parity.check_prefill(q, k, v, cfg["causal"], tau, o.cpu().numpy(),
                                    lse.cpu().numpy(), mask.cpu().numpy(), sas=degree)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_prefill_sas_degree_zero_is_attn_prefill():
    import torch
    import long_context_tiled_amd as lib
    q, k, v = synth.make_prefill(SMALL[1][1])
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    a = lib.prefill(dq, dk, dv, True, 4.0, want_mask=True)
    b = lib.prefill(dq, dk, dv, True, 4.0, want_mask=True, sas=0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_prefill_sas_rejects_bad_degree():
    import torch
    import long_context_tiled_amd as lib
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.SkipAttnError) as e:
        lib.prefill(q, q, q, True, 1.0, sas=4)
    assert e.value.code == lib.EINVAL


@pytest.mark.parametrize("degree", [2, 3])
def test_prefill_sas_workload_8k_sampled(degree):
    """prefill_8k in the launch configuration the benchmark times, query
    blocks spread over heads and positions, at every tau of the workload."""
    import torch
    import long_context_tiled_amd as lib
    cfg = synth.workload("prefill_8k")
    q, k, v = synth.make_prefill(cfg)
    dq, dk, dv = _dev(q), _dev(k), _dev(v)
    B, Hq, N, _ = q.shape
    nt = N // 64
    rng = np.random.default_rng(7)
    blocks = sorted({(0, int(rng.integers(Hq)), int(rng.integers(nt))) for _ in range(10)}
                    | {(0, 0, 0), (0, Hq - 1, nt - 1)})
    for tau in cfg["taus"]:
        print(f"[prefill_sas] prefill_8k degree={degree} tau={tau}", flush=True)
        o, lse, mask = lib.prefill(dq, dk, dv, True, tau, want_mask=True, sas=degree)
        torch.cuda.synchronize()
        rep = _parity.check_prefill(q, k, v, True, tau, o.cpu().numpy(), lse.cpu().numpy(),
                                    mask.cpu().numpy(), blocks=blocks, sas=degree)
        print(f"  {rep}", flush=True)
        assert rep.ok(), str(rep)
