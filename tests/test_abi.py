"""The C ABI on the CPU: the library loads, exports every declared symbol,
and validates arguments (no GPU needed: validation runs before any HIP call)."""
import math
import os
import re

import pytest

import long_context_tiled_amd as lib

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "skipattn.h")
P = 0x10000          # a fake, 16-byte aligned device address; never dereferenced
INF = math.inf


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(attn_\w+)\s*\(", text))


def test_exports_every_declared_symbol():
    names = _declared()
    assert names == set(lib.EXPORTS)
    so = lib.load()
    for n in names:
        assert hasattr(so, n), n


HEAD_LIMIT = (1 << 31) - (1 << 16)  # bytes of one (b, head) slice of K or V


def _pcheck(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=8, Hkv=2, N=1024, d=128, causal=1,
             tau=4.0, mask=None)
    a.update(kw)
    return lib.load().attn_prefill_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                         a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                                         a["tau"], a["mask"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0), ({"tau": INF}, 0), ({"tau": 0.0}, 0), ({"d": 64}, 0), ({"causal": 0}, 0),
    ({"N": 1000}, 0), ({"B": 0}, 0), ({"N": 0}, 0), ({"Hq": 6, "Hkv": 2}, 0),
    ({"q": None}, 1), ({"k": None}, 1), ({"v": None}, 1), ({"o": None}, 1), ({"lse": None}, 1),
    ({"B": -1}, 1), ({"N": -5}, 1), ({"Hq": 0}, 1), ({"Hkv": 0}, 1), ({"Hq": 7, "Hkv": 2}, 1),
    ({"causal": 2}, 1), ({"tau": math.nan}, 1), ({"tau": -1.0}, 1), ({"tau": -INF}, 1),
    ({"q": P + 8}, 1), ({"o": P + 4}, 1), ({"B": 1 << 20, "N": 1 << 20}, 1),
    ({"d": 96}, 2), ({"d": 256}, 2), ({"d": 0}, 2),
    # one head of K/V must stay below 2^31 - 2^16 bytes (32-bit buffer offsets)
    ({"N": HEAD_LIMIT // 256}, 0), ({"N": HEAD_LIMIT // 256 + 1}, 2),
    ({"N": HEAD_LIMIT // 128 + 1, "d": 64}, 2),
])
def test_prefill_validation(kw, code):
    assert _pcheck(**kw) == code
    if code:
        assert lib.attn_last_error()


def test_prefill_entry_rejects_before_any_launch():
    so = lib.load()
    rc = so.attn_prefill(None, P, P, P, P, 1, 8, 2, 1024, 128, 1, 4.0, None, None)
    assert rc == lib.EINVAL and "NULL" in lib.attn_last_error()
    rc = so.attn_prefill(P, P, P, P, P, 1, 8, 2, 1024, 96, 1, 4.0, None, None)
    assert rc == lib.EUNSUPPORTED


def _dcheck(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=16, Hq=64, Hkv=8, L=131072, d=128, tau=4.0,
             mask=None, ws=P, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.attn_decode_workspace_bytes(a["B"], a["Hq"], a["L"], a["d"])
    return lib.load().attn_decode_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                        a["Hq"], a["Hkv"], a["L"], a["d"], a["tau"],
                                        a["mask"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0), ({"tau": INF}, 0), ({"L": 1}, 0), ({"L": 4097}, 0), ({"d": 64}, 0),
    ({"Hq": 16, "Hkv": 1}, 0), ({"B": 0, "ws": None, "wsb": 0}, 0),
    ({"q": None}, 1), ({"Hq": 65}, 1), ({"tau": math.nan}, 1), ({"tau": -0.5}, 1),
    ({"L": -1}, 1), ({"ws": P + 4}, 1),
    ({"Hq": 17, "Hkv": 1}, 2), ({"d": 80}, 2),
    ({"L": HEAD_LIMIT // 256}, 0), ({"L": HEAD_LIMIT // 256 + 1}, 2),
    ({"L": HEAD_LIMIT // 128 + 1, "d": 64}, 2),
    ({"ws": None}, 3), ({"wsb": 100}, 3),
])
def test_decode_validation(kw, code):
    assert _dcheck(**kw) == code


def test_decode_workspace_size():
    assert lib.attn_decode_workspace_bytes(16, 64, 131072, 128) == 16 * 64 * 32 * 129 * 4
    assert lib.attn_decode_workspace_bytes(1, 8, 4097, 64) == 8 * 2 * 65 * 4
    assert lib.attn_decode_workspace_bytes(0, 8, 100, 64) == 0
    need = lib.attn_decode_workspace_bytes(2, 8, 5000, 128)
    assert _dcheck(B=2, Hq=8, Hkv=2, L=5000, wsb=need) == 0
    assert _dcheck(B=2, Hq=8, Hkv=2, L=5000, wsb=need - 1) == 3


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    o = torch.zeros((1, 2, 64, 64), dtype=torch.float32)
    lse = torch.zeros((1, 2, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        lib.attn_prefill(q, q, q, o, lse, True, 1.0)


def _q4check(**kw):
    a = dict(q=P, kq=P, kp=P, vq=P, vp=P, o=P, lse=P, B=16, Hq=64, Hkv=8, L=131072, d=128,
             tau=4.0, mask=None, ws=P, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.attn_decode_workspace_bytes(a["B"], a["Hq"], a["L"], a["d"])
    return lib.load().attn_decode_q4_check(a["q"], a["kq"], a["kp"], a["vq"], a["vp"], a["o"],
                                           a["lse"], a["B"], a["Hq"], a["Hkv"], a["L"], a["d"],
                                           a["tau"], a["mask"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0), ({"tau": INF}, 0), ({"L": 70, "d": 64}, 0), ({"B": 0, "ws": None, "wsb": 0}, 0),
    ({"kq": None}, 1), ({"kp": None}, 1), ({"vq": None}, 1), ({"vp": None}, 1),
    ({"kp": P + 4}, 1), ({"vq": P + 8}, 1), ({"q": None}, 1), ({"tau": -1.0}, 1),
    ({"d": 96}, 2), ({"Hq": 34, "Hkv": 2}, 2), ({"L": HEAD_LIMIT // 256 + 1}, 2),
    ({"wsb": 64}, 3),
])
def test_decode_q4_validation(kw, code):
    assert _q4check(**kw) == code


def test_quantise_q4_rejects_before_any_launch():
    so = lib.load()
    # every case returns before any HIP call (B = 0 is empty work)
    assert so.attn_kv_quantize_q4(P, P, P, P, P, P, 0, 8, 4096, 128, None) == lib.OK
    assert so.attn_kv_quantize_q4(None, P, P, P, P, P, 1, 8, 4096, 128, None) == lib.EINVAL
    assert so.attn_kv_quantize_q4(P, P, P, P + 4, P, P, 1, 8, 4096, 128, None) == lib.EINVAL
    assert so.attn_kv_quantize_q4(P, P, P, P, P, P, 1, 0, 4096, 128, None) == lib.EINVAL
    assert so.attn_kv_quantize_q4(P, P, P, P, P, P, 1, 8, 4096, 80, None) == lib.EUNSUPPORTED
    assert so.attn_kv_quantize_q4(P, P, P, P, P, P, 1, 1, HEAD_LIMIT // 256 + 1, 128,
                                  None) == lib.EUNSUPPORTED


def test_q4_shapes():
    s = lib.q4_shapes(2, 3, 130, 64)
    assert s == dict(kq=(2, 3, 130, 32), kp=(2, 3, 130), vq=(2, 3, 3, 64, 32), vp=(2, 3, 3, 64))


def _ccheck(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=8, Hkv=2, Nq=512, N=4096, d=128, causal=1,
             tau=4.0, mask=None)
    a.update(kw)
    return lib.load().attn_prefill_chunk_check(a["q"], a["k"], a["v"], a["o"], a["lse"],
                                               a["B"], a["Hq"], a["Hkv"], a["Nq"], a["N"],
                                               a["d"], a["causal"], a["tau"], a["mask"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0), ({"Nq": 4096}, 0), ({"Nq": 0}, 0), ({"Nq": 64, "N": 4160}, 0),
    ({"Nq": 100, "N": 164}, 0), ({"Nq": 100, "N": 4096, "causal": 0}, 0),
    ({"Nq": 4097}, 1), ({"Nq": -1}, 1), ({"q": None}, 1), ({"causal": 3}, 1),
    ({"Nq": 100, "N": 4096}, 2), ({"Nq": 1, "N": 4096}, 2), ({"d": 96}, 2),
])
def test_prefill_chunk_validation(kw, code):
    assert _ccheck(**kw) == code


def test_quantise_q4_range_rejects_before_any_launch():
    so = lib.load()
    r = so.attn_kv_quantize_q4_range
    assert r(P, P, P, P, P, P, 1, 8, 4096, 128, 64, 64, None) == lib.OK       # empty range
    assert r(P, P, P, P, P, P, 1, 8, 4096, 128, 10, 100, None) == lib.EUNSUPPORTED
    assert r(P, P, P, P, P, P, 1, 8, 4096, 128, 128, 64, None) == lib.EINVAL
    assert r(P, P, P, P, P, P, 1, 8, 4096, 128, 0, 4097, None) == lib.EINVAL
    assert r(P, P, P, P, P, P, 1, 8, 4096, 128, -64, 64, None) == lib.EINVAL
