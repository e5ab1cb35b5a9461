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
    ({"d": 96}, 1), ({"d": 256}, 1), ({"d": 0}, 1), ({"d": 32}, 1),
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
    assert rc == lib.EINVAL and "d must be" in lib.attn_last_error()


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
    ({"Hq": 16, "Hkv": 1}, 0), ({"Hq": 17, "Hkv": 1}, 0), ({"Hq": 64, "Hkv": 1}, 0),
    ({"B": 0, "ws": None, "wsb": 0}, 0),
    ({"q": None}, 1), ({"Hq": 65}, 1), ({"tau": math.nan}, 1), ({"tau": -0.5}, 1),
    ({"L": -1}, 1), ({"ws": P + 4}, 1),
    ({"d": 80}, 1),
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
    ({"d": 96}, 1), ({"Hq": 34, "Hkv": 2}, 0), ({"L": HEAD_LIMIT // 256 + 1}, 2),
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
    assert so.attn_kv_quantize_q4(P, P, P, P, P, P, 1, 8, 4096, 80, None) == lib.EINVAL
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
    ({"Nq": 100, "N": 4096}, 2), ({"Nq": 1, "N": 4096}, 2), ({"d": 96}, 1),
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


def test_capacity_entry_points_reject_before_any_launch():
    # a cache allocated for `cap` keys of which the first L (N) are used:
    # cap below the attended length is EINVAL; every case here returns before
    # any HIP call
    so = lib.load()
    ws = lib.attn_decode_workspace_bytes(2, 8, 5000, 128)
    assert so.attn_decode_cap(P, P, P, P, P, 2, 8, 2, 5000, 4999, 128, 4.0, 0, None, P, ws,
                              None) == lib.EINVAL
    assert "cap" in lib.attn_last_error()
    assert so.attn_decode_cap(P, P, P, P, P, 2, 8, 2, 5000, 8192, 128, 4.0, 1, None, P, ws,
                              None) == lib.EINVAL            # degree 1
    assert so.attn_decode_cap(P, P, P, P, P, 2, 8, 2, 5000, 8192, 128, 4.0, 0, None, P, ws - 4,
                              None) == lib.EWORKSPACE
    assert so.attn_decode_cap(P, P, P, P, P, 0, 8, 2, 5000, 8192, 128, 4.0, 0, None, None, 0,
                              None) == lib.OK                # empty work
    for fn in (so.attn_decode_q4_cap, so.attn_decode_q2_cap):
        assert fn(P, P, P, P, P, P, P, 2, 8, 2, 5000, 4096, 128, 4.0, 0, None, P, ws,
                  None) == lib.EINVAL
        assert fn(P, P, None, P, P, P, P, 2, 8, 2, 5000, 8192, 128, 4.0, 0, None, P, ws,
                  None) == lib.EINVAL
        assert fn(P, P, P, P, P, P, P, 2, 8, 2, 5000, 8192, 96, 4.0, 0, None, P, ws,
                  None) == lib.EINVAL
        assert fn(P, P, P, P, P, P, P, 0, 8, 2, 5000, 8192, 128, 4.0, 0, None, P, ws,
                  None) == lib.OK
    r = so.attn_prefill_chunk_cap
    assert r(P, P, P, P, P, 1, 8, 2, 512, 4096, 4095, 128, 1, 4.0, None, None) == lib.EINVAL
    assert r(P, P, P, P, P, 1, 8, 2, 100, 4096, 8192, 128, 1, 4.0, None, None) == lib.EUNSUPPORTED
    assert r(P, P, P, P, P, 0, 8, 2, 512, 4096, 8192, 128, 1, 4.0, None, None) == lib.OK
    assert r(P, P, P, P, P, 1 << 12, 8, 2, 512, 4096, 1 << 28, 128, 1, 4.0, None,
             None) == lib.EINVAL                             # cache beyond 2^40 elements


def test_noalloc_decode_rejects_before_any_launch():
    # the device scratch holds 32 MiB of per-split partials: a call needing
    # more is refused before any HIP call, as are invalid arguments
    so = lib.load()
    assert lib.attn_decode_workspace_bytes(16, 64, 131072, 128) <= lib.DECODE_SCRATCH_BYTES
    assert lib.attn_decode_workspace_bytes(32, 64, 131072, 128) > lib.DECODE_SCRATCH_BYTES
    rc = so.attn_decode_noalloc(P, P, P, P, P, 32, 64, 8, 131072, 128, INF, None, None)
    assert rc == lib.EWORKSPACE and "scratch" in lib.attn_last_error()
    assert so.attn_decode_noalloc(P, P, P, P, P, 16, 64, 8, 131072, 96, INF, None,
                                  None) == lib.EINVAL
    assert so.attn_decode_noalloc(None, P, P, P, P, 16, 64, 8, 131072, 128, INF, None,
                                  None) == lib.EINVAL
    assert so.attn_decode_noalloc(P, P, P, P, P, 0, 64, 8, 131072, 128, INF, None,
                                  None) == lib.OK


def test_prefill_sas_rejects_before_any_launch():
    so = lib.load()
    # an unknown degree, and attn_prefill's own checks (NULL pointer, head dim)
    assert so.attn_prefill_sas(P, P, P, P, P, 1, 8, 2, 1024, 128, 1, 4.0, 1, None,
                               None) == lib.EINVAL
    assert "degree" in lib.attn_last_error()
    assert so.attn_prefill_sas(None, P, P, P, P, 1, 8, 2, 1024, 128, 1, 4.0, 2, None,
                               None) == lib.EINVAL
    assert so.attn_prefill_sas(P, P, P, P, P, 1, 8, 2, 1024, 96, 1, 4.0, 3, None,
                               None) == lib.EINVAL


def _bits(*b):
    import ctypes
    return (ctypes.c_uint8 * len(b))(*b)


def test_hybrid_entry_points_reject_before_any_launch():
    so = lib.load()
    c4, c2 = [P] * 4, [P] * 4
    # quantiser: widths other than 4 and 2, NULL kv_bits, too many heads,
    # NULL arrays of a width that has heads, the single-width checks
    q = so.attn_kv_quantize_hybrid
    assert q(P, P, _bits(4, 3), *c4, *c2, 1, 2, 4096, 128, None) == lib.EINVAL
    assert "kv_bits[1]" in lib.attn_last_error()
    assert q(P, P, None, *c4, *c2, 1, 2, 4096, 128, None) == lib.EINVAL
    assert q(P, P, _bits(*([4] * 257)), *c4, *c2, 1, 257, 4096, 128, None) == lib.EUNSUPPORTED
    assert q(P, P, _bits(4, 2), *c4, None, P, P, P, 1, 2, 4096, 128, None) == lib.EINVAL
    assert q(P, P, _bits(4, 2), *c4, *c2, 1, 2, 4096, 96, None) == lib.EINVAL
    # the arrays of a width with no head are not looked at
    assert q(P, P, _bits(2, 2), P + 4, P, P, P, *c2, 0, 2, 4096, 128, None) == lib.OK
    assert q(P, P, _bits(4, 2), P + 4, P, P, P, *c2, 0, 2, 4096, 128, None) == lib.EINVAL
    # a width with no head takes NULL arrays (B = 0: nothing launched)
    assert q(P, P, _bits(2, 2), None, None, None, None, *c2, 0, 2, 4096, 128, None) == lib.OK
    assert q(P, P, _bits(4, 4), *c4, None, None, None, None, 0, 2, 4096, 128, None) == lib.OK
    r = so.attn_kv_quantize_hybrid_range
    assert r(P, P, _bits(4, 2), *c4, *c2, 1, 2, 4096, 128, 32, 64, None) == lib.EUNSUPPORTED
    assert r(P, P, _bits(4, 2), *c4, *c2, 1, 2, 4096, 128, 0, 4097, None) == lib.EINVAL
    # decode
    ws = lib.attn_decode_workspace_bytes(16, 64, 4096, 128)
    d = so.attn_decode_hybrid
    args = lambda bits, a4, a2, **kw: ([P, bits, *a4, *a2, P, P, kw.get("B", 16), kw.get("Hq", 64),
                                        kw.get("Hkv", 8), 4096, kw.get("d", 128), 4.0, None, P,
                                        kw.get("ws", ws), None])
    b8 = _bits(4, 2, 4, 2, 4, 2, 4, 2)
    assert d(*args(b8, c4, c2, d=96)) == lib.EINVAL
    assert d(*args(b8, c4, c2, ws=ws - 1)) == lib.EWORKSPACE
    assert d(*args(b8, c4, [P, None, P, P])) == lib.EINVAL
    assert d(*args(b8, [P, P, P + 8, P], c2)) == lib.EINVAL
    assert d(*args(_bits(4, 2, 4, 2, 4, 2, 4, 1), c4, c2)) == lib.EINVAL
    assert d(*args(b8, c4, c2, Hq=60)) == lib.EINVAL
    assert d(*args(_bits(4, 4, 4, 4, 4, 4, 4, 4), c4, [None] * 4, B=0)) == lib.OK
    dc = so.attn_decode_hybrid_cap
    base = [P, b8, *c4, *c2, P, P, 16, 64, 8, 4096]
    tail = [None, P, lib.attn_decode_workspace_bytes(16, 64, 4096, 128), None]
    assert dc(*base, 4000, 128, 4.0, 0, *tail) == lib.EINVAL      # cap < L
    assert dc(*base, 8192, 128, 4.0, 1, *tail) == lib.EINVAL      # degree 1
    assert "degree" in lib.attn_last_error()


def test_prefill_pv8_rejects_before_any_launch():
    so = lib.load()
    ws = lib.attn_prefill_pv8_workspace_bytes(1, 8, 2, 1024, 128, True)
    assert ws > lib.attn_prefill_pv8_workspace_bytes(1, 8, 2, 1024, 128, False) > 0
    assert lib.attn_prefill_pv8_workspace_bytes(1, 8, 2, 1024, 96, False) == 0
    call = lambda **kw: so.attn_prefill_pv8(
        kw.get("q", P), P, P, P, P, 1, 8, 2, 1024, kw.get("d", 128), 1, 4.0, kw.get("qk8", 1),
        None, kw.get("ws", P), kw.get("wsb", ws), None)
    assert call(qk8=2) == lib.EINVAL and "qk8" in lib.attn_last_error()
    assert call(wsb=ws - 1) == lib.EWORKSPACE
    assert call(ws=None) == lib.EWORKSPACE
    assert call(ws=P + 8) == lib.EINVAL
    assert call(q=None) == lib.EINVAL
    assert call(d=96) == lib.EINVAL


def test_prefill_8bit_qk_rejects_before_any_launch():
    # fp8 and int8 QK^T share the workspace layout and the checks
    so = lib.load()
    ws = lib.attn_prefill_qk8_workspace_bytes(1, 8, 2, 1024, 128)
    assert ws > 0 and lib.attn_prefill_qk8_workspace_bytes(1, 8, 2, 1024, 96) == 0
    for fn in (so.attn_prefill_qk8, so.attn_prefill_qki8):
        call = lambda fn=fn, **kw: fn(
            kw.get("q", P), P, P, P, P, 1, 8, 2, 1024, kw.get("d", 128), 1, kw.get("tau", 4.0),
            None, kw.get("ws", P), kw.get("wsb", ws), None)
        assert call(wsb=ws - 1) == lib.EWORKSPACE and "workspace" in lib.attn_last_error()
        assert call(ws=None) == lib.EWORKSPACE
        assert call(ws=P + 8) == lib.EINVAL
        assert call(q=None) == lib.EINVAL
        assert call(d=96) == lib.EINVAL
        assert call(tau=-1.0) == lib.EINVAL
