"""ctypes binding of libskipattn (include/skipattn.h).

Argument marshalling only: torch tensors are checked for dtype, device,
contiguity and shape, turned into device pointers, and passed with torch's
current HIP stream. Every step of the computation runs in the library's HIP
kernels; there is no fallback path. Loading fails loudly if the library has
not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libskipattn.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
TILE = 64
SPLIT = 4096
KEPT, SKIPPED, NOT_VISITED = 0, 1, 2

EXPORTS = ("attn_prefill", "attn_decode", "attn_decode_workspace_bytes",
           "attn_prefill_check", "attn_decode_check", "attn_last_error",
           "attn_kv_quantize_q4", "attn_decode_q4", "attn_decode_q4_check",
           "attn_prefill_chunk", "attn_prefill_chunk_check", "attn_kv_quantize_q4_range",
           "attn_kv_quantize_q2", "attn_kv_quantize_q2_range", "attn_decode_q2",
           "attn_decode_q2_check", "attn_decode_sas", "attn_decode_q4_sas", "attn_prefill_sas",
           "attn_decode_q2_sas", "attn_prefill_chunk_cap", "attn_decode_cap",
           "attn_decode_q4_cap", "attn_decode_q2_cap", "attn_decode_noalloc",
           "attn_prefill_qk8", "attn_prefill_qk8_workspace_bytes", "attn_kv_quantize_hybrid",
           "attn_kv_quantize_hybrid_range", "attn_decode_hybrid", "attn_decode_hybrid_cap",
           "attn_prefill_pv8", "attn_prefill_pv8_workspace_bytes", "attn_prefill_qki8")

_lib = None


class SkipAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libskipattn error {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libskipattn.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build it with `python -m long_context_tiled_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, f32p, u8p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i, f, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, u8p, vp]
    lib.attn_prefill.restype = i
    lib.attn_prefill_check.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, u8p]
    lib.attn_prefill_check.restype = i
    lib.attn_prefill_chunk.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, i, f, u8p, vp]
    lib.attn_prefill_chunk.restype = i
    lib.attn_prefill_chunk_check.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, i, f, u8p]
    lib.attn_prefill_chunk_cap.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, i, i, f, u8p,
                                           vp]
    lib.attn_prefill_chunk_cap.restype = i
    lib.attn_prefill_chunk_check.restype = i
    lib.attn_decode.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp, sz, vp]
    lib.attn_decode.restype = i
    lib.attn_decode_sas.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, f, i, u8p, vp, sz, vp]
    lib.attn_decode_sas.restype = i
    lib.attn_prefill_sas.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, i, u8p, vp]
    lib.attn_prefill_sas.restype = i
    lib.attn_decode_cap.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, i, u8p, vp, sz,
                                    vp]
    lib.attn_decode_cap.restype = i
    lib.attn_prefill_qk8.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, u8p, vp, sz,
                                     vp]
    lib.attn_prefill_qk8.restype = i
    lib.attn_prefill_qki8.argtypes = lib.attn_prefill_qk8.argtypes
    lib.attn_prefill_qki8.restype = i
    lib.attn_prefill_pv8.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, i, u8p, vp, sz,
                                     vp]
    lib.attn_prefill_pv8.restype = i
    lib.attn_prefill_pv8_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_prefill_pv8_workspace_bytes.restype = sz
    lib.attn_prefill_qk8_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_prefill_qk8_workspace_bytes.restype = sz
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp]
    lib.attn_decode_noalloc.restype = i
    lib.attn_decode_check.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp, sz]
    lib.attn_decode_check.restype = i
    lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_decode_workspace_bytes.restype = sz
    for w in ("q4", "q2"):
        fn = getattr(lib, f"attn_kv_quantize_{w}")
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        fn.restype = i
        fn = getattr(lib, f"attn_kv_quantize_{w}_range")
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        fn.restype = i
        fn = getattr(lib, f"attn_decode_{w}")
        fn.argtypes = [vp, vp, vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp, sz, vp]
        fn.restype = i
        fn = getattr(lib, f"attn_decode_{w}_sas")
        fn.argtypes = [vp, vp, vp, vp, vp, f32p, f32p, i, i, i, i, i, f, i, u8p, vp, sz, vp]
        fn.restype = i
        fn = getattr(lib, f"attn_decode_{w}_cap")
        fn.argtypes = [vp, vp, vp, vp, vp, f32p, f32p, i, i, i, i, i, i, f, i, u8p, vp, sz, vp]
        fn.restype = i
        fn = getattr(lib, f"attn_decode_{w}_check")
        fn.argtypes = [vp, vp, vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp, sz]
        fn.restype = i
    c8 = [vp] * 8   # the two caches' kq, kp, vq, vp
    lib.attn_kv_quantize_hybrid.argtypes = [vp, vp, vp] + c8 + [i, i, i, i, vp]
    lib.attn_kv_quantize_hybrid.restype = i
    lib.attn_kv_quantize_hybrid_range.argtypes = [vp, vp, vp] + c8 + [i, i, i, i, i, i, vp]
    lib.attn_kv_quantize_hybrid_range.restype = i
    lib.attn_decode_hybrid.argtypes = [vp, vp] + c8 + [f32p, f32p, i, i, i, i, i, f, u8p, vp, sz,
                                                       vp]
    lib.attn_decode_hybrid.restype = i
    lib.attn_decode_hybrid_cap.argtypes = [vp, vp] + c8 + [f32p, f32p, i, i, i, i, i, i, f, i, u8p,
                                                           vp, sz, vp]
    lib.attn_decode_hybrid_cap.restype = i
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def _raise(rc: int):
    if rc != OK:
        raise SkipAttnError(rc, attn_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, shape):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def attn_prefill(q, k, v, o, lse, causal: bool, tau: float, skip_mask=None,
                 stream=None) -> None:
    """Enqueue prefill attention: q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16;
    writes o [B,Hq,N,d] fp32, lse [B,Hq,N] fp32 and, if given, skip_mask
    [B,Hq,ceil(N/64),ceil(N/64)] uint8."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _check(q, "q", torch.bfloat16, (B, Hq, N, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, N, d))
    _check(o, "o", torch.float32, (B, Hq, N, d))
    _check(lse, "lse", torch.float32, (B, Hq, N))
    if skip_mask is not None:
        nt = (N + TILE - 1) // TILE
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, nt, nt))
    rc = load().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                             Hkv, N, d, int(bool(causal)), float(tau),
                             _ptr(skip_mask), _stream(stream))
    _raise(rc)


def attn_prefill_sas(q, k, v, o, lse, causal: bool, tau: float, degree: int, skip_mask=None,
                     stream=None) -> None:
    """Enqueue attn_prefill_sas: attn_prefill with the SAS exponential of
    polynomial degree ``degree`` (2 or 3; 0 = exact)."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _check(q, "q", torch.bfloat16, (B, Hq, N, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, N, d))
    _check(o, "o", torch.float32, (B, Hq, N, d))
    _check(lse, "lse", torch.float32, (B, Hq, N))
    if skip_mask is not None:
        nt = (N + TILE - 1) // TILE
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, nt, nt))
    rc = load().attn_prefill_sas(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N,
                                 d, int(bool(causal)), float(tau), int(degree), _ptr(skip_mask),
                                 _stream(stream))
    _raise(rc)


def attn_prefill_chunk(q, k, v, o, lse, causal: bool, tau: float, skip_mask=None,
                       stream=None, N=None) -> None:
    """Enqueue chunked prefill: q [B,Hq,Nq,d] are the last Nq of the N
    positions held in k/v [B,Hkv,cap,d] (N = cap unless given: a cache
    allocated for cap keys whose first N exist); writes o [B,Hq,Nq,d],
    lse [B,Hq,Nq] and, if given, skip_mask [B,Hq,ceil(Nq/64),ceil(N/64)]."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    N = cap if N is None else int(N)
    _check(q, "q", torch.bfloat16, (B, Hq, Nq, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, cap, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, cap, d))
    _check(o, "o", torch.float32, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8,
               (B, Hq, (Nq + TILE - 1) // TILE, (N + TILE - 1) // TILE))
    so = load()
    if N == cap:
        rc = so.attn_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                   Nq, N, d, int(bool(causal)), float(tau), _ptr(skip_mask),
                                   _stream(stream))
    else:
        rc = so.attn_prefill_chunk_cap(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                       Hkv, Nq, N, cap, d, int(bool(causal)), float(tau),
                                       _ptr(skip_mask), _stream(stream))
    _raise(rc)


def attn_prefill_qk8_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(load().attn_prefill_qk8_workspace_bytes(B, Hq, Hkv, N, d))


def qk8_workspace_parts(workspace, B: int, Hq: int, Hkv: int, N: int, d: int) -> dict:
    """Views of an attn_prefill_qk8 workspace: Q codes uint8 [B,Hq,N,d], K
    codes [B,Hkv,N,d], Q scales fp32 [B,Hq,ceil(N/64)], K scales
    [B,Hkv,ceil(N/64)] (each part starts on a 256-byte boundary)."""
    import torch
    nt = (N + TILE - 1) // TILE
    al = lambda x: (x + 255) // 256 * 256
    sizes = [("qc", B * Hq * N * d), ("kc", B * Hkv * N * d), ("qs", B * Hq * nt * 4),
             ("ks", B * Hkv * nt * 4)]
    out, off = {}, 0
    w = workspace.view(torch.uint8)
    for name, n in sizes:
        out[name] = w[off:off + n]
        off += al(n)
    out["qc"] = out["qc"].view(B, Hq, N, d)
    out["kc"] = out["kc"].view(B, Hkv, N, d)
    out["qs"] = out["qs"].view(torch.float32).view(B, Hq, nt)
    out["ks"] = out["ks"].view(torch.float32).view(B, Hkv, nt)
    return out


def attn_prefill_qk8(q, k, v, o, lse, causal: bool, tau: float, workspace, skip_mask=None,
                     stream=None, int8: bool = False) -> None:
    """attn_prefill with QK^T on block-quantised fp8 (E4M3) Q and K, or
    (``int8``, attn_prefill_qki8) symmetric int8 ones; the workspace
    (attn_prefill_qk8_workspace_bytes) receives the codes and scales
    (qk8_workspace_parts)."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _check(q, "q", torch.bfloat16, (B, Hq, N, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, N, d))
    _check(o, "o", torch.float32, (B, Hq, N, d))
    _check(lse, "lse", torch.float32, (B, Hq, N))
    if skip_mask is not None:
        nt = (N + TILE - 1) // TILE
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, nt, nt))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    fn = load().attn_prefill_qki8 if int8 else load().attn_prefill_qk8
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)),
            float(tau), _ptr(skip_mask), _ptr(workspace), nbytes, _stream(stream))
    _raise(rc)


def attn_prefill_pv8_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int,
                                     qk8: bool) -> int:
    return int(load().attn_prefill_pv8_workspace_bytes(B, Hq, Hkv, N, d, int(bool(qk8))))


def pv8_workspace_parts(workspace, B: int, Hq: int, Hkv: int, N: int, d: int, qk8: bool) -> dict:
    """Views of an attn_prefill_pv8 workspace: V code blocks uint8
    [B,Hkv,ceil(N/64),d,64], the V tiles' largest |v| fp32 [B,Hkv,ceil(N/64)],
    the V scales fp32 [B,Hkv], and (qk8) the attn_prefill_qk8 parts (each
    part starts on a 256-byte boundary)."""
    import torch
    nt = (N + TILE - 1) // TILE
    al = lambda x: (x + 255) // 256 * 256
    w = workspace.view(torch.uint8)
    out, off = {}, 0
    for name, n in (("vc", B * Hkv * nt * TILE * d), ("vt", B * Hkv * nt * 4), ("vs", B * Hkv * 4)):
        out[name] = w[off:off + n]
        off += al(n)
    out["vc"] = out["vc"].view(B, Hkv, nt, d, TILE)
    out["vt"] = out["vt"].view(torch.float32).view(B, Hkv, nt)
    out["vs"] = out["vs"].view(torch.float32).view(B, Hkv)
    if qk8:
        out.update(qk8_workspace_parts(w[off:], B, Hq, Hkv, N, d))
    return out


def attn_prefill_pv8(q, k, v, o, lse, causal: bool, tau: float, workspace, qk8: bool = False,
                     skip_mask=None, stream=None) -> None:
    """attn_prefill with P.V on 8-bit operands (V as E4M3 codes with one scale
    per KV head, probabilities rounded to E4M3), QK^T in bf16 or (qk8) as in
    attn_prefill_qk8; the workspace (attn_prefill_pv8_workspace_bytes)
    receives the codes and scales (pv8_workspace_parts)."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _check(q, "q", torch.bfloat16, (B, Hq, N, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, N, d))
    _check(o, "o", torch.float32, (B, Hq, N, d))
    _check(lse, "lse", torch.float32, (B, Hq, N))
    if skip_mask is not None:
        nt = (N + TILE - 1) // TILE
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, nt, nt))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    rc = load().attn_prefill_pv8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N,
                                 d, int(bool(causal)), float(tau), int(bool(qk8)),
                                 _ptr(skip_mask), _ptr(workspace), nbytes, _stream(stream))
    _raise(rc)


def attn_decode_workspace_bytes(B: int, Hq: int, L: int, d: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, Hq, L, d))


def attn_decode(q, k, v, o, lse, tau: float, workspace, skip_mask=None,
                stream=None) -> None:
    """Enqueue split-K decode: q [B,Hq,d], k/v [B,Hkv,L,d] bf16; writes o
    [B,Hq,d] fp32, lse [B,Hq] fp32 and, if given, skip_mask [B,Hq,ceil(L/64)]
    uint8. ``workspace`` is a device tensor of at least
    attn_decode_workspace_bytes(B, Hq, L, d) bytes."""
    attn_decode_sas(q, k, v, o, lse, tau, 0, workspace, skip_mask, stream)


def attn_decode_sas(q, k, v, o, lse, tau: float, degree: int, workspace, skip_mask=None,
                    stream=None, L=None) -> None:
    """attn_decode with the SAS exponential of polynomial degree 2 or 3
    (0: exact exponentials, i.e. attn_decode). k/v may be a cache allocated
    for cap = k.shape[2] keys of which the first ``L`` are attended
    (attn_decode_cap); L defaults to cap."""
    import torch
    B, Hq, d = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    L = cap if L is None else int(L)
    _check(q, "q", torch.bfloat16, (B, Hq, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, cap, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, cap, d))
    _check(o, "o", torch.float32, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, (L + TILE - 1) // TILE))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    so = load()
    if L == cap:
        rc = so.attn_decode_sas(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                L, d, float(tau), int(degree), _ptr(skip_mask),
                                _ptr(workspace), nbytes, _stream(stream))
    else:
        rc = so.attn_decode_cap(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                L, cap, d, float(tau), int(degree), _ptr(skip_mask),
                                _ptr(workspace), nbytes, _stream(stream))
    _raise(rc)


DECODE_SCRATCH_BYTES = 32 << 20


def attn_decode_noalloc(q, k, v, o, lse, tau: float, skip_mask=None, stream=None) -> None:
    """attn_decode without a workspace: the per-split partials go to the
    library's 32 MiB device scratch (calls that overlap on one GPU race)."""
    import torch
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    _check(q, "q", torch.bfloat16, (B, Hq, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, L, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, L, d))
    _check(o, "o", torch.float32, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, (L + TILE - 1) // TILE))
    rc = load().attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                    L, d, float(tau), _ptr(skip_mask), _stream(stream))
    _raise(rc)


def q4_shapes(B: int, Hkv: int, L: int, d: int) -> dict:
    """Shapes of the 4-bit cache arrays (kq, kp, vq, vp)."""
    return _cache_shapes(4, B, Hkv, L, d)


def q2_shapes(B: int, Hkv: int, L: int, d: int) -> dict:
    """Shapes of the 2-bit cache arrays (kq, kp, vq, vp)."""
    return _cache_shapes(2, B, Hkv, L, d)


def _cache_shapes(bits, B, Hkv, L, d):
    T = (L + TILE - 1) // TILE
    per_byte = 8 // bits
    return dict(kq=(B, Hkv, L, d // per_byte), kp=(B, Hkv, L),
                vq=(B, Hkv, T, d, TILE // per_byte), vp=(B, Hkv, T, d))


def _check_cache(bits, cache, B, Hkv, L, d):
    import torch
    shp = _cache_shapes(bits, B, Hkv, L, d)
    for name, dt in (("kq", torch.uint8), ("kp", torch.int32), ("vq", torch.uint8),
                     ("vp", torch.int32)):
        _check(cache[name], name, dt, shp[name])


def _quantize(bits, k, v, cache, stream, key_range):
    import torch
    B, Hkv, L, d = k.shape
    _check(k, "k", torch.bfloat16, (B, Hkv, L, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, L, d))
    _check_cache(bits, cache, B, Hkv, L, d)
    k0, k1 = (0, L) if key_range is None else key_range
    fn = getattr(load(), f"attn_kv_quantize_q{bits}_range")
    rc = fn(_ptr(k), _ptr(v), _ptr(cache["kq"]), _ptr(cache["kp"]), _ptr(cache["vq"]),
            _ptr(cache["vp"]), B, Hkv, L, d, int(k0), int(k1), _stream(stream))
    _raise(rc)


def _decode_cache(bits, q, cache, L, o, lse, tau, workspace, skip_mask, stream, sas=0):
    import torch
    B, Hq, d = q.shape
    Hkv, cap = cache["kp"].shape[1], cache["kp"].shape[2]   # arrays sized for cap keys
    _check(q, "q", torch.bfloat16, (B, Hq, d))
    _check_cache(bits, cache, B, Hkv, cap, d)
    _check(o, "o", torch.float32, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, (L + TILE - 1) // TILE))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    ptrs = [_ptr(q), _ptr(cache["kq"]), _ptr(cache["kp"]), _ptr(cache["vq"]),
            _ptr(cache["vp"]), _ptr(o), _ptr(lse)]
    tail = [_ptr(skip_mask), _ptr(workspace), nbytes, _stream(stream)]
    so = load()
    if L != cap:
        rc = getattr(so, f"attn_decode_q{bits}_cap")(*ptrs, B, Hq, Hkv, int(L), cap, d,
                                                      float(tau), int(sas), *tail)
    elif sas:
        rc = getattr(so, f"attn_decode_q{bits}_sas")(*ptrs, B, Hq, Hkv, int(L), d, float(tau),
                                                      int(sas), *tail)
    else:
        rc = getattr(so, f"attn_decode_q{bits}")(*ptrs, B, Hq, Hkv, int(L), d, float(tau), *tail)
    _raise(rc)


def attn_kv_quantize_q4(k, v, cache, stream=None, key_range=None) -> None:
    """Enqueue the 4-bit quantiser: k/v [B,Hkv,L,d] bf16 -> cache dict of
    kq uint8, kp int32 (parameter words), vq uint8, vp int32 tensors with the
    shapes of q4_shapes(). ``key_range=(k0, k1)`` writes only those keys
    (k0 a multiple of 64), e.g. a chunk appended after a chunked prefill."""
    _quantize(4, k, v, cache, stream, key_range)


def attn_kv_quantize_q2(k, v, cache, stream=None, key_range=None) -> None:
    """The 2-bit quantiser; arguments as attn_kv_quantize_q4, shapes of q2_shapes()."""
    _quantize(2, k, v, cache, stream, key_range)


def attn_decode_q4(q, cache, L: int, o, lse, tau: float, workspace, skip_mask=None,
                   stream=None) -> None:
    """Enqueue split-K decode over a 4-bit cache (dict as for
    attn_kv_quantize_q4) of the first L keys; arrays sized for more keys
    than L (an appended cache) go through attn_decode_q4_cap. Other
    arguments as attn_decode."""
    _decode_cache(4, q, cache, L, o, lse, tau, workspace, skip_mask, stream)


def attn_decode_q2(q, cache, L: int, o, lse, tau: float, workspace, skip_mask=None,
                   stream=None) -> None:
    """Split-K decode over a 2-bit cache; arguments as attn_decode_q4."""
    _decode_cache(2, q, cache, L, o, lse, tau, workspace, skip_mask, stream)


def _bits_arg(bits):
    bits = tuple(int(b) for b in bits)
    return bits, (ctypes.c_uint8 * max(1, len(bits)))(*bits)


def _hybrid_ptrs(cache):
    out = []
    for w in ("q4", "q2"):
        c = cache[w]
        out += [None] * 4 if c is None else [_ptr(c["kq"]), _ptr(c["kp"]), _ptr(c["vq"]),
                                             _ptr(c["vp"])]
    return out


def hybrid_shapes(kv_bits, B: int, L: int, d: int) -> dict:
    """Shapes of a hybrid cache's two sub-caches: {"q4": shapes or None,
    "q2": shapes or None}; KV head g is stored at kv_bits[g] (4 or 2) bits,
    each width's heads in increasing order."""
    n4 = sum(1 for b in kv_bits if b == 4)
    n2 = sum(1 for b in kv_bits if b == 2)
    return {"q4": _cache_shapes(4, B, n4, L, d) if n4 else None,
            "q2": _cache_shapes(2, B, n2, L, d) if n2 else None}


def _check_hybrid(cache, B, Hkv, L, d):
    bits = tuple(cache["bits"])
    if len(bits) != Hkv:
        raise ValueError(f"kv_bits has {len(bits)} entries for {Hkv} KV heads")
    n = {4: sum(1 for b in bits if b == 4), 2: sum(1 for b in bits if b == 2)}
    for w, key in ((4, "q4"), (2, "q2")):
        if n[w]:
            _check_cache(w, cache[key], B, n[w], L, d)
        elif cache[key] is not None:
            raise ValueError(f"no head is stored at {w} bits but cache['{key}'] is given")


def attn_kv_quantize_hybrid(k, v, cache, stream=None, key_range=None) -> None:
    """Enqueue the hybrid quantiser: k/v [B,Hkv,L,d] bf16 -> cache dict
    {"bits": per-KV-head widths (4 or 2), "q4": 4-bit cache dict of the
    4-bit heads or None, "q2": likewise} (shapes of hybrid_shapes());
    ``key_range`` as for attn_kv_quantize_q4."""
    import torch
    B, Hkv, L, d = k.shape
    _check(k, "k", torch.bfloat16, (B, Hkv, L, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, L, d))
    _check_hybrid(cache, B, Hkv, L, d)
    _, arr = _bits_arg(cache["bits"])
    k0, k1 = (0, L) if key_range is None else key_range
    rc = load().attn_kv_quantize_hybrid_range(_ptr(k), _ptr(v), arr, *_hybrid_ptrs(cache), B, Hkv,
                                              L, d, int(k0), int(k1), _stream(stream))
    _raise(rc)


def attn_decode_hybrid(q, cache, L: int, o, lse, tau: float, workspace, skip_mask=None,
                       stream=None, sas: int = 0) -> None:
    """Enqueue split-K decode over a hybrid cache (dict as for
    attn_kv_quantize_hybrid) of the first L keys; the sub-caches may be sized
    for more keys. Other arguments as attn_decode; ``sas`` as for
    decode_q4."""
    import torch
    B, Hq, d = q.shape
    sub = cache["q4"] if cache["q4"] is not None else cache["q2"]
    cap = sub["kp"].shape[2]
    Hkv = len(cache["bits"])
    _check(q, "q", torch.bfloat16, (B, Hq, d))
    _check_hybrid(cache, B, Hkv, cap, d)
    _check(o, "o", torch.float32, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, (L + TILE - 1) // TILE))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _, arr = _bits_arg(cache["bits"])
    so = load()
    head = [_ptr(q), arr] + _hybrid_ptrs(cache) + [_ptr(o), _ptr(lse)]
    tail = [_ptr(skip_mask), _ptr(workspace), nbytes, _stream(stream)]
    if L != cap or sas:
        rc = so.attn_decode_hybrid_cap(*head, B, Hq, Hkv, int(L), cap, d, float(tau), int(sas),
                                       *tail)
    else:
        rc = so.attn_decode_hybrid(*head, B, Hq, Hkv, int(L), d, float(tau), *tail)
    _raise(rc)


# ---- allocation conveniences around the entry points ----

def _empty_cache(bits, B, Hkv, L, d, device):
    import torch
    shp = _cache_shapes(bits, B, Hkv, L, d)
    return {n: torch.empty(shp[n], dtype=torch.uint8 if n in ("kq", "vq") else torch.int32,
                           device=device) for n in shp}


def empty_q4(B: int, Hkv: int, L: int, d: int, device) -> dict:
    """Allocate (uninitialised) 4-bit cache arrays for L keys."""
    return _empty_cache(4, B, Hkv, L, d, device)


def empty_q2(B: int, Hkv: int, L: int, d: int, device) -> dict:
    """Allocate (uninitialised) 2-bit cache arrays for L keys."""
    return _empty_cache(2, B, Hkv, L, d, device)


def quantize_q4(k, v, stream=None) -> dict:
    """Allocate a 4-bit cache with torch and fill it from bf16 k, v."""
    B, Hkv, L, d = k.shape
    cache = empty_q4(B, Hkv, L, d, k.device)
    attn_kv_quantize_q4(k, v, cache, stream)
    return cache


def quantize_q2(k, v, stream=None) -> dict:
    """Allocate a 2-bit cache with torch and fill it from bf16 k, v."""
    B, Hkv, L, d = k.shape
    cache = empty_q2(B, Hkv, L, d, k.device)
    attn_kv_quantize_q2(k, v, cache, stream)
    return cache


def empty_hybrid(kv_bits, B: int, L: int, d: int, device) -> dict:
    """Allocate (uninitialised) hybrid cache arrays for L keys."""
    bits = tuple(int(b) for b in kv_bits)
    n4 = sum(1 for b in bits if b == 4)
    n2 = sum(1 for b in bits if b == 2)
    return {"bits": bits,
            "q4": _empty_cache(4, B, n4, L, d, device) if n4 else None,
            "q2": _empty_cache(2, B, n2, L, d, device) if n2 else None}


def quantize_hybrid(k, v, kv_bits, stream=None) -> dict:
    """Allocate a hybrid cache with torch (KV head g at kv_bits[g] bits) and
    fill it from bf16 k, v."""
    B, Hkv, L, d = k.shape
    cache = empty_hybrid(kv_bits, B, L, d, k.device)
    attn_kv_quantize_hybrid(k, v, cache, stream)
    return cache


def _decode_alloc(bits, q, cache, L, tau, want_mask, workspace, stream, sas=0):
    import torch
    B, Hq, d = q.shape
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        mask = torch.empty((B, Hq, (L + TILE - 1) // TILE), dtype=torch.uint8,
                           device=q.device)
    if workspace is None:
        nbytes = max(16, attn_decode_workspace_bytes(B, Hq, L, d))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if bits == "hybrid":
        attn_decode_hybrid(q, cache, L, o, lse, tau, workspace, mask, stream, sas)
    else:
        _decode_cache(bits, q, cache, L, o, lse, tau, workspace, mask, stream, sas)
    return o, lse, mask


def decode_q4(q, cache, L: int, tau: float = math.inf, want_mask: bool = False,
              workspace=None, stream=None, sas: int = 0):
    """Allocate outputs (and the workspace if not given) and call
    attn_decode_q4 (attn_decode_q4_sas of degree ``sas`` if nonzero).
    Returns (o, lse, mask)."""
    return _decode_alloc(4, q, cache, L, tau, want_mask, workspace, stream, sas)


def decode_q2(q, cache, L: int, tau: float = math.inf, want_mask: bool = False,
              workspace=None, stream=None, sas: int = 0):
    """As decode_q4, over a 2-bit cache."""
    return _decode_alloc(2, q, cache, L, tau, want_mask, workspace, stream, sas)


def decode_hybrid(q, cache, L: int, tau: float = math.inf, want_mask: bool = False,
                  workspace=None, stream=None, sas: int = 0):
    """As decode_q4, over a hybrid cache (dict of quantize_hybrid)."""
    return _decode_alloc("hybrid", q, cache, L, tau, want_mask, workspace, stream, sas)


# ---- allocation conveniences around the two bf16 entry points ----

def prefill(q, k, v, causal: bool, tau: float = math.inf, want_mask: bool = False,
            stream=None, sas: int = 0):
    """Allocate outputs with torch and call attn_prefill (attn_prefill_sas of
    polynomial degree ``sas`` if nonzero). Returns (o, lse, mask)."""
    import torch
    B, Hq, N, d = q.shape
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        nt = (N + TILE - 1) // TILE
        mask = torch.empty((B, Hq, nt, nt), dtype=torch.uint8, device=q.device)
    if sas:
        attn_prefill_sas(q, k, v, o, lse, causal, tau, sas, mask, stream)
    else:
        attn_prefill(q, k, v, o, lse, causal, tau, mask, stream)
    return o, lse, mask


def prefill_qk8(q, k, v, causal: bool, tau: float = math.inf, want_mask: bool = False,
                workspace=None, stream=None, int8: bool = False):
    """Allocate outputs (and the workspace if not given) and call
    attn_prefill_qk8 (``int8``: attn_prefill_qki8). Returns (o, lse, mask,
    workspace)."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        nt = (N + TILE - 1) // TILE
        mask = torch.empty((B, Hq, nt, nt), dtype=torch.uint8, device=q.device)
    if workspace is None:
        nbytes = max(256, attn_prefill_qk8_workspace_bytes(B, Hq, Hkv, N, d))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    attn_prefill_qk8(q, k, v, o, lse, causal, tau, workspace, mask, stream, int8=int8)
    return o, lse, mask, workspace


def prefill_pv8(q, k, v, causal: bool, tau: float = math.inf, qk8: bool = False,
                want_mask: bool = False, workspace=None, stream=None):
    """Allocate outputs (and the workspace if not given) and call
    attn_prefill_pv8. Returns (o, lse, mask, workspace)."""
    import torch
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        nt = (N + TILE - 1) // TILE
        mask = torch.empty((B, Hq, nt, nt), dtype=torch.uint8, device=q.device)
    if workspace is None:
        nbytes = max(256, attn_prefill_pv8_workspace_bytes(B, Hq, Hkv, N, d, qk8))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    attn_prefill_pv8(q, k, v, o, lse, causal, tau, workspace, qk8, mask, stream)
    return o, lse, mask, workspace


def prefill_chunk(q, k, v, causal: bool, tau: float = math.inf, want_mask: bool = False,
                  stream=None, N=None):
    """Allocate outputs with torch and call attn_prefill_chunk (k/v may be a
    cache allocated for more than the N keys that exist). Returns (o, lse, mask)."""
    import torch
    B, Hq, Nq, d = q.shape
    N = k.shape[2] if N is None else int(N)
    o = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        mask = torch.empty((B, Hq, (Nq + TILE - 1) // TILE, (N + TILE - 1) // TILE),
                           dtype=torch.uint8, device=q.device)
    attn_prefill_chunk(q, k, v, o, lse, causal, tau, mask, stream, N=N)
    return o, lse, mask


def decode(q, k, v, tau: float = math.inf, want_mask: bool = False, workspace=None,
           stream=None, sas: int = 0, L=None):
    """Allocate outputs (and the workspace if not given) and call attn_decode
    (attn_decode_sas with polynomial degree ``sas`` if nonzero; over the
    first ``L`` keys of a larger cache, attn_decode_cap). Returns
    (o, lse, mask)."""
    import torch
    B, Hq, d = q.shape
    L = k.shape[2] if L is None else int(L)
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        mask = torch.empty((B, Hq, (L + TILE - 1) // TILE), dtype=torch.uint8,
                           device=q.device)
    if workspace is None:
        nbytes = max(16, attn_decode_workspace_bytes(B, Hq, L, d))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    attn_decode_sas(q, k, v, o, lse, tau, sas, workspace, mask, stream, L=L)
    return o, lse, mask
