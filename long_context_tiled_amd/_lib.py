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
           "attn_decode_q2_check", "attn_decode_sas", "attn_decode_q4_sas",
           "attn_decode_q2_sas")

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
    lib.attn_prefill_chunk_check.restype = i
    lib.attn_decode.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp, sz, vp]
    lib.attn_decode.restype = i
    lib.attn_decode_sas.argtypes = [vp, vp, vp, f32p, f32p, i, i, i, i, i, f, i, u8p, vp, sz, vp]
    lib.attn_decode_sas.restype = i
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
        fn = getattr(lib, f"attn_decode_{w}_check")
        fn.argtypes = [vp, vp, vp, vp, vp, f32p, f32p, i, i, i, i, i, f, u8p, vp, sz]
        fn.restype = i
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


def attn_prefill_chunk(q, k, v, o, lse, causal: bool, tau: float, skip_mask=None,
                       stream=None) -> None:
    """Enqueue chunked prefill: q [B,Hq,Nq,d] are the last Nq of the N
    positions of k/v [B,Hkv,N,d]; writes o [B,Hq,Nq,d], lse [B,Hq,Nq] and, if
    given, skip_mask [B,Hq,ceil(Nq/64),ceil(N/64)]."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    _check(q, "q", torch.bfloat16, (B, Hq, Nq, d))
    _check(k, "k", torch.bfloat16, (B, Hkv, N, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, N, d))
    _check(o, "o", torch.float32, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8,
               (B, Hq, (Nq + TILE - 1) // TILE, (N + TILE - 1) // TILE))
    rc = load().attn_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                   Nq, N, d, int(bool(causal)), float(tau), _ptr(skip_mask),
                                   _stream(stream))
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
                    stream=None) -> None:
    """attn_decode with the SAS exponential of polynomial degree 2 or 3
    (0: exact exponentials, i.e. attn_decode)."""
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
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    rc = load().attn_decode_sas(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                L, d, float(tau), int(degree), _ptr(skip_mask),
                                _ptr(workspace), nbytes, _stream(stream))
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
    Hkv = cache["kp"].shape[1]
    _check(q, "q", torch.bfloat16, (B, Hq, d))
    _check_cache(bits, cache, B, Hkv, L, d)
    _check(o, "o", torch.float32, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if skip_mask is not None:
        _check(skip_mask, "skip_mask", torch.uint8, (B, Hq, (L + TILE - 1) // TILE))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    args = [_ptr(q), _ptr(cache["kq"]), _ptr(cache["kp"]), _ptr(cache["vq"]),
            _ptr(cache["vp"]), _ptr(o), _ptr(lse), B, Hq, Hkv, L, d, float(tau)]
    tail = [_ptr(skip_mask), _ptr(workspace), nbytes, _stream(stream)]
    if sas:
        rc = getattr(load(), f"attn_decode_q{bits}_sas")(*args, int(sas), *tail)
    else:
        rc = getattr(load(), f"attn_decode_q{bits}")(*args, *tail)
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
    attn_kv_quantize_q4, holding L keys); other arguments as attn_decode."""
    _decode_cache(4, q, cache, L, o, lse, tau, workspace, skip_mask, stream)


def attn_decode_q2(q, cache, L: int, o, lse, tau: float, workspace, skip_mask=None,
                   stream=None) -> None:
    """Split-K decode over a 2-bit cache; arguments as attn_decode_q4."""
    _decode_cache(2, q, cache, L, o, lse, tau, workspace, skip_mask, stream)


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


# ---- allocation conveniences around the two bf16 entry points ----

def prefill(q, k, v, causal: bool, tau: float = math.inf, want_mask: bool = False,
            stream=None):
    """Allocate outputs with torch and call attn_prefill. Returns (o, lse, mask)."""
    import torch
    B, Hq, N, d = q.shape
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        nt = (N + TILE - 1) // TILE
        mask = torch.empty((B, Hq, nt, nt), dtype=torch.uint8, device=q.device)
    attn_prefill(q, k, v, o, lse, causal, tau, mask, stream)
    return o, lse, mask


def prefill_chunk(q, k, v, causal: bool, tau: float = math.inf, want_mask: bool = False,
                  stream=None):
    """Allocate outputs with torch and call attn_prefill_chunk. Returns (o, lse, mask)."""
    import torch
    B, Hq, Nq, d = q.shape
    N = k.shape[2]
    o = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        mask = torch.empty((B, Hq, (Nq + TILE - 1) // TILE, (N + TILE - 1) // TILE),
                           dtype=torch.uint8, device=q.device)
    attn_prefill_chunk(q, k, v, o, lse, causal, tau, mask, stream)
    return o, lse, mask


def decode(q, k, v, tau: float = math.inf, want_mask: bool = False, workspace=None,
           stream=None, sas: int = 0):
    """Allocate outputs (and the workspace if not given) and call attn_decode
    (attn_decode_sas with polynomial degree ``sas`` if nonzero). Returns
    (o, lse, mask)."""
    import torch
    B, Hq, d = q.shape
    L = k.shape[2]
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    mask = None
    if want_mask:
        mask = torch.empty((B, Hq, (L + TILE - 1) // TILE), dtype=torch.uint8,
                           device=q.device)
    if workspace is None:
        nbytes = max(16, attn_decode_workspace_bytes(B, Hq, L, d))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    attn_decode_sas(q, k, v, o, lse, tau, sas, workspace, mask, stream)
    return o, lse, mask
