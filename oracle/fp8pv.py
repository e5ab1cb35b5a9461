"""Oracle for prefill attention with an 8-bit P.V product.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive" and "Key
Findings"; its pre-fill workflow): both matrix products of blockwise
attention, QK^T and PV, run on 8-bit operands quantised block-wise inside the
blocks of the flash computation; the softmax statistics stay in higher
precision. ``fp8`` holds the QK^T half (E4M3 Q and K per 64-row tile). This
module is the PV half. Readings, where the pages are silent:

* V: E4M3 codes with one fp32 scale per (sequence, KV head):
  s_V = (largest |v| of the head) / 448, 1 for a head of zeros; codes of
  v / s_V rounded as in ``fp8``. A scale per key tile would not factor out of
  P.V's sum over the tiles, which one accumulator carries across the whole
  key loop; E4M3 keeps its 3-bit relative precision for 15 binades below the
  scale, so one scale per head costs little next to one per tile.
* P: each probability is taken relative to a reference maximum m_ref of its
  row, p = exp(s - m_ref), and enters P.V as the nearest E4M3 value (ties to
  even; below 2^-10 it is 0), with no further scale. m_ref is the running
  maximum as of the last rescale: it is set at the first kept tile and moves
  (for every row whose running maximum has grown) only when some row of the
  64-row decision block has grown past its m_ref by more than 8 ln 2, so
  p <= 2^8 stays inside E4M3's range (448). Each move multiplies everything
  accumulated by exp(m_ref_old - m_ref_new).
* The row sum l is taken over the unrounded p (same reference and rescales);
  O = s_V (sum over kept tiles of E4M3(p) . codes) / l and
  LSE = m_ref + ln l.
* Skip decisions: the exact rule on the scores (those of the dequantised Q
  and K when QK^T is 8-bit too).
* Layout of the V codes for the kernel: per (sequence, KV head) and 64-key
  tile t, a block of d rows of 64 bytes; row c holds channel c's codes of
  the tile's keys in the order of the kernel's P.V contraction index j:
  j = 32 h + 16 a + 4 i + e holds key 32 a + 8 i + 4 h + e of the tile
  (h, a in {0, 1}; i, e in 0..3), and the row's 16-byte chunk x is stored at
  chunk x ^ ((c >> 2) & 3). Keys at or past N have code 0.

Parity unpinned: the per-head V scale, the unscaled E4M3 probabilities and
the reference-maximum rule are readings. The tests pin that the code does
what is stated: reduction to the exact oracle when nothing is rounded,
hand-derived outputs of a one-tile row, a two-tile row whose maximum rises
past and short of the rescale margin, the scale of a hand-built head and
hand-derived byte positions of the layout.
"""
from __future__ import annotations

import math

import numpy as np

from . import fp8
from .attention import KEPT, TILE, _block_scores, _decide

LAZY = 8.0 * math.log(2.0)   # the reference moves when a row grows past it by more


def quantize_v(v: np.ndarray):
    """V fp32 (..., N, d) holding bf16 values -> (codes uint8 (..., N, d),
    scale fp32 (...,)): one scale per head."""
    v = np.asarray(v, np.float32)
    codes, s = fp8.quantize(v, rows=v.shape[-2])
    return codes, s[..., 0]


def v_layout(codes: np.ndarray) -> np.ndarray:
    """One head's V codes (N, d) -> the kernel's tile blocks (T, d, 64)."""
    N, d = codes.shape
    T = (N + TILE - 1) // TILE
    j = np.arange(TILE)
    h, a, i, e = j >> 5, (j >> 4) & 1, (j >> 2) & 3, j & 3
    keys = np.arange(T)[:, None] * TILE + (32 * a + 8 * i + 4 * h + e)[None, :]   # (T, 64)
    padded = np.zeros((T * TILE + TILE, d), np.uint8)
    padded[:N] = codes
    blk = padded[np.minimum(keys, T * TILE)].transpose(0, 2, 1)    # (T, d, 64), by j
    blk = np.where((keys < N)[:, None, :], blk, 0).astype(np.uint8)
    # byte p of row c holds contraction index 16 ((p >> 4) ^ ((c >> 2) & 3)) + (p & 15)
    p = np.arange(TILE)
    sw = (np.arange(d) >> 2) & 3
    src = 16 * ((p[None, :] >> 4) ^ sw[:, None]) + (p[None, :] & 15)          # (d, 64)
    return np.take_along_axis(blk, np.broadcast_to(src, blk.shape), axis=2)


def e4m3_round(p: np.ndarray) -> np.ndarray:
    """Non-negative values <= 448 -> the nearest E4M3 values (fp64)."""
    return fp8.e4m3_value(fp8.e4m3_encode(p))


def _e4m3_spacing(p: np.ndarray) -> np.ndarray:
    """Spacing of the E4M3 values around p >= 0 (the subnormal step below 2^-6)."""
    a = np.where(p > 0, p, 1.0)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1.0, fp8.MIN_NORMAL_EXP)
    return np.exp2(e - 3.0)


def _near_midpoint(p: np.ndarray, rel: np.ndarray) -> np.ndarray:
    """True where p lies within rel * p of a point halfway between two E4M3
    values, so that a p off by that much may round to the other neighbour."""
    sp = _e4m3_spacing(p)
    f = p / sp - np.floor(p / sp)
    return (p > 0) & (np.abs(f - 0.5) * sp <= rel * p)


def pv8_blocks(qrows: np.ndarray, k: np.ndarray, vvals: np.ndarray, v_scale: float, qb0: int,
               causal: bool, tau: float, forced: np.ndarray | None = None,
               score_err: np.ndarray | float = 0.0, round_p=e4m3_round,
               lin_err: np.ndarray | float | None = None):
    """8-bit P.V prefill for consecutive 64-row query blocks of one (batch,
    head).

    qrows (R, d) rows qb0*64 ..; k (N, d) fp64 keys; vvals (N, d) the E4M3
    values of V's codes, v_scale their scale. ``score_err`` bounds, per
    score (R, N) or for all, how far a kernel's score may sit from this one
    (in logits); ``lin_err`` (default: score_err) is the error carried to
    first order into the slack of LSE and O (0 where the kernel's scores are
    as exact as the tolerances already assume). ``round_p`` rounds the
    probabilities (identity: no rounding).

    Returns o (R, d), lse (R,), decisions (nb, nt), margins (nb, nt), slack
    (R, 2) and amb (nb,) bool. slack bounds, to first order, how far LSE
    (slack[:, 0]) and O (slack[:, 1]) may move when every score is off by up
    to lin_err: the probability-weighted mean of lin_err for the LSE;
    for O that times 2 max |v|, plus the change of probabilities within
    score_err of an E4M3 rounding midpoint that round the other way. amb
    marks blocks where the rescale test came within score_err of its margin
    (the kernel's reference may then move at another tile).
    """
    R, d = qrows.shape
    N = k.shape[0]
    s, t, valid, visited = _block_scores(qrows, k, qb0, causal)
    dec, margin = _decide(t, valid, visited, tau, forced)
    nblk, nt = dec.shape
    err = np.broadcast_to(np.asarray(score_err, np.float64), s.shape)
    lerr = err if lin_err is None else np.broadcast_to(np.asarray(lin_err, np.float64), s.shape)
    vkey = np.abs(vvals).max(axis=1) if vvals.size else np.zeros(N)
    vmax = float(vkey.max()) if vkey.size else 0.0
    o = np.empty((R, d))
    lse = np.empty(R)
    slack = np.zeros((R, 2))
    amb = np.zeros(nblk, bool)
    for bi in range(nblk):
        r0, r1 = bi * TILE, min(R, (bi + 1) * TILE)
        n = r1 - r0
        m = np.full(n, -np.inf)
        mref = np.full(n, -np.inf)
        acc = np.zeros((n, d))
        l = np.zeros(n)
        jo = np.zeros(n)
        je = np.zeros(n)      # sum of p times the score error
        for tt in range(nt):
            if dec[bi, tt] != KEPT:
                continue
            k0, k1 = tt * TILE, min(N, (tt + 1) * TILE)
            st = s[r0:r1, k0:k1]
            et = err[r0:r1, k0:k1]
            m = np.maximum(m, st.max(axis=1))
            fin = np.isfinite(m)
            over = np.where(fin, m - np.where(np.isfinite(mref), mref, -np.inf) - LAZY, -np.inf)
            if np.any(fin & np.isfinite(over) & (np.abs(over) <= et.max(axis=1))):
                amb[bi] = True
            if np.any(over > 0):
                up = fin & (m > mref)
                alpha = np.where(up, np.exp(np.where(np.isfinite(mref), mref, 0.0) - m), 1.0)
                alpha = np.where(up & ~np.isfinite(mref), 0.0, alpha)
                acc *= alpha[:, None]
                l *= alpha
                jo *= alpha
                je *= alpha
                mref = np.where(up, m, mref)
            ok = np.isfinite(st) & np.isfinite(mref)[:, None]
            p = np.where(ok, np.exp(np.where(ok, st - mref[:, None], 0.0)), 0.0)
            acc += round_p(p) @ vvals[k0:k1]
            l += p.sum(axis=1)
            je += (p * lerr[r0:r1, k0:k1]).sum(axis=1)
            # a probability off by a factor exp(+-err) may round to a neighbour
            near = _near_midpoint(p, np.expm1(et))
            jo += (near * _e4m3_spacing(p)) @ vkey[k0:k1]
        o[r0:r1] = v_scale * acc / l[:, None]
        lse[r0:r1] = mref + np.log(l)
        slack[r0:r1, 0] = je / l
        slack[r0:r1, 1] = v_scale * (jo + 2.0 * vmax * je) / l
    return o, lse, dec, margin, slack, amb


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, tau: float,
            qk8: bool = False, forced: np.ndarray | None = None):
    """Full 8-bit P.V prefill. q (B,Hq,N,d), k/v (B,Hkv,N,d) fp32 holding
    bf16 values; query head h reads KV head h // (Hq // Hkv). ``qk8``: Q and
    K quantised as in ``fp8`` too. Returns dict o, lse, mask, margin, slack
    (B,Hq,N,2) and amb (B,Hq,nt)."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if qk8:
        qc, qs = fp8.quantize(q)
        kc, ks = fp8.quantize(k)
        qf, kf = fp8.dequantize(qc, qs), fp8.dequantize(kc, ks)
    else:
        qf, kf = np.asarray(q, np.float64), np.asarray(k, np.float64)
    vc, vs = quantize_v(v)
    vvals = fp8.e4m3_value(vc)
    nt = (N + TILE - 1) // TILE
    out = dict(o=np.empty((B, Hq, N, d)), lse=np.empty((B, Hq, N)),
               mask=np.empty((B, Hq, nt, nt), np.uint8), margin=np.empty((B, Hq, nt, nt)),
               slack=np.empty((B, Hq, N, 2)), amb=np.empty((B, Hq, nt), bool))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            fc = None if forced is None else forced[b, h]
            o, lse, dec, margin, sl, amb = pv8_blocks(qf[b, h], kf[b, g], vvals[b, g],
                                                      float(vs[b, g]), 0, causal, tau, fc)
            out["o"][b, h], out["lse"][b, h] = o, lse
            out["mask"][b, h], out["margin"][b, h] = dec, margin
            out["slack"][b, h], out["amb"][b, h] = sl, amb
    return out
