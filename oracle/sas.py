"""Oracle for decode and prefill attention with the Sparse Activated
SoftMax (SAS) exponential in place of exp.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What the pages fix (TurboAttention talk page, "Technical Deep Dive", the
Sparse Activated SoftMax part, and "Key Results & Evaluation"): softmax's
exp(-X), X >= 0, is split into the integer part and the fractional part of
X; exp(-integer part) comes from a small precomputed table (six entries were
enough in their evaluation, larger integer parts giving negligible outputs),
and exp(-fractional part) from a low-degree polynomial (degree two "near
lossless", degree three "almost lossless").

Readings, where the pages are silent:

* Table: T[n] = e^-n for n = 0 .. 5; an integer part of 6 or more gives 0
  (the "sparse" outputs).
* Polynomial: the least-squares fit of e^-f on [0, 1] (continuous L2 norm)
  of degree 2 or 3. The pages give no coefficients; this is the plainest
  fit of that degree. SAS(X) = T[floor X] * p(X - floor X).
* Where it applies: every exponential of the online softmax, i.e. the
  probabilities p_j = SAS(m - s_j) and the rescale factor SAS(m_new - m_old)
  when a kept tile raises a row's running maximum m (scores s in
  natural-logit units, s = q.k / sqrt(d)). Decode: inside each split of the
  split-K decode; each split then yields O_s = acc / l and lse_s = m + ln l,
  and splits are merged exactly by log-sum-exp, as in the exact decode.
  Prefill: per query row over the kept tiles of its 64-row block, O = acc / l
  and lse = m + ln l. Because SAS(a) SAS(b) != SAS(a + b), the result
  depends on the order in which the running maximum rises, so this oracle
  follows the tiles in ascending order as the rule does, and m is the true
  running maximum (no deferred rescale).
* The skip decisions are those of the exact rule (SAS changes only the
  exponentials, not the scores or the maxima).

Parity unpinned: the table size, the fit and the places where SAS applies
are readings, not values the pages print. The tests pin the functions:
the fit's residual is orthogonal to 1, f, .., f^deg under numerical
quadrature; the table values and the cut at 6; the error bounds; with exact
exponentials the online loops reproduce the exact decode and prefill
oracles; with a single kept tile (no rescale) they equal the direct formula;
a hand-derived two-tile case, whose running maximum rises by 2.25 logits,
fixes SAS on the rescale factor as well as on the probabilities; and with
no tile skipped each prefill row equals the SAS decode of that row.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import KEPT, SPLIT, TILE, decode_head as exact_decode_head
from .attention import prefill_blocks as exact_prefill_blocks

TABLE_SIZE = 6


def poly_coeffs(degree: int) -> np.ndarray:
    """Least-squares coefficients a_0 .. a_deg of e^-f on [0, 1] (fp64).

    Normal equations: sum_j a_j / (i + j + 1) = int_0^1 f^i e^-f df, the
    moments by integration by parts: m_0 = 1 - 1/e, m_i = i m_(i-1) - 1/e.
    """
    if degree not in (2, 3):
        raise ValueError("SAS polynomial degree must be 2 or 3")
    n = degree + 1
    gram = np.array([[1.0 / (i + j + 1) for j in range(n)] for i in range(n)])
    mom = np.empty(n)
    mom[0] = 1.0 - math.exp(-1.0)
    for i in range(1, n):
        mom[i] = i * mom[i - 1] - math.exp(-1.0)
    return np.linalg.solve(gram, mom)


def table() -> np.ndarray:
    """T[n] = e^-n for n = 0 .. TABLE_SIZE - 1."""
    return np.exp(-np.arange(TABLE_SIZE, dtype=np.float64))


def sas_exp(x, degree: int) -> np.ndarray:
    """SAS approximation of e^-x for x >= 0 (+inf allowed), elementwise."""
    x = np.asarray(x, np.float64)
    if np.any(x < 0):
        raise ValueError("SAS takes x >= 0")
    a = poly_coeffs(degree)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    n = np.floor(xf)
    f = xf - n
    p = np.zeros_like(xf)
    for c in a[::-1]:
        p = p * f + c
    idx = np.minimum(n, TABLE_SIZE - 1).astype(np.int64)
    t = np.where(n < TABLE_SIZE, table()[idx], 0.0)
    return np.where(finite, t * p, 0.0)


def _boundary_jump(degree: int, k: int) -> float:
    """|SAS(k-) - SAS(k+)| at integer k >= 1 (the step between table rows)."""
    a = poly_coeffs(degree)
    below = math.exp(-(k - 1)) * float(np.polyval(a[::-1], 1.0))
    above = math.exp(-k) * float(a[0]) if k < TABLE_SIZE else 0.0
    return abs(below - above)


def decode_head(qvec: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float, degree: int,
                split: int = SPLIT, forced: np.ndarray | None = None, exp_fn=None,
                near: float = 1e-3):
    """SAS decode for one query token against one KV head.

    qvec (d,), k/v (L, d) fp64. Returns o (d,), lse, decisions (nt,),
    margins (nt,) and slack = (lse_slack, o_slack): bounds on how far the
    result may move if arguments within ``near`` of an integer (where SAS
    steps) round to the other side, for comparisons with a float32 kernel.
    ``exp_fn(x)`` replaces the SAS exponential (e.g. exact e^-x, to check the
    online loop against the exact oracle).
    """
    if exp_fn is None:
        def exp_fn(x):
            return sas_exp(x, degree)
    _, _, dec, margin = exact_decode_head(qvec, k, v, tau, split, forced)
    L, d = k.shape
    s = (k @ qvec) / math.sqrt(d)
    per = split // TILE
    nt = dec.shape[0]
    vmax = float(np.abs(v).max()) if v.size else 0.0
    parts = []
    lse_slack = 0.0
    o_slack = 0.0
    for t0 in range(0, nt, per):
        m = -math.inf
        acc = np.zeros(d)
        l = 0.0
        jump_abs = 0.0   # possible absolute change of l from rounding at steps
        jump_o = 0.0     # the same, weighted by 2 max |v_j| of the key
        jump_rel = 0.0   # possible relative change of everything accumulated
        for t in range(t0, min(nt, t0 + per)):
            if dec[t] != KEPT:
                continue
            st = s[TILE * t:min(L, TILE * (t + 1))]
            mn = max(m, float(st.max()))
            if mn > m:
                if math.isfinite(m):
                    xa = mn - m
                    alpha = float(exp_fn(np.array([xa]))[0])
                    jump_rel += _near_jump_rel(degree, xa, near)
                else:
                    alpha = 0.0
                acc *= alpha
                l *= alpha
                jump_abs *= alpha
                jump_o *= alpha
                m = mn
            x = m - st
            p = exp_fn(x)
            acc += p @ v[TILE * t:TILE * t + st.shape[0]]
            l += float(p.sum())
            steps = _near_jumps(degree, x, near)
            jump_abs += float(steps.sum())
            jump_o += float(steps @ (2.0 * np.abs(v[TILE * t:TILE * t + st.shape[0]]).max(axis=1)))
        if l > 0.0:
            parts.append((acc / l, m + math.log(l)))
            lse_slack = max(lse_slack, jump_abs / l + jump_rel)
            o_slack = max(o_slack, jump_o / l + 2.0 * jump_rel * vmax)
    if not parts:
        return np.full(d, np.nan), -math.inf, dec, margin, (lse_slack, o_slack)
    lses = np.array([p[1] for p in parts])
    top = lses.max()
    w = np.exp(lses - top)
    lse = top + math.log(w.sum())
    o = sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()
    return o, lse, dec, margin, (lse_slack, o_slack)


def _near_jumps(degree, x, near):
    """Per entry of x: the step of SAS at an integer within ``near`` of it, else 0."""
    x = np.asarray(x, np.float64)
    xf = np.where(np.isfinite(x), x, -1.0)
    k = np.rint(xf)
    hit = (k >= 1) & (k <= TABLE_SIZE) & (np.abs(xf - k) < near)
    out = np.zeros(x.shape)
    for i in np.nonzero(hit)[0]:
        out[i] = _boundary_jump(degree, int(k[i]))
    return out


def _near_jump_rel(degree, x, near):
    if not math.isfinite(x):
        return 0.0
    k = round(x)
    if k < 1 or k > TABLE_SIZE or abs(x - k) >= near:
        return 0.0
    below = math.exp(-(k - 1)) * float(np.polyval(poly_coeffs(degree)[::-1], 1.0))
    return _boundary_jump(degree, k) / below


def _near_steps(degree, x, near):
    """Elementwise over any shape: the step of SAS at an integer k in 1..6
    within ``near`` of x (0 elsewhere), absolute and relative to the value
    just below the step."""
    x = np.asarray(x, np.float64)
    xf = np.where(np.isfinite(x), x, -1.0)
    k = np.rint(xf)
    hit = (k >= 1) & (k <= TABLE_SIZE) & (np.abs(xf - k) < near)
    jump = np.array([0.0] + [_boundary_jump(degree, j) for j in range(1, TABLE_SIZE + 1)])
    top = float(np.polyval(poly_coeffs(degree)[::-1], 1.0))
    below = np.array([1.0] + [math.exp(-(j - 1)) * top for j in range(1, TABLE_SIZE + 1)])
    ki = np.clip(k, 0, TABLE_SIZE).astype(np.int64)
    return np.where(hit, jump[ki], 0.0), np.where(hit, jump[ki] / below[ki], 0.0)


def prefill_blocks(qrows: np.ndarray, k: np.ndarray, v: np.ndarray, qb0: int, causal: bool,
                   tau: float, degree: int, forced: np.ndarray | None = None, exp_fn=None,
                   near: float = 1e-3):
    """SAS prefill for consecutive 64-row query blocks of one (batch, head).

    qrows (R, d) rows qb0*64 ..; k, v (N, d) fp64. The skip decisions are the
    exact rule's. Returns o (R, d), lse (R,), decisions (nb, nt), margins
    (nb, nt) and slack (R, 2): per row, bounds on how far lse and o may move
    if SAS arguments within ``near`` of an integer round to the other side.
    ``exp_fn(x)`` replaces the SAS exponential.
    """
    if exp_fn is None:
        def exp_fn(x):
            return sas_exp(x, degree)
    _, _, dec, margin = exact_prefill_blocks(qrows, k, v, qb0, causal, tau, forced)
    R, d = qrows.shape
    N = k.shape[0]
    nt = (N + TILE - 1) // TILE
    rows = qb0 * TILE + np.arange(R)
    s = (qrows @ k.T) / math.sqrt(d)
    if causal:
        s = np.where(np.arange(N)[None, :] <= rows[:, None], s, -np.inf)
    vmax = float(np.abs(v).max()) if v.size else 0.0
    vkey = 2.0 * np.abs(v).max(axis=1) if v.size else np.zeros(N)
    o = np.empty((R, d))
    lse = np.empty(R)
    slack = np.zeros((R, 2))
    for bi in range(dec.shape[0]):
        r0, r1 = bi * TILE, min(R, (bi + 1) * TILE)
        n = r1 - r0
        m = np.full(n, -np.inf)
        acc = np.zeros((n, d))
        l = np.zeros(n)
        j_abs = np.zeros(n)   # possible absolute change of l at SAS steps
        j_o = np.zeros(n)     # the same weighted by 2 max |v| of the key
        j_rel = np.zeros(n)   # possible relative change of all accumulated so far
        for t in range(nt):
            if dec[bi, t] != KEPT:
                continue
            k0, k1 = t * TILE, min(N, (t + 1) * TILE)
            st = s[r0:r1, k0:k1]
            mn = np.maximum(m, st.max(axis=1))
            grow = mn > m
            first = grow & ~np.isfinite(m)
            rise = grow & np.isfinite(m)
            xa = np.where(rise, mn - np.where(np.isfinite(m), m, 0.0), 0.0)
            alpha = np.where(rise, exp_fn(xa), np.where(first, 0.0, 1.0))
            _, rel = _near_steps(degree, np.where(rise, xa, -1.0), near)
            acc *= alpha[:, None]
            l *= alpha
            j_abs *= alpha
            j_o *= alpha
            j_rel += rel
            m = mn
            fin = np.isfinite(m)
            x = np.where(fin[:, None], np.where(fin, m, 0.0)[:, None] - st, np.inf)
            p = exp_fn(x)
            acc += p @ v[k0:k1]
            l += p.sum(axis=1)
            step, _ = _near_steps(degree, x, near)
            j_abs += step.sum(axis=1)
            j_o += step @ vkey[k0:k1]
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
        slack[r0:r1, 0] = j_abs / l + j_rel
        slack[r0:r1, 1] = j_o / l + 2.0 * j_rel * vmax
    return o, lse, dec, margin, slack


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, tau: float, degree: int,
            forced: np.ndarray | None = None, exp_fn=None):
    """Full SAS prefill. q (B,Hq,N,d), k/v (B,Hkv,N,d) fp64; query head h
    reads KV head h // (Hq // Hkv). Returns dict o, lse, mask, margin, slack
    (B,Hq,N,2)."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    nt = (N + TILE - 1) // TILE
    out = dict(o=np.empty((B, Hq, N, d)), lse=np.empty((B, Hq, N)),
               mask=np.empty((B, Hq, nt, nt), np.uint8), margin=np.empty((B, Hq, nt, nt)),
               slack=np.empty((B, Hq, N, 2)))
    for b in range(B):
        for h in range(Hq):
            fc = None if forced is None else forced[b, h]
            o, lse, dec, margin, sl = prefill_blocks(q[b, h], k[b, h // G], v[b, h // G], 0,
                                                     causal, tau, degree, fc, exp_fn)
            out["o"][b, h], out["lse"][b, h] = o, lse
            out["mask"][b, h], out["margin"][b, h], out["slack"][b, h] = dec, margin, sl
    return out
