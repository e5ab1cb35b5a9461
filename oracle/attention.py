"""Plain fp64 CPU oracle for exact tiled softmax attention with Skip-Softmax.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg call it. It shares no code with the HIP library.

What it computes, and where the pages say so:

* Blockwise attention (TurboAttention talk page, "Technical Deep Dive": the
  Flash-Attention structure computes QK^T, softmax and PV block by block and
  never materialises the N x N matrix in GPU memory). Here the scores are
  formed in fp64 for the rows in hand; the tile structure only matters for
  the skip decisions.
* The Skip-Softmax rule (TensorRT-LLM Skip Softmax summary page, "Key Points"
  and "Detailed Analysis"): a key block whose local maximum score lies below
  the running maximum minus the threshold tau is skipped. Readings taken where
  that page is terse or garbled:
    - the running maximum ("MI - 1" in the extracted text) is m_i^(j-1), the
      row's maximum over the blocks kept before block j;
    - the test is per row, strict, and must hold for every valid row of the
      64-row decision block: skip <=> for all r, t_r < m_r - tau;
    - tau is in natural-logit units, s = q.k / sqrt(d); tau = +inf means
      dense attention; tau >= 0;
    - skipping removes the block's exp and PV work: it adds nothing to the
      numerator, to the normaliser or to the running maximum. The scores are
      still formed, since the test needs them;
    - blocks are visited in ascending key order; the first visited block
      (running max -inf) is never skipped.
* Decode (one query token per sequence): keys are cut into fixed splits of
  ``split`` keys (4096 by default); each split runs the same rule over its
  own 64-key tiles with its own running maximum, starting at -inf. The result
  is the softmax over the union of kept keys. Splitting and merging partial
  results by log-sum-exp is exact algebra, so it is not emulated here.

Outputs are O (softmax over the kept keys times V), LSE = ln(sum over kept
keys of e^s) in natural log, the per-tile decision (0 kept, 1 skipped,
2 not visited because the whole tile lies above the causal diagonal) and the
per-tile margin min_r (m_r - tau - t_r): the tile is skipped exactly when the
margin is positive.

``forced`` lets a caller impose decisions on chosen tiles (-1 free, 0 keep,
1 skip), so that a result computed with another rounding of the scores can be
re-evaluated under that caller's decisions.

Parity unpinned: the readings listed above (per-row test over every valid
row, natural-logit units with the 1/sqrt(d) scale, the strict comparison,
per-head decisions in decode, the split size) are conventions; the pages
print no numeric example of the rule, so no test can tie them to the pages.
The functions themselves are pinned outside their own code: a scalar
brute-force online softmax, the textbook softmax attention at tau = inf, the
prefix-max closed form of the decisions, the dropped-mass bound, hand-built
golden cases and the split/merge identity (the oracle tests).
"""
from __future__ import annotations

import math

import numpy as np

TILE = 64
SPLIT = 4096

KEPT, SKIPPED, NOT_VISITED = 0, 1, 2


def _scores(qrows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """s = q . k / sqrt(d) in fp64 for a block of query rows."""
    d = qrows.shape[-1]
    return (qrows @ k.T) / math.sqrt(d)


def _tile_max(s: np.ndarray, ntiles: int) -> np.ndarray:
    """Per-row maximum of each 64-key tile; pads a ragged last tile with -inf."""
    rows, n = s.shape
    pad = ntiles * TILE - n
    if pad:
        s = np.concatenate([s, np.full((rows, pad), -np.inf)], axis=1)
    return s.reshape(rows, ntiles, TILE).max(axis=2)


def _decide(t: np.ndarray, valid: np.ndarray, visited: np.ndarray, tau: float,
            forced: np.ndarray | None):
    """Run the skip rule over tiles in ascending order.

    t        (nb, R, nt) per-row tile maxima, nb independent decision blocks
    valid    (nb, R) rows that take part in the vote
    visited  (nb, nt) tiles each block visits
    tau      the threshold: a float, or an (nb, 1) array of one per block
    returns decisions (nb, nt) uint8 and margins (nb, nt) float64.
    """
    nb, R, nt = t.shape
    m = np.full((nb, R), -np.inf)
    dec = np.full((nb, nt), NOT_VISITED, np.uint8)
    margin = np.full((nb, nt), np.nan)
    for kb in range(nt):
        tk = t[:, :, kb]
        with np.errstate(invalid="ignore"):
            slack = (m - tau) - tk
        # a NaN slack (-inf minus -inf) means the strict comparison fails
        slack = np.where(np.isnan(slack), -np.inf, slack)
        slack = np.where(valid, slack, np.inf)
        mg = slack.min(axis=1)
        skip = mg > 0
        if forced is not None:
            fk = forced[:, kb]
            skip = np.where(fk >= 0, fk == 1, skip)
        vis = visited[:, kb]
        dec[vis, kb] = np.where(skip[vis], SKIPPED, KEPT)
        margin[vis, kb] = mg[vis]
        keep = vis & ~skip
        m = np.where(keep[:, None], np.maximum(m, tk), m)
    return dec, margin


def _softmax_kept(s: np.ndarray, kept: np.ndarray, v: np.ndarray):
    """Softmax over the kept entries of each row, then times V."""
    sk = np.where(kept, s, -np.inf)
    mx = sk.max(axis=1, keepdims=True)
    p = np.exp(sk - mx)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    lse = mx[:, 0] + np.log(l[:, 0])
    return o, lse


def _block_scores(qrows: np.ndarray, k: np.ndarray, qb0: int, causal: bool):
    """Scores of consecutive query rows qb0*64 ... (causal: -inf past the
    diagonal), the per-row tile maxima grouped into 64-row decision blocks,
    the rows that vote and the tiles each block visits."""
    R, d = qrows.shape
    N = k.shape[0]
    nt = (N + TILE - 1) // TILE
    nb = (R + TILE - 1) // TILE
    row0 = qb0 * TILE
    rows = row0 + np.arange(R)
    s = _scores(qrows, k)
    if causal:
        s = np.where(np.arange(N)[None, :] <= rows[:, None], s, -np.inf)
    t = _tile_max(s, nt)
    pad = nb * TILE - R
    valid = np.ones(nb * TILE, bool)
    if pad:
        t = np.concatenate([t, np.full((pad, nt), -np.inf)], axis=0)
        valid[R:] = False
    t = t.reshape(nb, TILE, nt)
    valid = valid.reshape(nb, TILE)
    qbs = qb0 + np.arange(nb)
    if causal:
        visited = np.arange(nt)[None, :] <= qbs[:, None]
    else:
        visited = np.ones((nb, nt), bool)
    return s, t, valid, visited


def prefill_decisions(qrows: np.ndarray, k: np.ndarray, qb0: int, causal: bool, taus):
    """The skip decisions alone (no softmax) of consecutive 64-row query
    blocks of one (batch, head), for each threshold in ``taus``: the scores
    and tile maxima are formed once and the rule is run per tau.
    Returns {tau: (decisions (nb, nt), margins (nb, nt))}."""
    _, t, valid, visited = _block_scores(qrows, k, qb0, causal)
    taus = list(taus)
    nb = t.shape[0]
    # one pass of the rule over the blocks repeated once per tau, each copy
    # with its own threshold (the copies are independent decision blocks)
    tau_col = np.repeat(np.asarray(taus, np.float64), nb)[:, None]
    dec, margin = _decide(np.concatenate([t] * len(taus)), np.concatenate([valid] * len(taus)),
                          np.concatenate([visited] * len(taus)), tau_col, None)
    return {tau: (dec[i * nb:(i + 1) * nb], margin[i * nb:(i + 1) * nb])
            for i, tau in enumerate(taus)}


def prefill_blocks(qrows: np.ndarray, k: np.ndarray, v: np.ndarray, qb0: int,
                   causal: bool, tau: float, forced: np.ndarray | None = None):
    """Oracle for consecutive 64-row query blocks of one (batch, head).

    qrows  (R, d) fp64 rows qb0*64 ... qb0*64 + R - 1 (R <= nb*64; the last
           block may be partial only if it ends at N)
    k, v   (N, d) fp64 keys and values of the head's KV group
    Returns o (R, d), lse (R,), decisions (nb, nt), margins (nb, nt).
    """
    R = qrows.shape[0]
    N = k.shape[0]
    s, t, valid, visited = _block_scores(qrows, k, qb0, causal)
    dec, margin = _decide(t, valid, visited, tau, forced)
    keep_tile = dec == KEPT
    kept = np.repeat(np.repeat(keep_tile, TILE, axis=1), TILE, axis=0)
    kept = kept[:R, :N] & np.isfinite(s)
    o, lse = _softmax_kept(s, kept, v)
    return o, lse, dec, margin


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
            tau: float, forced: np.ndarray | None = None, blocks_per_chunk: int = 8):
    """Full prefill oracle.

    q (B,Hq,N,d), k/v (B,Hkv,N,d), fp64. Query head h reads KV head
    h // (Hq // Hkv). forced, if given, is (B,Hq,nqb,nkb) int8.
    Returns dict with o (B,Hq,N,d), lse (B,Hq,N), mask (B,Hq,nqb,nkb) uint8
    and margin (B,Hq,nqb,nkb).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nt = (N + TILE - 1) // TILE
    o = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    mask = np.empty((B, Hq, nt, nt), np.uint8)
    margin = np.empty((B, Hq, nt, nt))
    step = blocks_per_chunk
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, h // G], v[b, h // G]
            for qb0 in range(0, nt, step):
                qb1 = min(nt, qb0 + step)
                r0, r1 = qb0 * TILE, min(N, qb1 * TILE)
                fc = None if forced is None else forced[b, h, qb0:qb1]
                ob, lb, db, mb = prefill_blocks(q[b, h, r0:r1], kk, vv, qb0,
                                                causal, tau, fc)
                o[b, h, r0:r1] = ob
                lse[b, h, r0:r1] = lb
                mask[b, h, qb0:qb1] = db
                margin[b, h, qb0:qb1] = mb
    return dict(o=o, lse=lse, mask=mask, margin=margin)


def decode_heads(qs: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float,
                 split: int = SPLIT, forced: np.ndarray | None = None):
    """Oracle for several query heads (one token each) against one KV head.

    qs (n, d), k/v (L, d) fp64. Each split of ``split`` keys (a multiple of
    64) runs the rule with its own running max, per head. ``forced`` (n, nt)
    int8, if given, imposes decisions where it is >= 0. Returns o (n, d),
    lse (n,), decisions (n, nt), margins (n, nt).
    """
    if split % TILE:
        raise ValueError("split must be a multiple of 64")
    n = qs.shape[0]
    L = k.shape[0]
    nt = (L + TILE - 1) // TILE
    s = _scores(qs, k)                     # (n, L)
    t = _tile_max(s, nt)                   # (n, nt)
    # every (head, split) is its own decision block with its own running
    # maximum: split sp holds tiles sp*per .. sp*per + per - 1 (the last one
    # may be short; its missing tiles are not visited)
    per = split // TILE
    nsp = (nt + per - 1) // per
    tt = np.full((n, nsp * per), -np.inf)
    tt[:, :nt] = t
    visited = np.zeros((n, nsp * per), bool)
    visited[:, :nt] = True
    fc = None
    if forced is not None:
        fc = np.full((n, nsp * per), -1, np.int8)
        fc[:, :nt] = forced
        fc = fc.reshape(n * nsp, per)
    dd, mm = _decide(tt.reshape(n * nsp, 1, per), np.ones((n * nsp, 1), bool),
                     visited.reshape(n * nsp, per), tau, fc)
    dec = dd.reshape(n, nsp * per)[:, :nt].copy()
    margin = mm.reshape(n, nsp * per)[:, :nt].copy()
    kept = np.repeat(dec == KEPT, TILE, axis=1)[:, :L]
    o, lse = _softmax_kept(s, kept, v)
    return o, lse, dec, margin


def decode_head(qvec: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float,
                split: int = SPLIT, forced: np.ndarray | None = None):
    """Oracle for one query token against one KV head: decode_heads for a
    single head. qvec (d,), k/v (L, d) fp64. Returns o (d,), lse,
    decisions (nt,), margins (nt,)."""
    fc = None if forced is None else np.asarray(forced)[None, :]
    o, lse, dec, margin = decode_heads(qvec[None, :], k, v, tau, split, fc)
    return o[0], lse[0], dec[0], margin[0]


def decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float,
           split: int = SPLIT, forced: np.ndarray | None = None, heads=None):
    """Decode oracle: q (B,Hq,d), k/v (B,Hkv,L,d) fp64.

    ``heads`` optionally restricts the work to a list of (b, h) pairs (the
    other entries of the outputs are left NaN / 255). Returns dict with o
    (B,Hq,d), lse (B,Hq), mask (B,Hq,nt) and margin (B,Hq,nt).
    """
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    nt = (L + TILE - 1) // TILE
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    mask = np.full((B, Hq, nt), 255, np.uint8)
    margin = np.full((B, Hq, nt), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        fc = None if forced is None else forced[b, h]
        ob, lb, db, mb = decode_head(q[b, h], k[b, h // G], v[b, h // G], tau,
                                     split, fc)
        o[b, h], lse[b, h], mask[b, h], margin[b, h] = ob, lb, db, mb
    return dict(o=o, lse=lse, mask=mask, margin=margin)
