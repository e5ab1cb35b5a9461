"""Pure-Python brute force of the tile-ordered online softmax, for tiny inputs.

This is the literal streaming computation that blockwise attention performs
(TurboAttention talk page, "Technical Deep Dive"), with the Skip-Softmax test
of the TensorRT-LLM Skip Softmax summary page ("Key Points", "Detailed
Analysis") applied before a tile's exp and PV work: per query row a running
max m, a running normaliser l and an accumulator are updated one 64-key tile
at a time, in ascending key order, and the tile is dropped when every row of
the 64-row block has its tile maximum strictly below m - tau.

It uses scalar loops and ``math.exp`` only, so it shares nothing with the
vectorised oracle, whose decisions and outputs it pins.
"""
import math

TILE = 64
NEG = -math.inf


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def prefill_head(q, k, v, causal, tau):
    """q, k, v: lists of N rows (lists of d floats). Returns (o, lse, dec)."""
    n, d = len(q), len(q[0])
    scale = 1.0 / math.sqrt(d)
    nt = (n + TILE - 1) // TILE
    o = [None] * n
    lse = [None] * n
    dec = [[2] * nt for _ in range(nt)]
    for qb in range(nt):
        rows = list(range(qb * TILE, min(n, qb * TILE + TILE)))
        m = {r: NEG for r in rows}
        l = {r: 0.0 for r in rows}
        acc = {r: [0.0] * d for r in rows}
        for kb in range(nt):
            if causal and kb > qb:
                continue
            keys = list(range(kb * TILE, min(n, kb * TILE + TILE)))
            sc = {}
            for r in rows:
                sc[r] = [(_dot(q[r], k[j]) * scale) if (not causal or j <= r) else NEG
                         for j in keys]
            tmax = {r: max(sc[r]) for r in rows}
            if all(tmax[r] < m[r] - tau for r in rows):
                dec[qb][kb] = 1
                continue
            dec[qb][kb] = 0
            for r in rows:
                mn = max(m[r], tmax[r])
                alpha = math.exp(m[r] - mn) if m[r] != NEG else 0.0
                l[r] *= alpha
                acc[r] = [a * alpha for a in acc[r]]
                for jj, j in enumerate(keys):
                    if sc[r][jj] == NEG:
                        continue
                    p = math.exp(sc[r][jj] - mn)
                    l[r] += p
                    acc[r] = [a + p * x for a, x in zip(acc[r], v[j])]
                m[r] = mn
        for r in rows:
            o[r] = [a / l[r] for a in acc[r]]
            lse[r] = m[r] + math.log(l[r])
    return o, lse, dec


def decode_head(qv, k, v, tau, split):
    """One query (list of d) against L keys; splits of ``split`` keys, each
    with its own running max; partial results merged by log-sum-exp."""
    L, d = len(k), len(qv)
    scale = 1.0 / math.sqrt(d)
    nt = (L + TILE - 1) // TILE
    dec = [0] * nt
    parts = []
    for s0 in range(0, L, split):
        s1 = min(L, s0 + split)
        m, l, acc = NEG, 0.0, [0.0] * d
        for t0 in range(s0, s1, TILE):
            keys = list(range(t0, min(s1, t0 + TILE)))
            sc = [_dot(qv, k[j]) * scale for j in keys]
            tmax = max(sc)
            if tmax < m - tau:
                dec[t0 // TILE] = 1
                continue
            mn = max(m, tmax)
            alpha = math.exp(m - mn) if m != NEG else 0.0
            l *= alpha
            acc = [a * alpha for a in acc]
            for jj, j in enumerate(keys):
                p = math.exp(sc[jj] - mn)
                l += p
                acc = [a + p * x for a, x in zip(acc, v[j])]
            m = mn
        parts.append((m + math.log(l), [a / l for a in acc]))
    big = max(p[0] for p in parts)
    w = [math.exp(p[0] - big) for p in parts]
    tot = sum(w)
    lse = big + math.log(tot)
    o = [sum(wi * p[1][c] for wi, p in zip(w, parts)) / tot for c in range(d)]
    return o, lse, dec
