"""Parity between the HIP library and the fp64 oracle.

Rules (tolerances of the Skip-Softmax attention workloads):
* skip masks must match bit for bit, except tiles whose oracle margin
  |min_r (m_r - tau - t_r)| is below 1e-3 logits: there the GPU's fp32
  scores may round either way. Such tiles are counted; the oracle then
  re-evaluates the affected query block (or decode head) under the GPU's
  decision before outputs are compared;
* max |O_gpu - O_oracle| <= 1e-2 (fp32 accumulation of bf16 inputs and a
  bf16-rounded P in the PV product);
* max |LSE_gpu - LSE_oracle| <= 1e-3.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle
import synth

O_TOL = 1e-2
LSE_TOL = 1e-3
MARGIN_EPS = 1e-3


@dataclass
class Report:
    tiles: int = 0
    ambiguous: int = 0
    hard_mismatch: int = 0
    skipped: int = 0
    o_err: float = 0.0
    lse_err: float = 0.0
    notes: list = field(default_factory=list)

    def merge(self, other: "Report"):
        self.tiles += other.tiles
        self.ambiguous += other.ambiguous
        self.hard_mismatch += other.hard_mismatch
        self.skipped += other.skipped
        self.o_err = max(self.o_err, other.o_err)
        self.lse_err = max(self.lse_err, other.lse_err)
        self.notes += other.notes

    def ok(self) -> bool:
        return (self.hard_mismatch == 0 and self.o_err <= O_TOL
                and self.lse_err <= LSE_TOL)

    def __str__(self):
        return (f"tiles={self.tiles} skipped={self.skipped} ambiguous={self.ambiguous} "
                f"hard_mismatch={self.hard_mismatch} o_err={self.o_err:.3e} "
                f"lse_err={self.lse_err:.3e} {self.notes[:3]}")


def max_abs_err(got, want) -> float:
    """Largest |got - want|; +inf if any entry of either side is not finite
    (a NaN must fail the tolerance, not vanish in a max)."""
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(d.max()) if np.all(np.isfinite(d)) else math.inf


def _compare_decisions(gpu_dec, ref_dec, margin, visited):
    """Return (forced array or None, n_ambiguous, n_hard) for one block."""
    diff = (gpu_dec != ref_dec) & visited
    amb = diff & (np.abs(margin) < MARGIN_EPS)
    hard = diff & ~amb
    forced = None
    if amb.any():
        forced = np.full(gpu_dec.shape, -1, np.int8)
        forced[amb] = gpu_dec[amb]
    return forced, int(amb.sum()), int(hard.sum())


class PrefillChecker:
    """Caches fp64 copies of K/V per (b, kv head) for repeated block checks."""

    def __init__(self, q_bits, k_bits, v_bits, causal: bool, q0: int = 0, qf=None, kf=None,
                 sas: int = 0, pv8: bool = False, score_err_rel: float = 0.0,
                 lin_err: bool = True):
        """q_bits may be a chunk: its row r sits at key position q0 + r
        (q0 a multiple of 64 when causal). ``qf`` / ``kf``, fp64 arrays of
        the same shapes, replace the bf16 Q / K values (e.g. the oracle's
        dequantised 8-bit Q and K). ``sas`` = 2 or 3: the reference is the
        SAS prefill oracle of that degree, and each row's error beyond the
        slack its SAS steps allow counts against the tolerance. ``pv8``: the
        reference is the 8-bit P.V oracle on the oracle's V codes; a kernel
        score may differ from the oracle's by up to score_err_rel times the
        sum of |q_i k_i| / sqrt(d) (plus 2^-17), which sets how close to an
        E4M3 rounding point a probability must be for either rounding to
        count as right (the slack), and a block whose rescale test came that
        close to its margin is counted as ambiguous, its outputs unchecked.
        ``lin_err``: the same error also widens O and LSE to first order
        (for 8-bit QK^T, whose MFMA sums are inexact; bf16 QK^T scores are as
        exact as the bf16 prefill's tolerances already assume)."""
        self.q, self.k, self.v = q_bits, k_bits, v_bits
        self.sas = sas
        self.pv8 = pv8
        self.score_err_rel = score_err_rel
        self.lin_err = lin_err
        self._amb = False
        self.qf, self.kf = qf, kf
        self.causal = causal
        B, Hq, N, d = q_bits.shape
        self.B, self.Hq, self.N, self.d = B, Hq, N, d
        self.Hkv = k_bits.shape[1]
        self.G = Hq // self.Hkv
        self.nt = (N + 63) // 64
        self.q0t = q0 // 64
        self._kv = {}

    def kv(self, b, g):
        key = (b, g)
        if key not in self._kv:
            if len(self._kv) > 2:
                self._kv.clear()
            kk = self.kf[b, g] if self.kf is not None else synth.bf16_bits_to_f64(self.k[b, g])
            if self.pv8:
                codes, sv = oracle.fp8pv.quantize_v(synth.bf16_bits_to_f32(self.v[b, g]))
                self._kv[key] = (kk, (oracle.fp8.e4m3_value(codes), float(sv)))
            else:
                self._kv[key] = (kk, synth.bf16_bits_to_f64(self.v[b, g]))
        return self._kv[key]

    def qrows(self, b, h, r0, r1):
        if self.qf is not None:
            return np.asarray(self.qf[b, h, r0:r1], np.float64)
        return synth.bf16_bits_to_f64(self.q[b, h, r0:r1])

    def _ref(self, qrows, k, v, qb, tau, forced=None):
        """o, lse, decisions, margins, slack (rows, 2) or None."""
        if self.pv8:
            vvals, sv = v
            err = (self.score_err_rel * (np.abs(qrows) @ np.abs(k).T) / math.sqrt(k.shape[1])
                   + 2.0 ** -17)
            o, lse, dec, margin, slack, amb = oracle.fp8pv.pv8_blocks(
                qrows, k, vvals, sv, qb + self.q0t, self.causal, tau, forced, score_err=err,
                lin_err=None if self.lin_err else 0.0)
            self._amb = bool(amb.any())
            return o, lse, dec, margin, slack
        if self.sas:
            return oracle.sas.prefill_blocks(qrows, k, v, qb + self.q0t, self.causal, tau,
                                             self.sas, forced)
        o, lse, dec, margin = oracle.prefill_blocks(qrows, k, v, qb + self.q0t, self.causal,
                                                    tau, forced)
        return o, lse, dec, margin, None

    @staticmethod
    def _errs(o_gpu, lse_gpu, o, lse, slack):
        if slack is None:
            return max_abs_err(o_gpu, o), max_abs_err(lse_gpu, lse)
        eo = np.abs(np.asarray(o_gpu, np.float64) - o).max(axis=1)
        el = np.abs(np.asarray(lse_gpu, np.float64) - lse)
        if not (np.all(np.isfinite(eo)) and np.all(np.isfinite(el))):
            return math.inf, math.inf
        return (float(np.maximum(eo - slack[:, 1], 0.0).max()),
                float(np.maximum(el - slack[:, 0], 0.0).max()))

    def check_block(self, b, h, qb, tau, o_gpu, lse_gpu, mask_gpu) -> Report:
        """o_gpu/lse_gpu: numpy rows of this block; mask_gpu: (nt,) uint8."""
        rep = Report()
        k, v = self.kv(b, h // self.G)
        r0, r1 = qb * 64, min(self.N, qb * 64 + 64)
        qrows = self.qrows(b, h, r0, r1)
        o, lse, dec, margin, slack = self._ref(qrows, k, v, qb, tau)
        dec, margin = dec[0], margin[0]
        visited = dec != oracle.NOT_VISITED
        if not np.array_equal(mask_gpu[~visited], dec[~visited]):
            rep.hard_mismatch += int((mask_gpu[~visited] != dec[~visited]).sum())
            rep.notes.append(f"not-visited marks differ at b={b} h={h} qb={qb}")
        forced, amb, hard = _compare_decisions(mask_gpu.astype(np.int16),
                                               dec.astype(np.int16), margin, visited)
        rep.ambiguous += amb
        rep.hard_mismatch += hard
        if hard:
            bad = np.nonzero((mask_gpu != dec) & visited)[0][:4]
            rep.notes.append(f"b={b} h={h} qb={qb} kb={bad.tolist()} margin={margin[bad].tolist()}")
        if forced is not None:
            o, lse, _, _, slack = self._ref(qrows, k, v, qb, tau, forced[None, :])
        rep.tiles += int(visited.sum())
        rep.skipped += int((mask_gpu[visited] == 1).sum())
        if self.pv8 and self._amb:
            rep.ambiguous += 1
            rep.notes.append(f"b={b} h={h} qb={qb}: rescale test at its margin, outputs unchecked")
            return rep
        rep.o_err, rep.lse_err = self._errs(o_gpu, lse_gpu, o, lse, slack)
        return rep


    def check_blocks(self, b, h, qb0, qb1, tau, o_gpu, lse_gpu, mask_gpu) -> Report:
        """Query blocks qb0 .. qb1 - 1 of one head in one oracle call (the
        rule runs over all of them at once); o_gpu/lse_gpu are their rows,
        mask_gpu (qb1 - qb0, nt)."""
        rep = Report()
        k, v = self.kv(b, h // self.G)
        r0, r1 = qb0 * 64, min(self.N, qb1 * 64)
        qrows = self.qrows(b, h, r0, r1)
        o, lse, dec, margin = oracle.prefill_blocks(qrows, k, v, qb0 + self.q0t, self.causal, tau)
        visited = dec != oracle.NOT_VISITED
        if not np.array_equal(mask_gpu[~visited], dec[~visited]):
            rep.hard_mismatch += int((mask_gpu[~visited] != dec[~visited]).sum())
            rep.notes.append(f"not-visited marks differ at b={b} h={h} qb={qb0}..{qb1 - 1}")
        forced, amb, hard = _compare_decisions(mask_gpu.astype(np.int16),
                                               dec.astype(np.int16), margin, visited)
        rep.ambiguous += amb
        rep.hard_mismatch += hard
        if hard:
            bad = np.argwhere((mask_gpu != dec) & visited)[:4]
            rep.notes.append(f"b={b} h={h} (qb-{qb0}, kb)={bad.tolist()}")
        if forced is not None:
            o, lse, _, _ = oracle.prefill_blocks(qrows, k, v, qb0 + self.q0t, self.causal, tau,
                                                 forced)
        rep.tiles += int(visited.sum())
        rep.skipped += int((mask_gpu[visited] == 1).sum())
        rep.o_err = max_abs_err(o_gpu, o)
        rep.lse_err = max_abs_err(lse_gpu, lse)
        return rep


def check_prefill(q_bits, k_bits, v_bits, causal, tau, o, lse, mask, blocks=None,
                  q0: int = 0, qf=None, kf=None, sas: int = 0, pv8: bool = False,
                  score_err_rel: float = 0.0, lin_err: bool = True) -> Report:
    """Compare full GPU outputs (numpy) over the given (b, h, qb) blocks
    (q_bits and the outputs may be a chunk starting at key position q0;
    qf / kf / sas / pv8 / score_err_rel / lin_err as for PrefillChecker)."""
    chk = PrefillChecker(q_bits, k_bits, v_bits, causal, q0, qf, kf, sas, pv8, score_err_rel,
                         lin_err)
    if blocks is None:
        blocks = [(b, h, qb) for b in range(chk.B) for h in range(chk.Hq)
                  for qb in range(chk.nt)]
    blocks = sorted(blocks, key=lambda x: (x[0], x[1] // chk.G, x[1], x[2]))
    rep = Report()
    for b, h, qb in blocks:
        r0, r1 = qb * 64, min(chk.N, qb * 64 + 64)
        rep.merge(chk.check_block(b, h, qb, tau, o[b, h, r0:r1], lse[b, h, r0:r1],
                                  mask[b, h, qb]))
    return rep


def check_decode(q_bits, k_bits, v_bits, tau, o, lse, mask, heads=None,
                 split=oracle.SPLIT, kv_for=None, Hkv=None, sas=0) -> Report:
    """``kv_for(b, g)`` -> (k, v) fp64 (L, d) replaces the bf16 K/V (then
    k_bits and v_bits may be None and Hkv must be given): the 4-bit cache
    is checked against the oracle on its dequantised values. ``sas`` = 2 or
    3 checks against the SAS decode oracle of that degree; its tolerances
    grow by the oracle's bound on the steps of SAS that the kernel's fp32
    arguments may fall on the other side of."""
    B, Hq, d = q_bits.shape
    if kv_for is None:
        Hkv = k_bits.shape[1]

        def kv_for(b, g):
            return synth.bf16_bits_to_f64(k_bits[b, g]), synth.bf16_bits_to_f64(v_bits[b, g])
    G = Hq // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    groups = {}
    for b, h in sorted(heads):
        groups.setdefault((b, h // G), []).append(h)
    rep = Report()
    for (b, g), hs in groups.items():
        k, v = kv_for(b, g)
        qs = synth.bf16_bits_to_f64(q_bits[b, hs])
        gpu_mask = mask[b, hs]

        def run(sel, forced=None):
            """Oracle for heads hs[i], i in sel: o, lse, dec, margin, slack."""
            if sas:
                outs = [oracle.sas.decode_head(qs[i], k, v, tau, sas, split,
                                               None if forced is None else forced[j])
                        for j, i in enumerate(sel)]
                return (np.stack([x[0] for x in outs]), np.array([x[1] for x in outs]),
                        np.stack([x[2] for x in outs]), np.stack([x[3] for x in outs]),
                        [x[4] for x in outs])
            ro, rl, dec, margin = oracle.decode_heads(qs[sel], k, v, tau, split, forced)
            return ro, rl, dec, margin, [(0.0, 0.0)] * len(sel)

        allh = list(range(len(hs)))
        ro, rl, dec, margin, slack = run(allh)
        visited = np.ones(dec.shape, bool)
        forced, amb, hard = _compare_decisions(gpu_mask.astype(np.int16),
                                               dec.astype(np.int16), margin, visited)
        if hard:
            bad = np.argwhere(gpu_mask != dec)[:4]
            rep.notes.append(f"b={b} (head, tile)={[(hs[i], t) for i, t in bad.tolist()]} "
                             f"margin={[float(margin[i, t]) for i, t in bad.tolist()]}")
        if forced is not None:
            redo = [i for i in allh if (forced[i] >= 0).any()]
            o2, l2, _, _, s2 = run(redo, forced[redo])
            for j, i in enumerate(redo):
                ro[i], rl[i], slack[i] = o2[j], l2[j], s2[j]
        rep.tiles += dec.size
        rep.skipped += int((gpu_mask == 1).sum())
        rep.ambiguous += amb
        rep.hard_mismatch += hard
        # errors beyond the slack the SAS steps allow count against the tolerance
        for i, h in enumerate(hs):
            rep.o_err = max(rep.o_err, max(0.0, max_abs_err(o[b, h], ro[i]) - slack[i][1]))
            rep.lse_err = max(rep.lse_err, max(0.0, max_abs_err(lse[b, h], rl[i]) - slack[i][0]))
    return rep


def sample_blocks(B, Hq, nt, causal, count, seed=0):
    """A spread of (b, h, qb): every head's first and last block plus random
    ones, biased to late (long) blocks for causal attention."""
    rng = np.random.default_rng(seed)
    out = set()
    for b in range(B):
        for h in range(Hq):
            out.add((b, h, nt - 1))
    out.add((0, 0, 0))
    while len(out) < count:
        b = int(rng.integers(B))
        h = int(rng.integers(Hq))
        qb = int(nt - 1 - math.floor(rng.random() ** 2 * nt)) if causal else int(rng.integers(nt))
        out.add((b, h, qb))
    return sorted(out)
