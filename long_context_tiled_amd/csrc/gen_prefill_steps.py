#!/usr/bin/env python3
"""Writes prefill_steps.inc: the per-key-tile steps of the prefill kernel as
hand-scheduled gfx950 instruction blocks.

Blockwise attention keeps, per query row, a running maximum and rescaled sums
while it walks the key tiles in order (TurboAttention talk page, "Technical
Deep Dive"); the Skip-Softmax rule adds a per-tile test on the tile's row
maxima before the exponentials and the PV product (TensorRT-LLM Skip Softmax
summary page, "Key Points"). One wave owns 64 queries of one head. Per key
tile it does two MFMA products, S^T = K Q^T and O^T += V^T P^T, and vector
work: the row maxima of S for the test, and exp2 / bf16 packing / row sums
for P. In a plain loop these alternate and the matrix cores idle while the
vector ALUs work. Here each step overlaps two tiles:

  phase A: the 4 KS MFMAs of S^T for tile n + 1, and
  phase B: the 8 MB MFMAs of O^T += V^T P^T for tile n,
  with the exponentials of tile n and the row maxima of tile n + 1 spread
  over the MFMA issue slots of both phases.

An MFMA takes 32 cycles; vector instructions issued after it run meanwhile.
Measured on gfx950 for one wave per SIMD: every instruction costs about 4
issue cycles (an s_nop too), v_exp about 8, an MFMA issue about 8; up to six
plain VALU instructions hide completely behind one 32-cycle MFMA. The
scheduler below fills each MFMA slot with about BUDGET cycles of vector work.

The step variants:
  full  - phase A (S of tile n + 1 into buffer Y) and phase B (exp and PV of
          tile n from buffer X), row maxima of Y.
  qk    - S of tile n + 1 into Y and its row maxima (tile n was skipped, or
          there is no tile n yet).
  pv    - exp and PV of tile n from X (the wave's last tile).

Register plan (fixed, so the blocks can name registers directly):
  a[0 : 32 MB)          O^T accumulators, block (mb, nb) at 16 (2 mb + nb)
  a[QB : QB + 8 KS)     Q^T fragments (QB = 32 MB), k-step ks, half nb at
                        QB + 8 ks + 4 nb; loaded once per wave
  v[128:191] v[192:255] score buffers A and B: S^T block (a, nb) of a tile at
                        base + 16 (2 a + nb), element r at + r
  v[64:95]              K fragments (phase A) / V^T fragments (phase B)
  v[96:127]             P^T operand, key step kp, query half nb at
                        96 + 4 (2 kp + nb)
  v[48:63]              exp temporaries and LDS read addresses
  v[40:46)              vote temporaries
Everything below v40 (and a40) is left to the compiler.

After the row maxima of the new tile, the full and qk steps also take the
Skip-Softmax vote on it: the per-query maxima of the two lane halves are
combined (v_permlane32_swap), compared with m - tau, and any valid row that
does not clear the threshold keeps the tile. A kept tile raises the running
maxima m (unless the caller flags the tile as needing a mask first), and the
step reports whether some m now exceeds the reference max by more than the
lazy-rescale margin.

Hazards are resolved here, not by the compiler (which does not look inside
asm): every read of a register is checked against its last writer and
s_nop / s_waitcnt lgkmcnt are inserted as needed:
  MFMA (8 passes) write -> VALU read           12 wait states
  VALU write -> MFMA read                      4 (2 required)
  transcendental write -> VALU read            1
  ds_read -> any use                           s_waitcnt lgkmcnt
  MFMA read of a fragment -> ds_read over it   2
Back-to-back accumulation into the same MFMA destination needs none.

Run:  python gen_prefill_steps.py [OUT]   (default: prefill_steps.inc beside it)
"""
import os
import re
import sys

NOP_MFMA_VALU = 12       # 8-pass MFMA (bf16 32x32x16) result -> VALU read
NOP_MFMA16_VALU = 20     # 16-pass MFMA (fp8 32x32x64) result -> VALU read
NOP_VALU_MFMA = 4
NOP_TRANS_VALU = 1
NOP_MFMA_READ_LOAD = 2
NOP_MFMA16_READ_LOAD = 4
NOP_VALU_PERM = 2

COST = {"v_exp_f32": 8.2, "v_cvt_pk_bf16_f32": 6.0, "v_cvt_pk_fp8_f32": 6.0}
COST_DEFAULT = 4.2

SBUF = {"A": 128, "B": 192}
KREG = 64     # K / V^T fragments, v[64:95]
PREG = 96     # P^T operand, v[96:127] (8-bit P.V: v[96:111])
VF8 = (80, 88, 64, 72)  # 8-bit P.V: V^T fragment of 32-d block mb, 8 registers
TREG = 48     # exp temporaries, three pairs v[48:53]
VADR = 54     # V^T read addresses, v[54 : 54 + 2 MB)
KADR = 62     # K read addresses, v62 / v63 alternating
KADR8 = 40    # fp8 QK: K read addresses of k-step / half pairs, v[40:43) (phase A only;
              # the vote uses these registers after phase A)
VOTE = 40     # vote temporaries, v[40:46)
PSUM = 46     # this tile's partial row sums, v46 (query half 0) and v47 (half 1)
OB = 64       # first AGPR of O^T
COMPILER_VGPRS = 40  # v[0:40) and a[0:40) stay with the compiler


def expand(r):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", r)
    if m:
        return [f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    m = re.fullmatch(r"([va])(\d+)", r)
    return [r] if m else []


def rng(kind, lo, n):
    return f"{kind}[{lo}:{lo + n - 1}]"


class Ins:
    def __init__(self, text, kind, wr=(), rd=(), tag=None):
        self.text = text
        self.kind = kind  # mfma | valu | trans | lds
        self.wr = [x for r in wr for x in expand(r)]
        self.rd = [x for r in rd for x in expand(r)]
        self.tag = tag
        op = text.split()[0]
        self.cost = COST.get(op, COST_DEFAULT) if kind in ("valu", "trans", "perm") else (
            1.0 if kind == "salu" else 0.0)
        self.is_mfma = kind in ("mfma", "mfma16")


class Step:
    """One step variant for one head dim and buffer assignment."""

    def __init__(self, d, variant, x, y, budget, loop=False, dma=False, f8=False, sas=0,
                 v8=False, i8=False):
        self.loop = loop
        # QK^T on int8 codes: the fp8 operand layout (one byte per element),
        # each 32x32x64 fp8 MFMA replaced by two 32x32x32 int8 MFMAs over the
        # two 16-byte halves of the operands, int32 scores converted in place
        # before the row maxima
        self.i8 = i8
        self.v8 = v8          # P.V on fp8: one 32x32x64 MFMA per (d block, query half)
        self.sas = sas        # 0: exp2; 2 or 3: the SAS exponential of that degree
        self.dma = dma
        self.d = d
        self.f8 = f8          # QK^T on fp8 codes (32x32x64, 16 passes), PV in bf16
        self.MB = d // 32
        self.KS = d // 64 if f8 else d // 16   # QK k-steps
        self.QB = OB + 32 * self.MB
        self.rowBytes = 2 * d                  # V rows (bf16)
        self.vTileBytes = 64 * d if v8 else 64 * self.rowBytes
        self.kRowBytes = d if f8 else 2 * d    # K and Q rows
        self.variant = variant
        self.x = x  # buffer holding tile n (exp / PV)
        self.y = y  # buffer receiving tile n + 1 (QK / max)
        self.budget = budget
        self.qk = variant in ("full", "qk")
        self.pv = variant in ("full", "pv")

    # ---- instruction builders -------------------------------------------
    def s_reg(self, buf, a, nb, r=0):
        return SBUF[buf] + 16 * (2 * a + nb) + r

    def s_blk(self, buf, a, nb):
        return rng("v", self.s_reg(buf, a, nb), 16)

    def kfrag(self, j, a=0):
        if self.f8:
            # fragments of key half 0 in v[80:95], key half 1 in v[64:79]: the
            # V^T fragments of PV k-step 0 (v[80:95]) may then be loaded as
            # soon as key half 0's QK MFMAs have read theirs
            return rng("v", KREG + 8 * (j ^ 2), 8)
        return rng("v", KREG + 4 * j, 4)

    def vfrag(self, j, mb):
        # V^T fragments of one key step: MB tuples of 4 registers; two buffers
        return rng("v", KREG + 16 * j + 4 * mb, 4)

    def pfrag(self, kp, nb):
        return rng("v", PREG + 4 * (2 * kp + nb), 4)

    def pfrag8(self, nb):
        # 8-bit P.V: query half nb's probabilities of the whole tile, 32 bytes
        return rng("v", PREG + 8 * nb, 8)

    def vfrag8(self, mb):
        return rng("v", VF8[mb], 8)

    def v_loads8(self, mbs):
        """8-bit P.V: V^T fragments of the given 32-d blocks. Row c of the
        tile's code block (64 bytes) holds channel c in contraction order;
        lane l reads row 32 mb + (l & 31), 32 bytes: the chunk at %[vb0]
        and the one at %[vb1] (= %[vb0] ^ 16), block mb 2 KB further."""
        out = []
        for mb in mbs:
            base = VF8[mb]
            for half, adr in ((0, "%[vb0]"), (1, "%[vb1]")):
                dst = rng("v", base + 4 * half, 4)
                out.append(Ins(f"ds_read_b128 {dst}, {adr} offset:{2048 * mb}", "lds",
                               wr=[dst], rd=[adr]))
        return out

    def pv8_mfma(self, mb, nb):
        o = self.oblk(mb, nb)
        vf = self.vfrag8(mb)
        pf = self.pfrag8(nb)
        return Ins(f"v_mfma_f32_32x32x64_f8f6f4 {o}, {vf}, {pf}, {o}", "mfma16", wr=[o],
                   rd=[vf, pf, o], tag=("pv8", nb))

    def qfrag(self, ks, nb):
        if self.f8:
            return rng("a", self.QB + 16 * ks + 8 * nb, 8)
        return rng("a", self.QB + 8 * ks + 4 * nb, 4)

    def oblk(self, mb, nb):
        return rng("a", OB + 16 * (2 * mb + nb), 16)

    def k_load(self, a, ks, j):
        """K fragment (k-step ks, key half a) into fragment buffer j. The
        fragment address of k-step ks is the tile base XOR 32 ks (the swizzle
        only moves address bits 4..7; the tile base has bits 0..9 clear)."""
        out = []
        if self.f8:
            # 32 bytes per lane: 16-byte chunks 4 ks + 2 hh and the next one,
            # at address kb0 ^ 64 ks and that ^ 16 (the swizzle moves only
            # address bits 4..6 within a 128-byte row); key half 1 is the
            # immediate offset of 32 rows. The addresses of (ks, chunk) != (0, 0)
            # are formed once, with key half 0's loads.
            names = {(0, 0): "%[kb0]", (0, 1): f"v{KADR8}", (1, 0): f"v{KADR8 + 1}",
                     (1, 1): f"v{KADR8 + 2}"}
            if a == 0:
                for jj in range(2):
                    if (ks, jj) != (0, 0):
                        out.append(Ins(f"v_xor_b32 {names[(ks, jj)]}, {64 * ks + 16 * jj}, %[kb0]",
                                       "valu", wr=[names[(ks, jj)]]))
            dst = self.kfrag(j, 0)
            base = KREG + 8 * (j ^ 2)
            off = a * 32 * self.kRowBytes
            for jj in range(2):
                adr = names[(ks, jj)]
                part = rng("v", base + 4 * jj, 4)
                out.append(Ins(f"ds_read_b128 {part}, {adr} offset:{off}", "lds",
                               wr=[part], rd=[adr]))
            return out
        if ks == 0:
            adr = "%[kb0]"
        else:
            adr = f"v{KADR + (j & 1)}"
            out.append(Ins(f"v_xor_b32 {adr}, {32 * ks}, %[kb0]", "valu", wr=[adr]))
        dst = self.kfrag(j, 0)
        off = a * 32 * self.rowBytes
        out.append(Ins(f"ds_read_b128 {dst}, {adr} offset:{off}", "lds", wr=[dst], rd=[adr]))
        return out

    def v_addr(self):
        # V^T read address of (32-d block mb, 4-key half): the half's base
        # XOR 64 mb (the block moves the 16-byte chunk index by 4 mb)
        out = []
        for mb in range(self.MB):
            for half in range(2):
                r = f"v{VADR + 2 * mb + half}"
                if mb == 0:
                    out.append(Ins(f"v_mov_b32 {r}, %[vb{half}]", "valu", wr=[r]))
                else:
                    out.append(Ins(f"v_xor_b32 {r}, {64 * mb}, %[vb{half}]", "valu", wr=[r]))
        return out

    def v_loads(self, ks):
        out = []
        j = (ks + 1) & 1
        for mb in range(self.MB):
            base = KREG + 16 * j + 4 * mb
            off = ks * 16 * self.rowBytes
            for half in range(2):
                dst = rng("v", base + 2 * half, 2)
                adr = f"v{VADR + 2 * mb + half}"
                out.append(Ins(f"ds_read_b64_tr_b16 {dst}, {adr} offset:{off}", "lds",
                               wr=[dst], rd=[adr]))
        return out

    def dma_groups(self):
        """This wave's share of the copies of tile n + 2 (K then V), one group
        per instruction: the tile offset into the VGPR offset (the raw-buffer
        range check, which zero-fills keys past N, covers voffset only), the
        LDS destination into M0. %[t1] is the tile's byte offset, %[t2] this
        wave's LDS destination base."""
        groups = []
        n = 0
        if self.f8 or self.v8:
            # K and V tiles of different formats: %[t1] / %[t4] are their byte
            # offsets, %[t2] / %[t5] this wave's LDS bases
            parts = (("K", "%[krs]", "gk", "%[t1]", "%[t2]", 64 * self.kRowBytes // 4096),
                     ("V", "%[vrs]", "gv", "%[t4]", "%[t5]", self.vTileBytes // 4096))
        else:
            ipw = 64 // (1024 // self.rowBytes) // 4
            tile_bytes = 64 * self.rowBytes
            parts = (("K", "%[krs]", "gk", "%[t1]", "%[t2]", ipw),
                     ("V", "%[vrs]", "gv", "%[t1]", "%[t2]", ipw))
        for which, rs, g, toff, lbase, ipw in parts:
            for i in range(ipw):
                off = i * 1024
                if not (self.f8 or self.v8) and which == "V":
                    off += tile_bytes
                tmp = "%[vt]" if n % 2 == 0 else "%[vz]"
                n += 1
                # the VALU add sits between the M0 write and the copy that
                # reads M0, which needs one wait state there
                groups.append([Ins(f"s_add_u32 m0, {lbase}, {off}", "salu"),
                               Ins(f"v_add_u32 {tmp}, {toff}, %[{g}{i}]", "valu"),
                               Ins(f"buffer_load_dwordx4 {tmp}, {rs}, 0 offen lds", "vmem")])
        return groups

    def qk_mfmas(self, ks, a, nb, j):
        """The QK^T MFMAs of one (k-step, key half, query half): one, or two
        for int8 (contraction halves: operand registers 0-3, then 4-7; the
        A and B halves hold the same d positions, so the sum is the same).
        The int8 sums start from the bits of the inline constant 1/(2 pi),
        0x3e22f983: an int32 score s, |s| <= 127 * 127 * 128 < 2^21, comes
        out as the bits of the float K0 + s 2^-26 (K0 = 1/(2 pi) and the sum
        share the binade [1/8, 1/4), whose ulp is 2^-26), so the scores are
        exact fp32 values without a conversion, and their int32 order is
        the order of s."""
        if not self.i8:
            return [self.qk_mfma(ks, a, nb, j)]
        s = self.s_blk(self.y, a, nb)
        kb, qb = KREG + 8 * (j ^ 2), self.QB + 16 * ks + 8 * nb
        out = []
        for h in range(2):
            kf, qf = rng("v", kb + 4 * h, 4), rng("a", qb + 4 * h, 4)
            first = ks == 0 and h == 0
            src_c = "0.15915494" if first else s
            out.append(Ins(f"v_mfma_i32_32x32x32_i8 {s}, {kf}, {qf}, {src_c}", "mfma", wr=[s],
                           rd=[kf, qf] + ([] if first else [s])))
        return out

    def qk_mfma(self, ks, a, nb, j):
        s = self.s_blk(self.y, a, nb)
        kf = self.kfrag(j, 0)
        qf = self.qfrag(ks, nb)
        src_c = "0" if ks == 0 else s
        rd = [kf, qf] + ([] if ks == 0 else [s])
        if self.f8:
            return Ins(f"v_mfma_f32_32x32x64_f8f6f4 {s}, {kf}, {qf}, {src_c}", "mfma16", wr=[s],
                       rd=rd)
        return Ins(f"v_mfma_f32_32x32x16_bf16 {s}, {kf}, {qf}, {src_c}", "mfma", wr=[s], rd=rd)

    def pv_mfma(self, ks, mb, nb):
        o = self.oblk(mb, nb)
        vf = self.vfrag((ks + 1) & 1, mb)
        pf = self.pfrag(ks, nb)
        return Ins(f"v_mfma_f32_32x32x16_bf16 {o}, {vf}, {pf}, {o}", "mfma", wr=[o], rd=[vf, pf, o],
                   tag=("pv", ks))

    def exp_stream(self):
        if self.sas:
            return self.sas_stream()
        return self.exp2_stream()

    def pairs(self):
        """Score pairs (a, nb, r0) of a tile in exponential order: key step by
        key step for the bf16 P.V (its k-steps consume keys 16 at a time);
        query half by query half for the 8-bit P.V (one MFMA per query half
        takes all 64 keys)."""
        if self.v8:
            return [(a, nb, r0) for nb in range(2) for a in range(2) for r0 in range(0, 16, 2)]
        out = []
        for gp in range(32):
            ch, i2 = gp >> 2, gp & 3
            kp, nb = ch >> 1, ch & 1
            out.append((kp >> 1, nb, 8 * (kp & 1) + 2 * i2))
        return out

    def pack(self, a, nb, r0, t0, t1):
        """The pair's P^T operand write: bf16 pair (key step kp), or two fp8
        bytes of the query half's 32-byte operand: accumulator element r of
        key half a is contraction index 16 a + r, byte (r & 3) of register
        4 a + (r >> 2)."""
        if self.v8:
            w = f"v{PREG + 8 * nb + 4 * a + (r0 >> 2)}"
            if r0 & 2:   # bytes 2-3: the high half, the low half kept
                return Ins(f"v_cvt_pk_fp8_f32 {w}, {t0}, {t1} op_sel:[0,0,1]", "valu", wr=[w],
                           rd=[t0, t1, w], tag=("pf8", nb))
            return Ins(f"v_cvt_pk_fp8_f32 {w}, {t0}, {t1}", "valu", wr=[w], rd=[t0, t1],
                       tag=("pf8", nb))
        kp = 2 * a + (r0 >> 3)
        w = f"v{PREG + 4 * (2 * kp + nb) + ((r0 & 7) >> 1)}"
        return Ins(f"v_cvt_pk_bf16_f32 {w}, {t0}, {t1}", "valu", wr=[w], rd=[t0, t1],
                   tag=("pf", kp))

    def sas_stream(self):
        """The SAS exponential per score: x = (mref - s) / sqrt(d) clamped to
        [0, 7] (nm = mref / sqrt(d), %[c] = 1 / sqrt(d)), n = floor x,
        f = x - n, P = e^-n (the exponential unit on -n log2 e) x
        clamp(6 - n, 0, 1) (0 from n = 6 on) x p(f) (Horner on the SGPR
        coefficients %[sa0..3]); then pack, sums as exp2_stream. Pairs use two
        register slots: P in v48-v51, two temporaries per score in v52-v53
        and v40-v45 (the vote temporaries: every vote instruction of a step
        follows its last exponential)."""
        heads, tails = [], []
        first = {0: True, 1: True}
        tmp = [52, 53, 40, 41, 42, 43, 44, 45]
        deg = self.sas
        for gp in range(32):
            ch, i2 = gp >> 2, gp & 3
            kp, nb = ch >> 1, ch & 1
            a = kp >> 1
            r0 = 8 * (kp & 1) + 2 * i2
            sl = gp % 2
            ss = [f"v{self.s_reg(self.x, a, nb, r0 + i)}" for i in range(2)]
            ts = [f"v{TREG + 2 * sl + i}" for i in range(2)]
            us = [f"v{tmp[4 * sl + 2 * i]}" for i in range(2)]
            ws = [f"v{tmp[4 * sl + 2 * i + 1]}" for i in range(2)]
            w = f"v{PREG + 4 * (2 * kp + nb) + i2}"
            ps = f"v{PSUM + nb}"
            nm = f"%[nm{nb}]"
            seqs = []
            for sc, t, u, wf in zip(ss, ts, us, ws):
                q = [Ins(f"v_fma_f32 {t}, -{sc}, %[c], {nm}", "valu", wr=[t], rd=[sc]),
                     Ins(f"v_med3_f32 {t}, {t}, 0, %[c7]", "valu", wr=[t], rd=[t]),
                     Ins(f"v_floor_f32 {u}, {t}", "valu", wr=[u], rd=[t]),
                     Ins(f"v_sub_f32 {wf}, {t}, {u}", "valu", wr=[wf], rd=[t, u]),
                     Ins(f"v_sub_f32_e64 {t}, %[c6], {u} clamp", "valu", wr=[t], rd=[u]),
                     Ins(f"v_mul_f32 {u}, 0xbfb8aa3b, {u}", "valu", wr=[u], rd=[u]),
                     Ins(f"v_exp_f32 {u}, {u}", "trans", wr=[u], rd=[u]),
                     Ins(f"v_mul_f32 {u}, {u}, {t}", "valu", wr=[u], rd=[u, t]),
                     Ins(f"v_mov_b32 {t}, %[sa{deg}]", "valu", wr=[t])]
                q += [Ins(f"v_fma_f32 {t}, {t}, {wf}, %[sa{j}]", "valu", wr=[t], rd=[t, wf])
                      for j in range(deg - 1, -1, -1)]
                q.append(Ins(f"v_mul_f32 {t}, {t}, {u}", "valu", wr=[t], rd=[t, u]))
                seqs.append(q)
            heads.append([x for pair in zip(*seqs) for x in pair])
            t0, t1 = ts
            tail = [Ins(f"v_cvt_pk_bf16_f32 {w}, {t0}, {t1}", "valu", wr=[w], rd=[t0, t1],
                        tag=("pf", kp))]
            if first[nb]:
                tail.append(Ins(f"v_add_f32 {ps}, {t0}, {t1}", "valu", wr=[ps], rd=[t0, t1]))
                first[nb] = False
            else:
                tail += [Ins(f"v_add_f32 {t0}, {t0}, {t1}", "valu", wr=[t0], rd=[t0, t1]),
                         Ins(f"v_add_f32 {ps}, {ps}, {t0}", "valu", wr=[ps], rd=[ps, t0])]
            tails.append(tail)
        # pair gp's sequence runs ahead of pair gp - 1's pack and sums
        out = list(heads[0])
        for gp in range(1, 32):
            out += heads[gp] + tails[gp - 1]
        out += tails[31]
        for nb in range(2):
            out.append(Ins(f"v_add_f32 %[lo{nb}], %[lo{nb}], v{PSUM + nb}", "valu",
                           rd=[f"v{PSUM + nb}"]))
        return out

    def exp2_stream(self):
        """Per score pair: scale-and-shift, exp2, pack (bf16, or fp8 for the
        8-bit P.V: the weights stay below 2^8, inside E4M3's range, so they
        are rounded without a scale), pair sum into
        this tile's partial row sum; at the end each partial sum joins the
        running row sum once. (Adding every exponential straight into the
        running sum loses the small terms once that sum is large: over
        millions of keys the row sum, and so the LSE, came out low.)
        int8 QK^T: a "full" step's scores are the floats K0 + s 2^-26 (see
        qk_mfmas) and the multiplier is 2^26 times the code-unit one, so the
        offset's shift takes K0 2^26 times it off as well (nmc)."""
        heads, tails = [], []
        first = {0: True, 1: True}
        for gp, (a, nb, r0) in enumerate(self.pairs()):
            s0 = f"v{self.s_reg(self.x, a, nb, r0)}"
            s1 = f"v{self.s_reg(self.x, a, nb, r0 + 1)}"
            t0 = f"v{TREG + 2 * (gp % 3)}"
            t1 = f"v{TREG + 2 * (gp % 3) + 1}"
            ps = f"v{PSUM + nb}"
            nm = f"%[nm{nb}]"
            cc = "%[ce]" if self.f8 else "%[c]"
            heads.append([
                Ins(f"v_fma_f32 {t0}, {s0}, {cc}, {nm}", "valu", wr=[t0], rd=[s0]),
                Ins(f"v_fma_f32 {t1}, {s1}, {cc}, {nm}", "valu", wr=[t1], rd=[s1]),
                Ins(f"v_exp_f32 {t0}, {t0}", "trans", wr=[t0], rd=[t0]),
                Ins(f"v_exp_f32 {t1}, {t1}", "trans", wr=[t1], rd=[t1]),
            ])
            tail = [self.pack(a, nb, r0, t0, t1)]
            if first[nb]:
                tail.append(Ins(f"v_add_f32 {ps}, {t0}, {t1}", "valu", wr=[ps], rd=[t0, t1]))
                first[nb] = False
            else:
                tail += [Ins(f"v_add_f32 {t0}, {t0}, {t1}", "valu", wr=[t0], rd=[t0, t1]),
                         Ins(f"v_add_f32 {ps}, {ps}, {t0}", "valu", wr=[ps], rd=[ps, t0])]
            tails.append(tail)
        # Pairs are software-pipelined by one: the scale-and-shift of pair
        # gp + 1 sits between the exponentials of pair gp and their first
        # reader, so no wait state is needed after a v_exp (the temporaries
        # rotate over three register pairs).
        out = list(heads[0])
        for gp in range(1, 32):
            out += heads[gp][:-2] + tails[gp - 1] + heads[gp][-2:]
        out += tails[31]
        for nb in range(2):
            out.append(Ins(f"v_add_f32 %[lo{nb}], %[lo{nb}], v{PSUM + nb}", "valu",
                           rd=[f"v{PSUM + nb}"]))
        return out

    def max_stream(self):
        """Row maxima of the new tile: query half nb over both key halves
        (int8 QK^T: maxima of the int32 scores, which order as the scaled
        scores do; the vote converts the two maxima)."""
        out = []
        first = {0: True, 1: True}
        for a in range(2):
            for nb in range(2):
                for i in range(8):
                    r0 = self.s_reg(self.y, a, nb, 2 * i)
                    s0, s1 = f"v{r0}", f"v{r0 + 1}"
                    tm = f"%[tm{nb}]"
                    mx, mx3 = ("v_max_i32", "v_max3_i32") if self.i8 else ("v_max_f32", "v_max3_f32")
                    if first[nb]:
                        out.append(Ins(f"{mx} {tm}, {s0}, {s1}", "valu", rd=[s0, s1], tag=("blk", a)))
                        first[nb] = False
                    else:
                        out.append(Ins(f"{mx3} {tm}, {tm}, {s0}, {s1}", "valu", rd=[s0, s1],
                                       tag=("blk", a)))
        return out

    def vote_stream(self):
        v = [f"v{VOTE + i}" for i in range(6)]
        pre = []
        if self.i8:
            # int8: the maxima of the scores' bits, K0 + tm 2^-26, less K0
            # (exact: same binade); the tile's multiplier carries the 2^26
            pre = [Ins("v_subrev_f32 %[tm0], 0.15915494, %[tm0]", "valu"),
                   Ins("v_subrev_f32 %[tm1], 0.15915494, %[tm1]", "valu")]
        if self.f8:
            # 8-bit scores are in code units: times q scale x k scale of the tile
            pre += [Ins("v_mul_f32 %[tm0], %[tm0], %[qa]", "valu"),
                    Ins("v_mul_f32 %[tm1], %[tm1], %[qa]", "valu")]
        return pre + [
            Ins(f"v_mov_b32 {v[0]}, %[tm0]", "valu", wr=[v[0]]),
            Ins(f"v_mov_b32 {v[1]}, %[tm0]", "valu", wr=[v[1]]),
            Ins(f"v_mov_b32 {v[2]}, %[tm1]", "valu", wr=[v[2]]),
            Ins(f"v_mov_b32 {v[3]}, %[tm1]", "valu", wr=[v[3]]),
            Ins(f"v_subrev_f32 {v[4]}, %[tau], %[mi0]", "valu", wr=[v[4]]),
            Ins(f"v_subrev_f32 {v[5]}, %[tau], %[mi1]", "valu", wr=[v[5]]),
            Ins(f"v_permlane32_swap_b32 {v[0]}, {v[1]}", "perm", wr=[v[0], v[1]], rd=[v[0], v[1]]),
            Ins(f"v_permlane32_swap_b32 {v[2]}, {v[3]}", "perm", wr=[v[2], v[3]], rd=[v[2], v[3]]),
            Ins(f"v_max_f32 {v[0]}, {v[0]}, {v[1]}", "valu", wr=[v[0]], rd=[v[0], v[1]]),
            Ins(f"v_max_f32 {v[2]}, {v[2]}, {v[3]}", "valu", wr=[v[2]], rd=[v[2], v[3]]),
            Ins(f"v_cmp_nlt_f32 %[k0], {v[0]}, {v[4]}", "valu", rd=[v[0], v[4]]),
            Ins(f"v_cmp_nlt_f32 %[k1], {v[2]}, {v[5]}", "valu", rd=[v[2], v[5]]),
            Ins("s_and_b64 %[k0], %[k0], %[val0]", "salu"),
            Ins("s_and_b64 %[k1], %[k1], %[val1]", "salu"),
            Ins("s_or_b64 %[keep], %[k0], %[k1]", "salu"),
            Ins("s_cmp_lg_u64 %[keep], 0", "salu"),
            Ins("s_cselect_b64 %[keep], -1, 0", "salu"),
            Ins("s_andn2_b64 %[k0], %[keep], %[rare]", "salu"),
            Ins(f"v_max_f32 {v[1]}, %[mi0], {v[0]}", "valu", wr=[v[1]], rd=[v[0]]),
            Ins(f"v_max_f32 {v[3]}, %[mi1], {v[2]}", "valu", wr=[v[3]], rd=[v[2]]),
            Ins(f"v_cndmask_b32 %[mo0], %[mi0], {v[1]}, %[k0]", "valu", rd=[v[1]]),
            Ins(f"v_cndmask_b32 %[mo1], %[mi1], {v[3]}, %[k0]", "valu", rd=[v[3]]),
            Ins(f"v_add_f32 {v[4]}, %[lazy], %[mr0]", "valu", wr=[v[4]]),
            Ins(f"v_add_f32 {v[5]}, %[lazy], %[mr1]", "valu", wr=[v[5]]),
            Ins(f"v_cmp_gt_f32 %[k0], %[mo0], {v[4]}", "valu", rd=[v[4]]),
            Ins(f"v_cmp_gt_f32 %[k1], %[mo1], {v[5]}", "valu", rd=[v[5]]),
            Ins("s_or_b64 %[grow], %[k0], %[k1]", "salu"),
        ]

    # ---- schedule ---------------------------------------------------------
    def build(self):
        """Phase A walks key half a = 0 then a = 1, k-steps inside, both
        query halves per k-step: the S blocks of key half 0 are final at the
        middle of phase A, so their row maxima start there; key half 1's
        follow early in phase B, then the vote. Vector work is pulled into
        the MFMA slots against a cycle budget; a PV key step first forces
        the exponentials it consumes."""
        seq = []
        exp_q = self.exp_stream() if self.pv else []
        max_q = (self.max_stream() + self.vote_stream()) if self.qk else []
        KS, MB = self.KS, self.MB
        qk_w = 2 if self.f8 else 1      # a 16-pass QK MFMA holds two 8-pass slots
        pv_slots = 4 * MB if self.v8 else 8 * MB   # 2 MB 16-pass or 8 MB 8-pass MFMAs
        n_slots = (4 * KS * qk_w if self.qk else 0) + (pv_slots if self.pv else 0)
        total_valu = sum(i.cost for i in exp_q) + sum(i.cost for i in max_q)
        budget = max(self.budget, total_valu / max(n_slots, 1))
        pos = {"exp": 0, "max": 0}
        done_half = set()   # key halves whose S blocks are final (plus margin)
        dma_q = self.dma_groups() if self.dma else []

        def mfma(ins):      # an MFMA, then the next tile-copy group if any
            seq.append(ins)
            if dma_q and len([x for x in seq if x.is_mfma]) >= 2:
                seq.extend(dma_q.pop(0))

        def max_ready(ins):
            return ins.tag is None or ins.tag[1] in done_half

        def pull(limit, use_max=True):
            used = 0.0
            while True:
                cand = None
                if pos["exp"] < len(exp_q):
                    cand = ("exp", exp_q[pos["exp"]])
                elif use_max and pos["max"] < len(max_q) and max_ready(max_q[pos["max"]]):
                    cand = ("max", max_q[pos["max"]])
                if cand is None or used + cand[1].cost > limit + 1e-9:
                    return used
                seq.append(cand[1])
                used += cand[1].cost
                pos[cand[0]] += 1

        def exp_needed(ks, kind="pf"):
            last = -1
            for i, ins in enumerate(exp_q):
                if ins.tag and ins.tag[0] == kind and ins.tag[1] <= ks:
                    last = i
            return last + 1

        if self.pv:
            if not self.loop:
                seq += [Ins("v_mov_b32 %[lo0], %[li0]", "valu"),
                        Ins("v_mov_b32 %[lo1], %[li1]", "valu")]
            if not self.v8:
                seq += self.v_addr()
        # phase A --------------------------------------------------------
        if self.qk:
            order = [(a, ks) for a in range(2) for ks in range(KS)]
            v8_after = {}
            if self.v8:
                for mb in range(MB):
                    mine = set(expand(self.vfrag8(mb)))
                    v8_after[mb] = max([n for n in range(len(order))
                                        if mine & set(expand(self.kfrag(n & 3)))], default=-1)
            seq += self.k_load(*order[0], 0)
            seq += self.k_load(*order[1], 1)
            if self.pv:
                pull(2 * budget, use_max=False)
            for n, (a, ks) in enumerate(order):
                j = n & 3
                for nb in range(2):
                    for ins in self.qk_mfmas(ks, a, nb, j):
                        mfma(ins)
                    if nb == 0 and n + 2 < len(order):
                        seq += self.k_load(*order[n + 2], (n + 2) & 3)
                    # V^T fragments of PV k-step 0: bf16, once the K fragments
                    # they overwrite are read; fp8, after key half 0's MFMAs.
                    # 8-bit P.V: each block's fragment right after the last
                    # MFMA that reads a K fragment in its registers (after
                    # the first MFMA when none does)
                    if self.v8 and self.pv:
                        due = [mb for mb in range(MB)
                               if (v8_after[mb] == n and nb == 1)
                               or (v8_after[mb] < 0 and n == 0 and nb == 0)]
                        if due:
                            seq += self.v_loads8(due)
                    elif not self.v8:
                        v0_at = KS if self.f8 else len(order) // 2 + 2
                        if nb == 0 and self.pv and n == v0_at:
                            seq += self.v_loads(0)
                    pull(budget * qk_w)
                # key half 0 final after its last k-step; its maxima wait two
                # more k-steps (four MFMAs) to clear the MFMA result latency
                if a == 0 and ks == KS - 1:
                    pass
                if n == KS + 1:
                    done_half.add(0)
            done_half.add(1)
        elif self.pv:
            seq += self.v_loads8(range(MB)) if self.v8 else self.v_loads(0)

        # phase B --------------------------------------------------------
        if self.pv and self.v8:
            # one 16-pass MFMA per (d block, query half); a query half's
            # probabilities must all be packed before its first MFMA
            for nb in range(2):
                need = exp_needed(nb, "pf8")
                while pos["exp"] < need:
                    seq.append(exp_q[pos["exp"]])
                    pos["exp"] += 1
                for mb in range(MB):
                    mfma(self.pv8_mfma(mb, nb))
                    pull(2 * budget)
        elif self.pv:
            for ks in range(4):
                need = exp_needed(ks)
                while pos["exp"] < need:
                    seq.append(exp_q[pos["exp"]])
                    pos["exp"] += 1
                for i in range(2 * MB):
                    mb, nb = i >> 1, i & 1
                    mfma(self.pv_mfma(ks, mb, nb))
                    if i == 0 and ks + 1 < 4:
                        seq += self.v_loads(ks + 1)
                    pull(budget)
        # leftovers
        while dma_q:
            seq.extend(dma_q.pop(0))
        while pos["exp"] < len(exp_q):
            seq.append(exp_q[pos["exp"]])
            pos["exp"] += 1
        while pos["max"] < len(max_q):
            seq.append(max_q[pos["max"]])
            pos["max"] += 1
        self.seq = seq
        return self

    # ---- hazards --------------------------------------------------------
    def fix_hazards(self):
        out = []          # list of (text, slots)
        last_w = {}       # reg -> (index in out, kind)
        last_mfma_read = {}  # reg -> index in out
        lds_seq = []      # out-index of each lds op, in issue order
        lds_of_reg = {}   # reg -> position in lds_seq of its pending load
        waited = 0        # lds ops known complete (prefix of lds_seq)
        pos = []          # cumulative wait states at each out entry

        def slots_since(idx):
            return pos[-1] - pos[idx] if out else 0

        def emit(text, slots=1):
            out.append(text)
            pos.append((pos[-1] if pos else 0) + slots)

        for ins in self.seq:
            # outstanding loads feeding this instruction
            need_lds = -1
            for r in ins.rd:
                if r in lds_of_reg and lds_of_reg[r] >= waited:
                    need_lds = max(need_lds, lds_of_reg[r])
            # a load overwriting a fragment still to be read by an MFMA
            if ins.kind == "lds":
                for r in ins.wr:
                    if r in last_mfma_read:
                        ridx, rkind = last_mfma_read[r]
                        wait = NOP_MFMA16_READ_LOAD if rkind == "mfma16" else NOP_MFMA_READ_LOAD
                        gap = wait - slots_since(ridx)
                        if gap > 0:
                            emit(f"s_nop {gap - 1}", gap)
            if need_lds >= 0:
                cnt = len(lds_seq) - 1 - need_lds
                emit(f"s_waitcnt lgkmcnt({cnt})")
                waited = need_lds + 1
            need = 0
            for r in ins.rd:
                if r not in last_w:
                    continue
                widx, wkind = last_w[r]
                mwait = NOP_MFMA16_VALU if wkind == "mfma16" else NOP_MFMA_VALU
                if wkind in ("mfma", "mfma16") and ins.kind in ("valu", "trans"):
                    need = max(need, mwait - slots_since(widx))
                elif wkind in ("valu", "trans") and ins.kind in ("mfma", "mfma16"):
                    need = max(need, NOP_VALU_MFMA - slots_since(widx))
                elif wkind == "trans" and ins.kind in ("valu", "trans", "perm"):
                    need = max(need, NOP_TRANS_VALU - slots_since(widx))
                elif wkind in ("valu", "perm") and ins.kind == "perm":
                    need = max(need, NOP_VALU_PERM - slots_since(widx))
                elif wkind == "perm" and ins.kind in ("valu", "perm"):
                    need = max(need, 1 - slots_since(widx))
                if wkind in ("mfma", "mfma16") and ins.kind == "perm":
                    need = max(need, mwait - slots_since(widx))
            while need > 0:
                n = min(need, 8)
                emit(f"s_nop {n - 1}", n)
                need -= n
            emit(ins.text)
            idx = len(out) - 1
            if ins.kind == "lds":
                lds_seq.append(idx)
                for r in ins.wr:
                    lds_of_reg[r] = len(lds_seq) - 1
            for r in ins.wr:
                last_w[r] = (idx, ins.kind)
            if ins.kind in ("mfma", "mfma16"):
                for r in ins.rd:
                    last_mfma_read[r] = (idx, ins.kind)
        if len(lds_seq) > waited:
            emit("s_waitcnt lgkmcnt(0)")
        self.out = out
        return self

    def estimate(self):
        """Rough cycle estimate: each MFMA slot max(32, vector work + 8)."""
        t = 0.0
        cur = None
        slot = 32.0
        for ins in self.seq:
            if ins.is_mfma:
                if cur is not None:
                    t += max(slot, cur + 8.0)
                cur = 0.0
                slot = 64.0 if ins.kind == "mfma16" else 32.0
            elif cur is not None:
                cur += ins.cost
            else:
                t += ins.cost
        if cur is not None:
            t += max(slot, cur + 8.0)
        return t

    # ---- C++ ------------------------------------------------------------
    def cxx(self):
        MB = self.MB
        name = f"step_{self.variant}_{self.x if self.pv else ''}{self.y if self.qk else ''}"
        args, outs, ins_ = [], [], []
        if self.qk:
            args += ["float (&tm)[2]", "uint32_t kb0", "float (&m)[2]", "const float (&mref)[2]",
                     "float tau", "float lazy", "const uint64_t (&val)[2]", "uint64_t rare",
                     "uint64_t& keep", "uint64_t& grow"]
            outs += ['[tm0] "=&v"(tm[0])', '[tm1] "=&v"(tm[1])', '[mo0] "=&v"(mo[0])',
                     '[mo1] "=&v"(mo[1])', '[keep] "=&s"(keep)', '[grow] "=&s"(grow)',
                     '[k0] "=&s"(k0)', '[k1] "=&s"(k1)']
            ins_ += ['[kb0] "v"(kb0)', '[mi0] "v"(m[0])', '[mi1] "v"(m[1])', '[mr0] "v"(mref[0])',
                     '[mr1] "v"(mref[1])', '[tau] "s"(tau)', '[lazy] "v"(lazy)', '[val0] "s"(val[0])',
                     '[val1] "s"(val[1])', '[rare] "s"(rare)']
        if self.pv:
            args += ["float (&lsum)[2]", "const float (&nmc)[2]", "float c", "uint32_t vb0",
                     "uint32_t vb1"]
            outs += ['[lo0] "=&v"(lo[0])', '[lo1] "=&v"(lo[1])']
            ins_ += ['[li0] "v"(lsum[0])', '[li1] "v"(lsum[1])', '[nm0] "v"(nmc[0])', '[nm1] "v"(nmc[1])', '[c] "s"(c)', '[vb0] "v"(vb0)',
                     '[vb1] "v"(vb1)']
        clob = [f"v{r}" for r in range(PSUM, 128)]
        if self.qk:
            clob += [f"v{VOTE + i}" for i in range(6)] + ["scc"]
            clob += [f"v{r}" for r in range(SBUF[self.y], SBUF[self.y] + 64)]
        if self.pv:
            clob += [f"a{r}" for r in range(OB, OB + 32 * MB)]
        what = {"full": f"S^T of the next tile into buffer {self.y}, exp and PV of the "
                        f"current tile from buffer {self.x}",
                "qk": f"S^T of the next tile into buffer {self.y} and its row maxima",
                "pv": f"exp and PV of the current tile from buffer {self.x}"}[self.variant]
        head = (f"// {self.variant} step, d = {self.d}: {what} "
                f"({len(self.out)} instructions, ~{self.estimate():.0f} cycles)")
        # m and lsum are read and rewritten: they go in as inputs and come out
        # through early-clobber outputs, so that no other input (say mref,
        # which can hold the same value) shares their registers
        pre, post = [], []
        if self.qk:
            pre += ["uint64_t k0, k1;", "float mo[2];"]
            post += ["m[0] = mo[0];", "m[1] = mo[1];"]
        if self.pv:
            pre += ["float lo[2];"]
            post += ["lsum[0] = lo[0];", "lsum[1] = lo[1];"]
        return asm_function(head, name, args, self.out, outs, ins_, clob, pre, post)


def asm_function(head, name, args, body, outs, ins_, clob, pre=(), post=()):
    text = "\n".join(f'      "{t}\\n\\t"' for t in body)
    clob_s = ", ".join(f'"{c}"' for c in clob + ["memory"])
    return "\n".join([
        head,
        f"__device__ __forceinline__ void {name}({', '.join(args)}) {{",
        *[f"  {p}" for p in pre],
        "  asm volatile(",
        text,
        "      : " + ",\n        ".join(outs),
        "      : " + ",\n        ".join(ins_),
        "      : " + clob_s + ");",
        *[f"  {p}" for p in post],
        "}"])


def helpers_cxx(d, f8=False):
    """Blocks outside the key loop that touch the fixed registers."""
    MB, KS = d // 32, (d // 64 if f8 else d // 16)
    QB = OB + 32 * MB
    row_bytes = d if f8 else 2 * d      # Q rows in LDS
    o_regs = [f"a{r}" for r in range(OB, OB + 32 * MB)]
    parts = []

    # zero O
    body = [f"v_accvgpr_write_b32 {r}, 0" for r in o_regs]
    parts.append(asm_function(f"// O^T accumulators a[{OB}:{OB + 32 * MB - 1}] = 0",
                              "zero_o", [], body, [], [], o_regs))

    # Q^T fragments into AGPRs
    body = []
    if f8:
        # fp8 rows of d bytes: per k-step (64 d) and query half, 32 bytes per
        # lane from chunks at qb0 ^ 64 ks and that ^ 16
        for ks in range(KS):
            for jj in range(2):
                x = 64 * ks + 16 * jj
                adr = "%[qb0]" if x == 0 else f"v{KADR + jj}"
                if x:
                    body.append(f"v_xor_b32 {adr}, {x}, %[qb0]")
                for nb in range(2):
                    lo = QB + 16 * ks + 8 * nb + 4 * jj
                    body.append(f"ds_read_b128 a[{lo}:{lo + 3}], {adr} offset:{nb * 32 * row_bytes}")
            body.append("s_waitcnt lgkmcnt(0)")
        nq = 16 * KS
    else:
        for ks in range(KS):
            adr = "%[qb0]" if ks == 0 else f"v{KADR + (ks & 1)}"
            if ks:
                body.append(f"v_xor_b32 {adr}, {32 * ks}, %[qb0]")
            for nb in range(2):
                lo = QB + 8 * ks + 4 * nb
                body.append(f"ds_read_b128 a[{lo}:{lo + 3}], {adr} offset:{nb * 32 * row_bytes}")
        body.append("s_waitcnt lgkmcnt(0)")
        nq = 8 * KS
    parts.append(asm_function(
        f"// Q^T fragments of the wave's 64 queries into a[{QB}:{QB + nq - 1}]; qb0 is the "
        "k-step 0 fragment address",
        "load_q", ["uint32_t qb0"], body, [], ['[qb0] "v"(qb0)'],
        [f"a{r}" for r in range(QB, QB + nq)] + [f"v{KADR}", f"v{KADR + 1}"]))

    # rescale O: query half nb by alpha_nb (blocks (mb, nb))
    body = []
    for nb in range(2):
        for mb in range(MB):
            lo = OB + 16 * (2 * mb + nb)
            for r in range(lo, lo + 16, 4):
                for k in range(4):
                    body.append(f"v_accvgpr_read_b32 v{TREG + k}, a{r + k}")
                body.append("s_nop 1")
                for k in range(4):
                    body.append(f"v_mul_f32 v{TREG + k}, v{TREG + k}, %[al{nb}]")
                body.append("s_nop 1")
                for k in range(4):
                    body.append(f"v_accvgpr_write_b32 a{r + k}, v{TREG + k}")
    body.append("s_nop 4")
    parts.append(asm_function(
        "// O^T query half nb *= alpha_nb (the running-max rescale); the caller drains the MFMAs",
        "rescale_o", ["float al0", "float al1"], body, [], ['[al0] "v"(al0)', '[al1] "v"(al1)'],
        o_regs + [f"v{TREG + k}" for k in range(4)]))

    # read one O block into 16 floats
    for mb in range(MB):
        for nb in range(2):
            lo = OB + 16 * (2 * mb + nb)
            body = [f"v_accvgpr_read_b32 %[o{r}], a{lo + r}" for r in range(16)]
            outs = [f'[o{r}] "=v"(o[{r}])' for r in range(16)]
            parts.append(asm_function(f"// O^T block (mb {mb}, nb {nb}) -> 16 floats",
                                      f"read_o_{mb}{nb}", ["float (&o)[16]"], body, outs, [], []))

    # mask the scores of buffer Y and recompute its row maxima
    for y in ("A", "B"):
        body = [f"v_mov_b32 v{TREG}, 0xff800000"]
        for a in range(2):
            for nb in range(2):
                for r in range(16):
                    key = 32 * a + 8 * (r >> 2) + (r & 3)
                    reg = SBUF[y] + 16 * (2 * a + nb) + r
                    body.append(f"v_cmp_gt_i32 vcc, {key}, %[lim{nb}]")
                    body.append(f"v_cndmask_b32 v{reg}, v{reg}, v{TREG}, vcc")
        for nb in range(2):
            regs = [SBUF[y] + 16 * (2 * a + nb) + r for a in range(2) for r in range(16)]
            body.append(f"v_max_f32 %[tm{nb}], v{regs[0]}, v{regs[1]}")
            for i in range(2, 32, 2):
                body.append(f"v_max3_f32 %[tm{nb}], %[tm{nb}], v{regs[i]}, v{regs[i + 1]}")
        parts.append(asm_function(
            f"// Scores of buffer {y}: key offset k (within the tile, from this lane's first key) "
            "is masked to -inf when k > lim_nb; row maxima recomputed",
            f"mask_{y}", ["const int (&lim)[2]", "float (&tm)[2]"], body,
            ['[tm0] "=&v"(tm[0])', '[tm1] "=&v"(tm[1])'],
            ['[lim0] "v"(lim[0])', '[lim1] "v"(lim[1])'],
            [f"v{r}" for r in range(SBUF[y], SBUF[y] + 64)] + [f"v{TREG}", "vcc"]))
    return parts


# ---------------------------------------------------------------------------
# The whole key loop of one wave as one asm block.
#
# Between the generated steps the loop also needs: the workgroup barrier and
# the K/V tile copies (buffer_load ... lds), the choice of step variant from
# the vote, the lazy rescale, the masked re-vote of the causal-diagonal or
# ragged tile, and the skip-mask byte. Written in C++ that glue costs about
# as much as a quarter of a step (branches and register copies, at ~4 cycles
# per instruction for a lone wave), so it is emitted here as scalar control
# flow around the step blocks. Every block below starts with no hazard
# pending and leaves none behind (each ends with its LDS reads waited and
# its MFMA results read after the required wait states).
# ---------------------------------------------------------------------------

def _rename(lines, mapping):
    out = []
    for t in lines:
        for a, b in mapping.items():
            t = t.replace(a, b)
        out.append(t)
    return out


QA = {"A": "%[qa0]", "B": "%[qa1]"}   # fp8: q scale x k scale of the tile in buffer A / B


def _step_lines(d, variant, x, y, budget, dma=True, f8=False, sas=0, v8=False, i8=False):
    st = Step(d, variant, x, y, budget, loop=True, dma=dma, f8=f8, sas=sas,
              v8=v8, i8=i8).build().fix_hazards()
    return _rename(st.out, {"%[mi0]": "%[m0]", "%[mi1]": "%[m1]", "%[mo0]": "%[m0]",
                            "%[mo1]": "%[m1]", "%[lo0]": "%[ls0]", "%[lo1]": "%[ls1]",
                            "%[qa]": QA[y]})


def _vote_again_lines(f8=False, y="A"):
    """The vote once more on masked maxima (tm recomputed), m always updated
    when kept."""
    body = []
    for ins in Step(128, "qk", "A", "A", 0, loop=True, f8=f8).vote_stream():
        body.append(ins.text.replace("s_andn2_b64 %[k0], %[keep], %[rare]", "s_mov_b64 %[k0], %[keep]"))
    # vote temporaries: a VALU write feeds v_permlane32_swap after 4 instructions
    return _rename(body, {"%[mi0]": "%[m0]", "%[mi1]": "%[m1]", "%[mo0]": "%[m0]",
                          "%[mo1]": "%[m1]", "%[qa]": QA[y]})


def _mask_lines(d, y):
    body = [f"v_mov_b32 v{TREG}, 0xff800000"]
    for a in range(2):
        for nb in range(2):
            for r in range(16):
                key = 32 * a + 8 * (r >> 2) + (r & 3)
                reg = SBUF[y] + 16 * (2 * a + nb) + r
                body.append(f"v_cmp_gt_i32 vcc, {key}, %[lim{nb}]")
                body.append(f"v_cndmask_b32 v{reg}, v{reg}, v{TREG}, vcc")
    for nb in range(2):
        regs = [SBUF[y] + 16 * (2 * a + nb) + r for a in range(2) for r in range(16)]
        body.append(f"v_max_f32 %[tm{nb}], v{regs[0]}, v{regs[1]}")
        for i in range(2, 32, 2):
            body.append(f"v_max3_f32 %[tm{nb}], %[tm{nb}], v{regs[i]}, v{regs[i + 1]}")
    return body


def _sas_lines(x, t, u, w, deg):
    """x := SAS(x) for x in raw units times %[c] = 1 / sqrt(d) already (the
    sequence of Step.sas_stream, hazards written out)."""
    return [f"v_med3_f32 {x}, {x}, 0, %[c7]",
            f"v_floor_f32 {u}, {x}",
            f"v_sub_f32 {w}, {x}, {u}",
            f"v_sub_f32_e64 {t}, %[c6], {u} clamp",
            f"v_mul_f32 {u}, 0xbfb8aa3b, {u}",
            f"v_exp_f32 {u}, {u}", "s_nop 0",
            f"v_mul_f32 {u}, {u}, {t}",
            f"v_mov_b32 {x}, %[sa{deg}]"] + [
            f"v_fma_f32 {x}, {x}, {w}, %[sa{j}]" for j in range(deg - 1, -1, -1)] + [
            f"v_mul_f32 {x}, {x}, {u}"]


def _rescale_lines(d, sas=0):
    """alpha = m > mref ? exp2((mref - m) c) : 1 (SAS: SAS((m - mref) c),
    c = 1 / sqrt(d)); lsum *= alpha; mref = max; O half nb *= alpha_nb.
    Drains the MFMAs first."""
    MB = d // 32
    al = ["v52", "v53"]
    body = ["s_nop 7", "s_nop 7", "s_nop 7"]
    for nb in range(2):
        if sas:
            body += [f"v_sub_f32 {al[nb]}, %[m{nb}], %[mr{nb}]",
                     f"v_mul_f32 {al[nb]}, %[c], {al[nb]}"]
            body += _sas_lines(al[nb], f"v{TREG}", f"v{TREG + 1}", f"v{TREG + 2}", sas)
        else:
            body += [f"v_sub_f32 {al[nb]}, %[mr{nb}], %[m{nb}]",
                     f"v_mul_f32 {al[nb]}, {al[nb]}, %[c]",
                     f"v_exp_f32 {al[nb]}, {al[nb]}"]
        body += [f"v_cmp_gt_f32 vcc, %[m{nb}], %[mr{nb}]",
                 f"v_cndmask_b32 {al[nb]}, 1.0, {al[nb]}, vcc",
                 f"v_mul_f32 %[ls{nb}], %[ls{nb}], {al[nb]}",
                 f"v_max_f32 %[mr{nb}], %[mr{nb}], %[m{nb}]"]
    for nb in range(2):
        for mb in range(MB):
            lo = OB + 16 * (2 * mb + nb)
            for r in range(lo, lo + 16, 4):
                body += [f"v_accvgpr_read_b32 v{TREG + k}, a{r + k}" for k in range(4)]
                body.append("s_nop 1")
                body += [f"v_mul_f32 v{TREG + k}, v{TREG + k}, {al[nb]}" for k in range(4)]
                body.append("s_nop 1")
                body += [f"v_accvgpr_write_b32 a{r + k}, v{TREG + k}" for k in range(4)]
    body += ["s_nop 4", "s_mov_b64 %[grow], 0"]
    return body


LOOP_ARGS = """// Operands of the key loop. Scalars are wave-uniform (SGPRs); krs / vrs are
// raw buffer descriptors of the K and V head; mask_row is the skip-mask row
// of this wave's query tile (0 when no mask is written).{f8doc}
struct LoopArgs {{
  uint32_t frag, tr0, tr1, gk[{ipwk}], gv[{ipwv}];
  int lim_base[2];
  float lazy;
  int nkb_wg, nkb_w, qb, N;
  float tau, c;
  u32x4 krs, vrs;
  uint32_t wl, smem;
  uint64_t mask_row;
  uint64_t val[2];{f8fields}
}};
"""
LOOP_ARGS_F8_DOC = """
// fp8 QK^T: ksp points at the K tile scales of this KV head (one fp32 per
// 64-key tile), sqv is this wave's Q tile scale (int8: times 2^26, the
// unit of the scores as the loop reads them), nkbm1 the last key tile,
// wlv the wave's LDS base for V tile copies (wl: for K)."""
LOOP_ARGS_SAS_DOC = """
// SAS exponential: c is 1 / sqrt(d) (not log2(e) / sqrt(d)), lazy is 0 (the
// reference max is always the running max), sa the polynomial's
// coefficients a0 .. a3 (a3 unused at degree 2), c6 = 6, c7 = 7."""
LOOP_ARGS_SAS_FIELDS = """
  float sa[4];
  float c6, c7;"""
LOOP_ARGS_V8_DOC = """
// 8-bit P.V: V tiles are E4M3 code blocks (d rows of 64 bytes); wlv is the
// wave's LDS base for their copies (wl: for K)."""
LOOP_ARGS_V8_FIELDS = """
  uint32_t wlv;"""
LOOP_ARGS_F8_FIELDS = """
  uint64_t ksp;
  float sqv;
  int nkbm1;
  uint32_t wlv;"""


def loop_cxx(d, causal, budget, f8=False, sas=0, v8=False, i8=False):
    MB = d // 32
    row_bytes = 2 * d                        # V rows (bf16)
    krow = d if f8 else 2 * d                # K rows: fp8 codes or bf16
    tile_k = 64 * krow
    tile_v = 64 * d if v8 else 64 * row_bytes   # 8-bit P.V: d rows of 64 codes
    stage_bytes = tile_k + tile_v
    ipwk = tile_k // 1024 // 4               # copy instructions per wave and tile
    ipwv = tile_v // 1024 // 4
    L = []

    def lab(name):
        return f".L{name}_%="

    # Tile t lives in slot t % 5 (five K/V slots; slots 3-4 stage the Q tiles
    # before the loop).
    def slot_base(dst, t_off):
        return [f"s_add_u32 {dst}, %[kb], {t_off}" if t_off else f"s_mov_b32 {dst}, %[kb]",
                f"s_mul_hi_u32 %[t3], {dst}, 0xcccccccd", "s_lshr_b32 %[t3], %[t3], 2",
                "s_mul_i32 %[t3], %[t3], 5", f"s_sub_u32 {dst}, {dst}, %[t3]",
                f"s_mul_i32 {dst}, {dst}, {stage_bytes}", f"s_add_u32 {dst}, {dst}, %[smem]"]

    def kaddr():   # %[kb0] = K fragment base of tile kb + 1
        return slot_base("%[t0]", 1) + [
                "v_add_u32 %[kb0], %[t0], %[frag]"]

    def vaddr():   # %[vb0/1] = V^T read bases of tile kb
        return slot_base("%[t0]", 0) + [f"s_add_u32 %[t0], %[t0], {tile_k}",
                "v_add_u32 %[vb0], %[t0], %[tr0]", "v_add_u32 %[vb1], %[t0], %[tr1]"]

    def nmc(x, full=False):
        if sas:  # mref / sqrt(d), the exponent input's offset
            return ["v_mul_f32 %[nm0], %[mr0], %[c]", "v_mul_f32 %[nm1], %[mr1], %[c]"]
        out = ["v_mul_f32 %[nm0], %[mr0], %[c]", "v_mul_f32 %[nm1], %[mr1], %[c]",
               "v_xor_b32 %[nm0], 0x80000000, %[nm0]", "v_xor_b32 %[nm1], 0x80000000, %[nm1]"]
        if f8:
            # the exponent input's multiplier for tile kb's code-unit scores
            out.append(f"v_mul_f32 %[ce], {QA[x]}, %[c]")
        if i8 and full:
            # a "full" step's scores are K0 + s 2^-26 (exp2_stream): the
            # offset also takes off K0 times the multiplier
            out += ["v_fma_f32 %[nm0], -%[ce], 0.15915494, %[nm0]",
                    "v_fma_f32 %[nm1], -%[ce], 0.15915494, %[nm1]"]
        return out

    def rare(kbn):  # %[rare] = all ones when tile kbn needs the mask
        out = [f"s_lshl_b32 %[t3], {kbn}, 6", "s_add_u32 %[t3], %[t3], 64",
               "s_cmp_gt_i32 %[t3], %[N]", "s_cselect_b64 %[rare], -1, 0"]
        if causal:
            out += [f"s_cmp_eq_u32 {kbn}, %[qb]", "s_cselect_b64 %[k0], -1, 0",
                    "s_or_b64 %[rare], %[rare], %[k0]"]
        return out

    def after_vote(kbn, y, tag):  # masked re-vote if needed, then the mask byte
        out = []
        if i8:
            # int8: the wave's last tile goes to a "pv" step (and, when it is
            # the causal diagonal or the ragged end, through the masked
            # re-vote) with the scores s 2^-26: K0 comes off each in place
            # (exact), and the multiplier's 2^26 restores s. Every other
            # tile's scores stay K0 + s 2^-26 for the next "full" step.
            regs = [SBUF[y] + 16 * (2 * a + nb) + r for a in range(2) for nb in range(2)
                    for r in range(16)]
            out += [f"s_add_u32 %[t3], {kbn}, 1", "s_cmp_eq_u32 %[t3], %[nkbw]",
                    f"s_cbranch_scc0 {lab('nc' + tag)}"]
            out += [f"v_subrev_f32 v{r}, 0.15915494, v{r}" for r in regs]
            out += [f"{lab('nc' + tag)}:"]
        out += ["s_cmp_lg_u64 %[rare], 0", f"s_cbranch_scc0 {lab('nm' + tag)}",
               f"s_lshl_b32 %[t0], {kbn}, 6",
               "v_subrev_u32 %[lim0], %[t0], %[L0]", "v_subrev_u32 %[lim1], %[t0], %[L1]"]
        out += _mask_lines(d, y) + _vote_again_lines(f8, y)
        # skip-mask byte of tile kbn (0 kept, 1 skipped), written by lane 0
        out += [f"{lab('nm' + tag)}:",
                "s_cmp_lg_u64 %[mptr], 0", f"s_cbranch_scc0 {lab('ns' + tag)}",
                "s_cmp_lg_u64 %[keep], 0", "s_cselect_b32 %[t0], 0, 1",
                "v_mov_b32 %[vt], %[t0]", f"v_mov_b32 %[vz], {kbn}",
                "s_mov_b64 %[sx], exec", "s_mov_b64 exec, 1",
                "global_store_byte %[vz], %[vt], %[mptr]",
                "s_mov_b64 exec, %[sx]",
                f"{lab('ns' + tag)}:"]
        return out

    def dma_target():
        # %[t1] = byte offset of tile kb + 3, %[t2] = this wave's LDS base for
        # it. Its slot held tile kb - 2, which every wave finished before the
        # barrier at the top of this trip; a tile past the end only wastes
        # the copy (zero-filled past N). fp8: K and V tiles differ in size,
        # %[t4] / %[t5] are the V tile's offset and LDS base.
        out = slot_base("%[t2]", 3) + ["s_sub_u32 %[t2], %[t2], %[smem]"]
        if f8 or v8:
            out += ["s_add_u32 %[t5], %[t2], %[wlv]",
                    "s_add_u32 %[t4], %[kb], 3", f"s_mul_i32 %[t4], %[t4], {tile_v}"]
        out += ["s_add_u32 %[t2], %[t2], %[wl]",
                "s_add_u32 %[t1], %[kb], 3", f"s_mul_i32 %[t1], %[t1], {tile_k}"]
        return out

    def dma_alone():
        out = []
        for g in Step(d, "qk", "A", "A", 0, loop=True, dma=True, f8=f8, v8=v8).dma_groups():
            out += [i.text for i in g]
        return out

    def kscale_next(y):
        # fp8: the scale of tile kb + 1 (loaded a trip ago) into its buffer's
        # A = q scale x k scale, and the load of tile kb + 3's (same buffer
        # parity). Every LDS read is complete here, so lgkmcnt(0) only waits
        # for that scalar load; an SMEM load in flight during the steps only
        # makes their LDS waits stricter.
        sk = "%[sk0]" if y == "A" else "%[sk1]"
        return ["s_waitcnt lgkmcnt(0)",
                f"v_mul_f32 {QA[y]}, %[sqv], {sk}",
                "s_add_u32 %[t3], %[kb], 3", "s_min_u32 %[t3], %[t3], %[nkbm1]",
                "s_lshl_b32 %[t3], %[t3], 2", "s_nop 0",
                f"s_load_dword {sk}, %[ksp], %[t3]"]

    # -- init ------------------------------------------------------------
    L += ["v_mov_b32 %[m0], 0xff800000", "v_mov_b32 %[m1], 0xff800000",
          "v_mov_b32 %[mr0], 0xff800000", "v_mov_b32 %[mr1], 0xff800000",
          "v_mov_b32 %[ls0], 0", "v_mov_b32 %[ls1], 0",
          "s_mov_b32 %[kb], 0", "s_mov_b64 %[keep], 0", "s_mov_b64 %[grow], 0"]
    if f8:
        # scales of tiles 0 and 1; tile 0's A; then the load of tile 2's
        L += ["s_load_dword %[sk0], %[ksp], 0x0",
              "s_min_u32 %[t3], %[nkbm1], 1", "s_lshl_b32 %[t3], %[t3], 2",
              "s_load_dword %[sk1], %[ksp], %[t3]",
              "s_waitcnt lgkmcnt(0)",
              "v_mul_f32 %[qa0], %[sqv], %[sk0]",
              "s_min_u32 %[t3], %[nkbm1], 2", "s_lshl_b32 %[t3], %[t3], 2", "s_nop 0",
              "s_load_dword %[sk0], %[ksp], %[t3]"]
    # tile 0 scored into buffer A and voted on
    L += ["s_cmp_gt_i32 %[nkbw], 0", f"s_cbranch_scc0 {lab('loop')}"]
    L += ["s_mov_b32 %[t0], %[smem]", "v_add_u32 %[kb0], %[t0], %[frag]"]
    L += rare("0")
    L += _step_lines(d, "qk", "A", "A", budget, dma=False, f8=f8, v8=v8, i8=i8)
    L += after_vote("0", "A", "p0")
    L += [f"{lab('loop')}:"]
    for x, y in (("A", "B"), ("B", "A")):
        t = x + y
        # the copies of tile kb + 3 ride inside whichever step this wave runs
        if x == "A":
            # top of a trip (two tiles): every copy issued so far has landed
            # (tiles kb + 1, kb + 2), and every wave is past the previous
            # trip, so the slots of tiles kb - 2, kb - 1 are free
            L += ["s_waitcnt vmcnt(0)", "s_barrier"]
        L += dma_target() + [f"{lab('cp' + t)}:"]
        if f8:
            L += kscale_next(y)
        L += ["s_add_u32 %[t0], %[kb], 1", "s_cmp_lt_i32 %[t0], %[nkbw]",
              f"s_cbranch_scc0 {lab('last' + t)}"]
        L += kaddr() + ["s_add_u32 %[t0], %[kb], 1"] + rare("%[t0]")
        L += ["s_cmp_lg_u64 %[keep], 0", f"s_cbranch_scc0 {lab('skip' + t)}",
              "s_cmp_lg_u64 %[grow], 0", f"s_cbranch_scc0 {lab('nr' + t)}"]
        L += _rescale_lines(d, sas)
        L += [f"{lab('nr' + t)}:"] + nmc(x, full=True) + vaddr()
        L += _step_lines(d, "full", x, y, budget, f8=f8, sas=sas, v8=v8, i8=i8)
        L += [f"s_branch {lab('voted' + t)}", f"{lab('skip' + t)}:"]
        L += _step_lines(d, "qk", y, y, budget, f8=f8, v8=v8, i8=i8)
        L += [f"{lab('voted' + t)}:", "s_add_u32 %[t1], %[kb], 1"]
        L += after_vote("%[t1]", y, t)
        L += [f"s_branch {lab('end' + t)}",
              f"{lab('last' + t)}:", "s_cmp_eq_u32 %[t0], %[nkbw]", f"s_cbranch_scc0 {lab('idle' + t)}",
              "s_cmp_lg_u64 %[keep], 0", f"s_cbranch_scc0 {lab('idle' + t)}",
              "s_cmp_lg_u64 %[grow], 0", f"s_cbranch_scc0 {lab('nrl' + t)}"]
        L += _rescale_lines(d, sas)
        L += [f"{lab('nrl' + t)}:"] + nmc(x) + vaddr()
        L += _step_lines(d, "pv", x, x, budget, f8=f8, sas=sas, v8=v8)
        L += [f"s_branch {lab('ld' + t)}", f"{lab('idle' + t)}:"]
        L += dma_alone()
        L += [f"{lab('ld' + t)}:", "s_mov_b64 %[keep], 0",
              f"{lab('end' + t)}:",
              "s_add_u32 %[kb], %[kb], 1",
              "s_cmp_lt_i32 %[kb], %[nkbwg]", f"s_cbranch_scc0 {lab('done')}"]
    L += [f"s_branch {lab('loop')}", f"{lab('done')}:", "s_waitcnt vmcnt(0)"]
    if f8:
        L += ["s_waitcnt lgkmcnt(0)"]     # no scalar load may land after the block


    outs = ['[m0] "=&v"(m[0])', '[m1] "=&v"(m[1])', '[mr0] "=&v"(mref[0])', '[mr1] "=&v"(mref[1])',
            '[ls0] "=&v"(lsum[0])', '[ls1] "=&v"(lsum[1])',
            '[tm0] "=&v"(vtmp[0])', '[tm1] "=&v"(vtmp[1])', '[kb0] "=&v"(vtmp[2])',
            '[vb0] "=&v"(vtmp[3])', '[vb1] "=&v"(vtmp[4])', '[nm0] "=&v"(vtmp[5])',
            '[nm1] "=&v"(vtmp[6])', '[lim0] "=&v"(vtmp[7])', '[lim1] "=&v"(vtmp[8])',
            '[vt] "=&v"(vtmp[9])', '[vz] "=&v"(vtmp[10])',
            '[kb] "=&s"(s32[0])', '[t0] "=&s"(s32[4])', '[t1] "=&s"(s32[5])',
            '[t2] "=&s"(s32[6])', '[t3] "=&s"(s32[7])',
            '[keep] "=&s"(s64[0])', '[grow] "=&s"(s64[1])', '[k0] "=&s"(s64[2])',
            '[k1] "=&s"(s64[3])', '[rare] "=&s"(s64[4])', '[sx] "=&s"(s64[5])']
    ins_ = ['[frag] "v"(a.frag)', '[tr0] "v"(a.tr0)', '[tr1] "v"(a.tr1)',
            '[L0] "v"(a.lim_base[0])', '[L1] "v"(a.lim_base[1])', '[lazy] "v"(a.lazy)']
    ins_ += [f'[gk{i}] "v"(a.gk[{i}])' for i in range(ipwk)]
    ins_ += [f'[gv{i}] "v"(a.gv[{i}])' for i in range(ipwv)]
    ins_ += ['[nkbwg] "s"(a.nkb_wg)', '[nkbw] "s"(a.nkb_w)', '[qb] "s"(a.qb)', '[N] "s"(a.N)',
             '[tau] "s"(a.tau)', '[c] "s"(a.c)', '[krs] "s"(a.krs)', '[vrs] "s"(a.vrs)',
             '[wl] "s"(a.wl)', '[smem] "s"(a.smem)', '[mptr] "s"(a.mask_row)',
             '[val0] "s"(a.val[0])', '[val1] "s"(a.val[1])']
    nvt, ns32 = 11, 8
    if f8:
        outs += ['[qa0] "=&v"(vtmp[11])', '[qa1] "=&v"(vtmp[12])', '[ce] "=&v"(vtmp[13])',
                 '[sk0] "=&s"(s32[1])', '[sk1] "=&s"(s32[2])', '[t4] "=&s"(s32[3])',
                 '[t5] "=&s"(s32[8])']
        ins_ += ['[ksp] "s"(a.ksp)', '[sqv] "v"(a.sqv)', '[nkbm1] "s"(a.nkbm1)', '[wlv] "s"(a.wlv)']
        nvt, ns32 = 14, 9
    elif v8:
        outs += ['[t4] "=&s"(s32[3])', '[t5] "=&s"(s32[8])']
        ins_ += ['[wlv] "s"(a.wlv)']
        ns32 = 9
    if sas:
        ins_ += [f'[sa{j}] "s"(a.sa[{j}])' for j in range(sas + 1)]
        ins_ += ['[c6] "s"(a.c6)', '[c7] "s"(a.c7)']
    clob = [f"v{r}" for r in range(VOTE, 256)]
    clob += [f"a{r}" for r in range(OB, OB + 32 * MB)] + ["vcc", "scc", "m0"]
    body = []
    for t in L:
        body.append(t)
    # %[mpp] is the 64-bit pair (mp, mp_hi): spelled out below
    text = "\n".join(f'      "{t}\\n\\t"' for t in body)
    head = (f"// The key loop of one wave, d = {d}, {'causal' if causal else 'full'} attention"
            f"{(', QK^T on int8 codes' if i8 else ', QK^T on fp8 codes') if f8 else ''}"
            f"{', P.V on fp8 codes' if v8 else ''}"
            f"{f', SAS exponential of degree {sas}' if sas else ''} ({len(body)} lines)")
    name = f"key_loop_{'causal' if causal else 'full'}"
    return "\n".join([
        head,
        f"__device__ __forceinline__ void {name}(const LoopArgs& a, float (&m)[2], float (&mref)[2], "
        "float (&lsum)[2]) {",
        f"  float vtmp[{nvt}];",
        f"  uint32_t s32[{ns32}];",
        "  uint64_t s64[6];",
        "  asm volatile(",
        text,
        "      : " + ",\n        ".join(outs),
        "      : " + ",\n        ".join(ins_),
        "      : " + ", ".join(f'"{c}"' for c in clob + ["memory"]) + ");",
        "}"])


def main(out_path=None):
    here = os.path.dirname(os.path.abspath(__file__))
    parts = ["// Generated by gen_prefill_steps.py; edit that script, not this file.",
             f"// The compiler keeps v[0:{COMPILER_VGPRS}) and a[0:{COMPILER_VGPRS}); every other register is named here.",
             "// Per-key-tile steps of the prefill kernel (see the script's docstring for",
             "// the schedule, the register plan and the hazard rules).",
             "#pragma once", ""]
    for d, budget, f8, sas, v8, i8 in (
            (128, 26.0, False, 0, False, False), (64, 30.0, False, 0, False, False),
            (128, 26.0, True, 0, False, False), (64, 30.0, True, 0, False, False),
            (128, 26.0, False, 2, False, False), (128, 26.0, False, 3, False, False),
            (64, 30.0, False, 2, False, False), (64, 30.0, False, 3, False, False),
            (128, 26.0, False, 0, True, False), (64, 30.0, False, 0, True, False),
            (128, 26.0, True, 0, True, False), (64, 30.0, True, 0, True, False),
            (128, 26.0, True, 0, False, True), (64, 30.0, True, 0, False, True)):
        ns = ((f"d{d}" + ("i8" if i8 else "f8" if f8 else "") + ("v8" if v8 else ""))
              if not sas else f"d{d}s{sas}")
        parts.append(f"namespace {ns} {{")
        for h in helpers_cxx(d, f8):
            parts.append(h)
            parts.append("")
        ipwv = 64 * 2 * d // 1024 // 4
        ipwk = 64 * d // 1024 // 4 if f8 else ipwv
        if v8:
            ipwv = d // 64       # 64 d bytes per V tile, 1 KB per copy, 4 waves
        parts.append(LOOP_ARGS.format(ipwk=ipwk, ipwv=ipwv,
                                      f8doc=LOOP_ARGS_F8_DOC if f8 else (
                                          LOOP_ARGS_SAS_DOC if sas else (
                                              LOOP_ARGS_V8_DOC if v8 else "")),
                                      f8fields=LOOP_ARGS_F8_FIELDS if f8 else (
                                          LOOP_ARGS_SAS_FIELDS if sas else (
                                              LOOP_ARGS_V8_FIELDS if v8 else ""))))
        for causal in (True, False):
            parts.append(loop_cxx(d, causal, budget, f8, sas, v8, i8))
            parts.append("")
        parts.append(f"}}  // namespace {ns}")
        parts.append("")
    with open(out_path or os.path.join(here, "prefill_steps.inc"), "w") as f:
        f.write("\n".join(parts))


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else None)
