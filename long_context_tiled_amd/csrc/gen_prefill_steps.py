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
Measured issue costs on gfx950 (cycles per wave64 instruction): add / fma /
max3 4.2, exp 8.2, bf16 pack ~6, plus ~8 cycles per MFMA issue. The
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
  v[56:63]              exp temporaries
Everything below v56 is left to the compiler.

Hazards are resolved here, not by the compiler (which does not look inside
asm): every read of a register is checked against its last writer and
s_nop / s_waitcnt lgkmcnt are inserted as needed:
  MFMA (8 passes) write -> VALU read           12 wait states
  VALU write -> MFMA read                      4 (2 required)
  transcendental write -> VALU read            2 (1 required)
  ds_read -> any use                           s_waitcnt lgkmcnt
  MFMA read of a fragment -> ds_read over it   2
Back-to-back accumulation into the same MFMA destination needs none.

Run:  python gen_prefill_steps.py [OUT]   (default: prefill_steps.inc beside it)
"""
import os
import re
import sys

NOP_MFMA_VALU = 12
NOP_VALU_MFMA = 4
NOP_TRANS_VALU = 2
NOP_MFMA_READ_LOAD = 2

COST = {"v_exp_f32": 8.2, "v_cvt_pk_bf16_f32": 6.0}
COST_DEFAULT = 4.2

SBUF = {"A": 128, "B": 192}
KREG = 64     # K / V^T fragments, v[64:95]
PREG = 96     # P^T operand, v[96:127]
TREG = 48     # exp temporaries, three pairs v[48:53]
VADR = 54     # V^T read addresses, v[54 : 54 + 2 MB)
KADR = 62     # K read addresses, v62 / v63 alternating
OB = 64       # first AGPR of O^T
COMPILER_VGPRS = 48  # v[0:48) and a[0:48) stay with the compiler


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
        self.cost = COST.get(op, COST_DEFAULT) if kind in ("valu", "trans") else 0.0


class Step:
    """One step variant for one head dim and buffer assignment."""

    def __init__(self, d, variant, x, y, budget):
        self.d = d
        self.MB = d // 32
        self.KS = d // 16
        self.QB = OB + 32 * self.MB
        self.rowBytes = 2 * d
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

    def kfrag(self, j, a):
        return rng("v", KREG + 8 * j + 4 * a, 4)

    def vfrag(self, j, mb):
        # V^T fragments of one key step: MB tuples of 4 registers; two buffers
        return rng("v", KREG + 16 * j + 4 * mb, 4)

    def pfrag(self, kp, nb):
        return rng("v", PREG + 4 * (2 * kp + nb), 4)

    def qfrag(self, ks, nb):
        return rng("a", self.QB + 8 * ks + 4 * nb, 4)

    def oblk(self, mb, nb):
        return rng("a", OB + 16 * (2 * mb + nb), 16)

    def k_loads(self, ks):
        # fragment address of k-step ks: the tile base XOR 32 ks (the swizzle
        # only moves address bits 4..7, the tile base has bits 0..9 clear)
        out = []
        if ks == 0:
            adr = "%[kb0]"
        else:
            adr = f"v{KADR + (ks & 1)}"
            out.append(Ins(f"v_xor_b32 {adr}, {32 * ks}, %[kb0]", "valu", wr=[adr]))
        for a in range(2):
            dst = self.kfrag(ks & 1, a)
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

    def qk_mfma(self, ks, a, nb):
        s = self.s_blk(self.y, a, nb)
        kf = self.kfrag(ks & 1, a)
        qf = self.qfrag(ks, nb)
        src_c = "0" if ks == 0 else s
        rd = [kf, qf] + ([] if ks == 0 else [s])
        return Ins(f"v_mfma_f32_32x32x16_bf16 {s}, {kf}, {qf}, {src_c}", "mfma", wr=[s], rd=rd)

    def pv_mfma(self, ks, mb, nb):
        o = self.oblk(mb, nb)
        vf = self.vfrag((ks + 1) & 1, mb)
        pf = self.pfrag(ks, nb)
        return Ins(f"v_mfma_f32_32x32x16_bf16 {o}, {vf}, {pf}, {o}", "mfma", wr=[o], rd=[vf, pf, o],
                   tag=("pv", ks))

    def exp_stream(self):
        """Per score pair: scale-and-shift, exp2, row-sum, pack to bf16."""
        out = []
        for gp in range(32):
            ch, i2 = gp >> 2, gp & 3
            kp, nb = ch >> 1, ch & 1
            a = kp >> 1
            r0 = 8 * (kp & 1) + 2 * i2
            s0 = f"v{self.s_reg(self.x, a, nb, r0)}"
            s1 = f"v{self.s_reg(self.x, a, nb, r0 + 1)}"
            t0 = f"v{TREG + 2 * (gp % 3)}"
            t1 = f"v{TREG + 2 * (gp % 3) + 1}"
            w = f"v{PREG + 4 * (2 * kp + nb) + i2}"
            ls = f"%[ls{nb}]"
            nm = f"%[nm{nb}]"
            out += [
                Ins(f"v_fma_f32 {t0}, {s0}, %[c], {nm}", "valu", wr=[t0], rd=[s0]),
                Ins(f"v_fma_f32 {t1}, {s1}, %[c], {nm}", "valu", wr=[t1], rd=[s1]),
                Ins(f"v_exp_f32 {t0}, {t0}", "trans", wr=[t0], rd=[t0]),
                Ins(f"v_exp_f32 {t1}, {t1}", "trans", wr=[t1], rd=[t1]),
                Ins(f"v_add_f32 {ls}, {ls}, {t0}", "valu", rd=[t0]),
                Ins(f"v_cvt_pk_bf16_f32 {w}, {t0}, {t1}", "valu", wr=[w], rd=[t0, t1],
                    tag=("pf", kp)),
                Ins(f"v_add_f32 {ls}, {ls}, {t1}", "valu", rd=[t1]),
            ]
        return out

    def max_stream(self):
        """Row maxima of the new tile: query half nb over both key halves."""
        out = []
        first = {0: True, 1: True}
        for a in range(2):
            for nb in range(2):
                for i in range(8):
                    r0 = self.s_reg(self.y, a, nb, 2 * i)
                    s0, s1 = f"v{r0}", f"v{r0 + 1}"
                    tm = f"%[tm{nb}]"
                    if first[nb]:
                        out.append(Ins(f"v_max_f32 {tm}, {s0}, {s1}", "valu", rd=[s0, s1]))
                        first[nb] = False
                    else:
                        out.append(Ins(f"v_max3_f32 {tm}, {tm}, {s0}, {s1}", "valu", rd=[s0, s1]))
        return out

    # ---- schedule ---------------------------------------------------------
    def build(self):
        seq = []          # scheduled instructions (before hazard fixing)
        exp_q = self.exp_stream() if self.pv else []
        max_q = self.max_stream() if self.qk else []
        KS, MB = self.KS, self.MB

        # exp pairs needed before PV key step ks: pairs 0 .. 8 ks + 7, i.e.
        # the pack of chunk kp <= ks; index of the last such pack in exp_q
        def exp_needed(ks):
            last = -1
            for i, ins in enumerate(exp_q):
                if ins.tag == ("pf", ks) or (ins.tag and ins.tag[0] == "pf" and ins.tag[1] < ks):
                    last = i
            return last + 1

        exp_pos = 0
        max_pos = 0
        n_slots = (4 * KS if self.qk else 0) + (8 * MB if self.pv else 0)
        total_valu = sum(i.cost for i in exp_q) + sum(i.cost for i in max_q)
        per_slot = total_valu / max(n_slots, 1)
        budget = max(self.budget, per_slot)

        def pull_exp(limit_cycles):
            nonlocal exp_pos
            used = 0.0
            while exp_pos < len(exp_q) and used + exp_q[exp_pos].cost <= limit_cycles + 1e-9:
                seq.append(exp_q[exp_pos])
                used += exp_q[exp_pos].cost
                exp_pos += 1
            return used

        def pull_max(n):
            nonlocal max_pos
            used = 0.0
            for _ in range(n):
                if max_pos < len(max_q):
                    seq.append(max_q[max_pos])
                    used += max_q[max_pos].cost
                    max_pos += 1
            return used

        if self.pv:
            seq += self.v_addr()
        # phase A --------------------------------------------------------
        if self.qk:
            seq += self.k_loads(0)
            # vector work that needs no fragment, while the first loads fly
            if self.pv:
                pull_exp(2 * budget)
            for ks in range(KS):
                for blk in range(4):
                    a, nb = blk >> 1, blk & 1
                    seq.append(self.qk_mfma(ks, a, nb))
                    if blk == 0 and ks + 1 < KS:
                        seq += self.k_loads(ks + 1)
                    if blk == 0 and self.pv and ks == KS // 2:
                        seq += self.v_loads(0)
                    if self.pv:
                        pull_exp(budget)
        elif self.pv:
            seq += self.v_loads(0)

        # phase B --------------------------------------------------------
        if self.pv:
            for ks in range(4):
                need = exp_needed(ks)
                while exp_pos < need:
                    seq.append(exp_q[exp_pos])
                    exp_pos += 1
                for i in range(2 * MB):
                    mb, nb = i >> 1, i & 1
                    seq.append(self.pv_mfma(ks, mb, nb))
                    if i == 0 and ks + 1 < 4:
                        seq += self.v_loads(ks + 1)
                    used = pull_max(1) if (self.qk and (ks > 0 or i > 1)) else 0.0
                    pull_exp(budget - used)
        # leftovers
        while exp_pos < len(exp_q):
            seq.append(exp_q[exp_pos])
            exp_pos += 1
        while max_pos < len(max_q):
            seq.append(max_q[max_pos])
            max_pos += 1
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
                        gap = NOP_MFMA_READ_LOAD - slots_since(last_mfma_read[r])
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
                if wkind == "mfma" and ins.kind in ("valu", "trans"):
                    need = max(need, NOP_MFMA_VALU - slots_since(widx))
                elif wkind in ("valu", "trans") and ins.kind == "mfma":
                    need = max(need, NOP_VALU_MFMA - slots_since(widx))
                elif wkind == "trans" and ins.kind in ("valu", "trans"):
                    need = max(need, NOP_TRANS_VALU - slots_since(widx))
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
            if ins.kind == "mfma":
                for r in ins.rd:
                    last_mfma_read[r] = idx
        if len(lds_seq) > waited:
            emit("s_waitcnt lgkmcnt(0)")
        self.out = out
        return self

    def estimate(self):
        """Rough cycle estimate: each MFMA slot max(32, vector work + 8)."""
        t = 0.0
        cur = None
        for ins in self.seq:
            if ins.kind == "mfma":
                if cur is not None:
                    t += max(32.0, cur + 8.0)
                cur = 0.0
            elif cur is not None:
                cur += ins.cost
            else:
                t += ins.cost
        if cur is not None:
            t += max(32.0, cur + 8.0)
        return t

    # ---- C++ ------------------------------------------------------------
    def cxx(self):
        MB = self.MB
        name = f"step_{self.variant}_{self.x if self.pv else ''}{self.y if self.qk else ''}"
        args, outs, ins_ = [], [], []
        if self.qk:
            args += ["float (&tm)[2]", "uint32_t kb0"]
            outs += ['[tm0] "=&v"(tm[0])', '[tm1] "=&v"(tm[1])']
            ins_ += ['[kb0] "v"(kb0)']
        if self.pv:
            args += ["float (&lsum)[2]", "const float (&nmc)[2]", "float c", "uint32_t vb0",
                     "uint32_t vb1"]
            outs += ['[ls0] "+v"(lsum[0])', '[ls1] "+v"(lsum[1])']
            ins_ += ['[nm0] "v"(nmc[0])', '[nm1] "v"(nmc[1])', '[c] "s"(c)', '[vb0] "v"(vb0)',
                     '[vb1] "v"(vb1)']
        clob = [f"v{r}" for r in range(TREG, 128)]
        if self.qk:
            clob += [f"v{r}" for r in range(SBUF[self.y], SBUF[self.y] + 64)]
        if self.pv:
            clob += [f"a{r}" for r in range(OB, OB + 32 * MB)]
        what = {"full": f"S^T of the next tile into buffer {self.y}, exp and PV of the "
                        f"current tile from buffer {self.x}",
                "qk": f"S^T of the next tile into buffer {self.y} and its row maxima",
                "pv": f"exp and PV of the current tile from buffer {self.x}"}[self.variant]
        head = (f"// {self.variant} step, d = {self.d}: {what} "
                f"({len(self.out)} instructions, ~{self.estimate():.0f} cycles)")
        return asm_function(head, name, args, self.out, outs, ins_, clob)


def asm_function(head, name, args, body, outs, ins_, clob):
    text = "\n".join(f'      "{t}\\n\\t"' for t in body)
    clob_s = ", ".join(f'"{c}"' for c in clob + ["memory"])
    return "\n".join([
        head,
        f"__device__ __forceinline__ void {name}({', '.join(args)}) {{",
        "  asm volatile(",
        text,
        "      : " + ",\n        ".join(outs),
        "      : " + ",\n        ".join(ins_),
        "      : " + clob_s + ");",
        "}"])


def helpers_cxx(d):
    """Blocks outside the key loop that touch the fixed registers."""
    MB, KS = d // 32, d // 16
    QB = OB + 32 * MB
    row_bytes = 2 * d
    o_regs = [f"a{r}" for r in range(OB, OB + 32 * MB)]
    parts = []

    # zero O
    body = [f"v_accvgpr_write_b32 {r}, 0" for r in o_regs]
    parts.append(asm_function(f"// O^T accumulators a[{OB}:{OB + 32 * MB - 1}] = 0",
                              "zero_o", [], body, [], [], o_regs))

    # Q^T fragments into AGPRs
    body = []
    for ks in range(KS):
        adr = "%[qb0]" if ks == 0 else f"v{KADR + (ks & 1)}"
        if ks:
            body.append(f"v_xor_b32 {adr}, {32 * ks}, %[qb0]")
        for nb in range(2):
            lo = QB + 8 * ks + 4 * nb
            body.append(f"ds_read_b128 a[{lo}:{lo + 3}], {adr} offset:{nb * 32 * row_bytes}")
    body.append("s_waitcnt lgkmcnt(0)")
    parts.append(asm_function(
        f"// Q^T fragments of the wave's 64 queries into a[{QB}:{QB + 8 * KS - 1}]; qb0 is the "
        "k-step 0 fragment address",
        "load_q", ["uint32_t qb0"], body, [], ['[qb0] "v"(qb0)'],
        [f"a{r}" for r in range(QB, QB + 8 * KS)] + [f"v{KADR}", f"v{KADR + 1}"]))

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


def main(out_path=None):
    here = os.path.dirname(os.path.abspath(__file__))
    parts = ["// Generated by gen_prefill_steps.py; edit that script, not this file.",
             f"// The compiler keeps v[0:{COMPILER_VGPRS}) and a[0:{COMPILER_VGPRS}); every other register is named here.",
             "// Per-key-tile steps of the prefill kernel (see the script's docstring for",
             "// the schedule, the register plan and the hazard rules).",
             "#pragma once", ""]
    for d, budget in ((128, 22.0), (64, 30.0)):
        parts.append(f"namespace d{d} {{")
        for h in helpers_cxx(d):
            parts.append(h)
            parts.append("")
        for variant, pairs in (("full", (("A", "B"), ("B", "A"))), ("qk", (("A", "A"), ("B", "B"))),
                               ("pv", (("A", "A"), ("B", "B")))):
            for x, y in pairs:
                st = Step(d, variant, x, y, budget).build().fix_hazards()
                parts.append(st.cxx())
                parts.append("")
        parts.append(f"}}  // namespace d{d}")
        parts.append("")
    with open(out_path or os.path.join(here, "prefill_steps.inc"), "w") as f:
        f.write("\n".join(parts))


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else None)
