#!/usr/bin/env python3
"""Writes attn_fwd128_stream.h: the tile loop of attn_fwd128_kernel (prefill,
d = 128, one wave per SIMD) as one inline-asm instruction stream.

    python gen_fwd128_stream.py [SPLIT] [OUT] [--stats] [--show]

The MFMAs of a tile are fixed; the other instructions (softmax, LDS reads, the
barrier, the DMA of a later tile, loop control) come from in-order streams and
are placed greedily into the 32-cycle shadows of the MFMAs by a cycle model of
one wave per SIMD (an MFMA every 32 cycles, any other instruction 4 cycles, a
transcendental 8), earliest deadline first. Every placement is then checked
against the wait states gfx950 requires and the compiler would otherwise
insert (MFMA result -> VALU: 12; VALU result -> MFMA operand: 2, we use 3;
transcendental result -> other VALU: 1; VALU -> v_permlane: 2; M0 write ->
LDS DMA: 1) and against overwriting a register an MFMA in flight still reads
(2 MFMAs later at the earliest); out-of-line blocks are checked spliced in at
their branch. SPLIT is the number of QB1 probability pairs computed after the
scores of QB1 (the rest follows in the next tile's first MFMA group).

Per wave: 64 queries (QB0, QB1 of 32), one head. Per 64-key tile t, 64 MFMAs:
  M0-15  S0(t)   = K(t) Q0^T       (VGPR acc v224-255)
  M16-31 O1     += V(t-1)^T P1(t-1) (AGPR a64-127)
  M32-47 S1(t)   = K(t) Q1^T       (v192-223)
  M48-63 O0     += V(t)^T P0(t)    (a0-63)
VALU streams: X = softmax of QB0 tile t (after M15, before M48); Y = softmax of
QB1 tile t (head after M47 in iteration t, tail before M16 of iteration t+1).
"""
import sys

MF = "v_mfma_f32_32x32x16_bf16"
NEG_INF = "0xff800000"
THRESH = "0x43800000"   # 256.0: a tile's lane sum above this may hide p > 2^8

S_BASE = [224, 192]
P_BASE = [176, 160]
K_BASE = 96
O_BASE = [0, 64]
Q_BASE = [128, 160]
V_BASE = 192
TEMPS = [[(80, 81), (82, 83)], [(84, 85), (86, 87)]]
LT = [88, 89]
T0, T1, T2, T3, T4 = 90, 91, 92, 93, 94
SI, SX = 84, [85, 86]       # loop counter, mask-check scratch per QB
SINC, STMP, SRET = 88, 87, 89
SSKIP = 90                  # s[90:91]: lanes whose O needs the rescale
M_INIT = "0xf149f2ca"       # -1e30f, the reference max before any admitted key
LDS_PER_GAP = int(__import__("os").environ.get("LDS_PER_GAP", "2"))   # LDS reads per MFMA shadow

KST = 20480      # bytes per K stage (64 rows of 320: 16 chunks of 16 bytes, swizzled, and 4 pad slots)
VST = 16384      # bytes per V stage
V_REGION = 4 * KST


def vr(lo, n=1):
    return f"v{lo}" if n == 1 else f"v[{lo}:{lo + n - 1}]"


def ar(lo, n=1):
    return f"a{lo}" if n == 1 else f"a[{lo}:{lo + n - 1}]"


def vset(lo, n):
    return {f"v{i}" for i in range(lo, lo + n)}


def aset(lo, n):
    return {f"a{i}" for i in range(lo, lo + n)}


class Ins:
    def __init__(self, text, kind="valu", rd=(), wr=(), slots=1, after=-1, name=""):
        self.text = text
        self.kind = kind
        self.rd = set(rd)
        self.wr = set(wr)
        self.slots = slots
        self.after = after        # index of the MFMA that must be issued before this
        self.name = name
        self.deadline = 10 ** 9   # index of the first MFMA that must come after this
        self.deps = []            # items (other streams) that must be emitted first
        self.block = None         # out-of-line block (list of Ins) entered by this branch

    def ws(self):
        if self.kind == "nop":
            return int(self.text.split()[1]) + 1
        if self.kind == "label":
            return 0
        return max(1, self.text.count("\n") + 1)

    def __repr__(self):
        return self.text


def nop(n):
    return Ins(f"s_nop {n}", "nop", slots=n + 1)


# ---------------------------------------------------------------- MFMAs
def mfmas():
    out = []
    for i in range(16):                          # S0(t)
        kk, kb = divmod(i, 2)
        d = S_BASE[0] + 16 * kb
        k = K_BASE + 32 * kb + 4 * kk
        q = Q_BASE[0] + 4 * kk
        c = "0" if kk == 0 else vr(d, 16)
        out.append(Ins(f"{MF} {vr(d, 16)}, {vr(k, 4)}, {ar(q, 4)}, {c}", "mfma",
                       rd=vset(k, 4) | aset(q, 4) | (set() if kk == 0 else vset(d, 16)), wr=vset(d, 16)))
    for u in range(16):                          # O1 += V(t-1)^T P1(t-1)
        kb, r = divmod(u, 8)
        jj, db = divmod(r, 4)
        o = O_BASE[1] + 16 * db
        v = V_BASE + 16 * db + 8 * kb + 4 * jj
        p = P_BASE[1] + 8 * kb + 4 * jj
        out.append(Ins(f"{MF} {ar(o, 16)}, {ar(v, 4)}, {vr(p, 4)}, {ar(o, 16)}", "mfma",
                       rd=aset(o, 16) | aset(v, 4) | vset(p, 4), wr=aset(o, 16)))
    for i in range(16):                          # S1(t)
        kk, kb = divmod(i, 2)
        d = S_BASE[1] + 16 * kb
        k = K_BASE + 32 * kb + 4 * kk
        q = Q_BASE[1] + 4 * kk
        c = "0" if kk == 0 else vr(d, 16)
        out.append(Ins(f"{MF} {vr(d, 16)}, {vr(k, 4)}, {ar(q, 4)}, {c}", "mfma",
                       rd=vset(k, 4) | aset(q, 4) | (set() if kk == 0 else vset(d, 16)), wr=vset(d, 16)))
    for u in range(16):                          # O0 += V(t)^T P0(t)
        kb, r = divmod(u, 8)
        jj, db = divmod(r, 4)
        o = O_BASE[0] + 16 * db
        v = V_BASE + 16 * db + 8 * kb + 4 * jj
        p = P_BASE[0] + 8 * kb + 4 * jj
        out.append(Ins(f"{MF} {ar(o, 16)}, {ar(v, 4)}, {vr(p, 4)}, {ar(o, 16)}", "mfma",
                       rd=aset(o, 16) | aset(v, 4) | vset(p, 4), wr=aset(o, 16)))
    for i, m in enumerate(out):
        m.name = f"M{i}"
    return out


# ---------------------------------------------------------------- softmax pieces
def exps(j, pairs, first, lt):
    """fma/exp/cvt/dot over the given pairs of QB j; the lane sum goes to lt
    (started at 0 by the first pair when `first`)."""
    sb, pb = S_BASE[j], P_BASE[j]
    m = f"%[m{j}]"
    items = []
    pend = None
    if len(pairs) == 0:
        return items
    for n, p in enumerate(pairs):
        t0, t1 = TEMPS[j][n % 2]
        e0, e1 = sb + 2 * p, sb + 2 * p + 1
        items.append(Ins(f"v_fma_f32 v{t0}, v{e0}, %[c], -{m}", rd={f"v{e0}", m}, wr={f"v{t0}"}))
        items.append(Ins(f"v_fma_f32 v{t1}, v{e1}, %[c], -{m}", rd={f"v{e1}", m}, wr={f"v{t1}"}))
        if pend is not None:
            items += pend
        items.append(Ins(f"v_exp_f32 v{t0}, v{t0}", "trans", rd={f"v{t0}"}, wr={f"v{t0}"}, slots=2))
        items.append(Ins(f"v_exp_f32 v{t1}, v{t1}", "trans", rd={f"v{t1}"}, wr={f"v{t1}"}, slots=2))
        pend = [Ins(f"v_cvt_pk_bf16_f32 v{pb + p}, v{t0}, v{t1}", rd={f"v{t0}", f"v{t1}"}, wr={f"v{pb + p}"})]
        if first and n == 0:
            pend.append(Ins(f"v_add_f32 v{lt}, v{t0}, v{t1}", rd={f"v{t0}", f"v{t1}"}, wr={f"v{lt}"}))
        else:
            pend.append(Ins(f"v_add_f32 v{lt}, v{lt}, v{t0}", rd={f"v{lt}", f"v{t0}"}, wr={f"v{lt}"}))
            pend.append(Ins(f"v_add_f32 v{lt}, v{lt}, v{t1}", rd={f"v{lt}", f"v{t1}"}, wr={f"v{lt}"}))
    items += pend
    return items


def mask_block(j, lab):
    """Out of line: pick this tile's mask word for QB j (a special tile's per-lane
    word, else all masked) and set the masked scores to -inf."""
    sb = S_BASE[j]
    b = [Ins(f"{lab}:", "label")]
    for k in range(3):
        b.append(Ins(f"v_cmp_eq_u32 vcc, s{SI}, %[sp{j}{k}]\n\ts_cbranch_vccnz {lab}_{k}", "salu"))
    b.append(Ins(f"v_mov_b32 v{T0}, 0", wr={f"v{T0}"}))
    b.append(Ins(f"s_branch {lab}_a", "salu"))
    for k in range(3):
        b.append(Ins(f"{lab}_{k}:", "label"))
        b.append(Ins(f"v_mov_b32 v{T0}, %[mk{j}{k}]", rd={f"%[mk{j}{k}]"}, wr={f"v{T0}"}))
        if k < 2:
            b.append(Ins(f"s_branch {lab}_a", "salu"))
    b.append(Ins(f"{lab}_a:", "label"))
    b.append(Ins(f"v_mov_b32 v{T2}, {NEG_INF}", wr={f"v{T2}"}))
    for e in range(32):
        b.append(Ins(f"v_bfe_u32 v{T1}, v{T0}, {e}, 1", rd={f"v{T0}"}, wr={f"v{T1}"}))
        b.append(Ins(f"v_cmp_ne_u32 vcc, 0, v{T1}", rd={f"v{T1}"}, wr={"vcc"}))
        b.append(Ins(f"v_cndmask_b32 v{sb + e}, v{T2}, v{sb + e}, vcc", rd={f"v{T2}", f"v{sb + e}", "vcc"},
                     wr={f"v{sb + e}"}))
    b += ret_dispatch(lab)
    return b


def ret_dispatch(lab):
    """Return to the copy of the loop body that branched here (copy = i mod 4)."""
    b = [Ins(f"{lab}_ret:", "label"),
         Ins(f"s_and_b32 s{SRET}, s{SI}, 3", "salu")]
    for k in range(3):
        b.append(Ins(f"s_cmp_eq_u32 s{SRET}, {k}\n\ts_cbranch_scc1 {lab}_r{k}", "salu"))
    b.append(Ins(f"s_branch {lab}_r3", "salu"))
    return b


def slow_block(j, lab):
    """Out of line: the tile's lane sum exceeded the bound somewhere. Find the
    tile max; where it exceeds m by more than 2^8, raise m, rescale O and l, and
    recompute the tile's probabilities and sum."""
    sb = S_BASE[j]
    m, l = f"%[m{j}]", f"%[l{j}]"
    b = [Ins(f"{lab}:", "label")]
    b.append(Ins(f"v_max3_f32 v{T0}, v{sb}, v{sb + 1}, v{sb + 2}", rd=vset(sb, 3), wr={f"v{T0}"}))
    k = 3
    while k < 32:
        if k + 1 < 32:
            b.append(Ins(f"v_max3_f32 v{T0}, v{T0}, v{sb + k}, v{sb + k + 1}", rd={f"v{T0}"} | vset(sb + k, 2),
                         wr={f"v{T0}"}))
        else:
            b.append(Ins(f"v_max_f32 v{T0}, v{T0}, v{sb + k}", rd={f"v{T0}", f"v{sb + k}"}, wr={f"v{T0}"}))
        k += 2
    b.append(Ins(f"v_mov_b32 v{T1}, v{T0}", rd={f"v{T0}"}, wr={f"v{T1}"}))
    b.append(nop(1))
    b.append(Ins(f"v_permlane32_swap_b32 v{T0}, v{T1}", "perm", rd={f"v{T0}", f"v{T1}"}, wr={f"v{T0}", f"v{T1}"}))
    b.append(Ins(f"v_max_f32 v{T0}, v{T0}, v{T1}", rd={f"v{T0}", f"v{T1}"}, wr={f"v{T0}"}))
    b.append(Ins(f"v_mul_f32 v{T0}, %[c], v{T0}", rd={f"v{T0}"}, wr={f"v{T0}"}))
    b.append(Ins(f"v_add_f32 v{T1}, 0x41000000, {m}", rd={m}, wr={f"v{T1}"}))
    b.append(Ins(f"v_cmp_gt_f32 vcc, v{T0}, v{T1}", rd={f"v{T0}", f"v{T1}"}, wr={"vcc"}))
    b.append(Ins(f"s_cbranch_vccz {lab}_ret", "salu", rd={"vcc"}))
    # O needs no rescale where m was still its initial -1e30 (no key admitted
    # yet, so O is 0): skip it when that holds for every lane raising m
    b.append(Ins(f"v_mov_b32 v{T4}, {M_INIT}", wr={f"v{T4}"}))
    b.append(Ins(f"v_cmp_lg_f32 s[{SSKIP}:{SSKIP + 1}], v{T4}, {m}\n\ts_and_b64 s[{SSKIP}:{SSKIP + 1}], "
                 f"s[{SSKIP}:{SSKIP + 1}], vcc", rd={f"v{T4}", m, "vcc"}))
    b.append(Ins(f"v_sub_f32 v{T2}, {m}, v{T0}", rd={m, f"v{T0}"}, wr={f"v{T2}"}))
    b.append(Ins(f"v_exp_f32 v{T2}, v{T2}", "trans", rd={f"v{T2}"}, wr={f"v{T2}"}, slots=2))
    b.append(Ins(f"v_cndmask_b32 {m}, {m}, v{T0}, vcc", rd={m, f"v{T0}", "vcc"}, wr={m}))
    b.append(Ins(f"v_cndmask_b32 v{T2}, 1.0, v{T2}, vcc", rd={f"v{T2}", "vcc"}, wr={f"v{T2}"}))
    b.append(Ins(f"v_mul_f32 {l}, {l}, v{T2}", rd={l, f"v{T2}"}, wr={l}))
    b.append(Ins(f"s_cbranch_scc0 {lab}_x", "salu"))
    ob = O_BASE[j]
    for x in range(0, 64, 2):
        b.append(Ins(f"v_accvgpr_read_b32 v{T3}, a{ob + x}", rd={f"a{ob + x}"}, wr={f"v{T3}"}))
        b.append(Ins(f"v_accvgpr_read_b32 v{T4}, a{ob + x + 1}", rd={f"a{ob + x + 1}"}, wr={f"v{T4}"}))
        b.append(Ins(f"v_mul_f32 v{T3}, v{T3}, v{T2}", rd={f"v{T3}", f"v{T2}"}, wr={f"v{T3}"}))
        b.append(Ins(f"v_mul_f32 v{T4}, v{T4}, v{T2}", rd={f"v{T4}", f"v{T2}"}, wr={f"v{T4}"}))
        b.append(Ins(f"v_accvgpr_write_b32 a{ob + x}, v{T3}", rd={f"v{T3}"}, wr={f"a{ob + x}"}))
        b.append(Ins(f"v_accvgpr_write_b32 a{ob + x + 1}, v{T4}", rd={f"v{T4}"}, wr={f"a{ob + x + 1}"}))
    b.append(Ins(f"{lab}_x:", "label"))
    b += exps(j, range(16), True, LT[j])
    b += ret_dispatch(lab)
    return b


def fix_block(b):
    """Insert the wait states a straight-line out-of-line block needs."""
    out = []
    for it in b:
        if it.kind != "label":
            h = hazard_ws([x for x in out if x.kind != "label"], it)
            if h:
                out.append(nop(h - 1))
        out.append(it)
    return out


def stream_x_or_y(j, lab_mask, lab_slow, pairs_head, pairs_tail, part, st):
    """Items of QB j's softmax: part 'head' = mask check + pairs_head,
    part 'tail' = pairs_tail + sum check + l update."""
    sb, pb = S_BASE[j], P_BASE[j]
    items = []
    if part in ("head", "all"):
        items.append(Ins(f"s_sub_u32 s{SX[j]}, s{SI}, %[fd{j}]", "salu", name=f"mchk{j}"))
        br = Ins(f"s_cmp_lt_u32 s{SX[j]}, %[fc{j}]\n\ts_cbranch_scc0 {lab_mask}\n{lab_mask}_r{st}:", "br",
                 rd=vset(sb, 32), wr=vset(sb, 32) | {"vcc"}, slots=2, name=f"mbr{j}")
        br.block = fix_block(mask_block(j, lab_mask))
        items.append(br)
        items += exps(j, pairs_head, True, LT[j])
    if part in ("tail", "all"):
        items += exps(j, pairs_tail, len(pairs_head) == 0, LT[j])
        chk = Ins(f"v_cmp_lt_f32 vcc, {THRESH}, v{LT[j]}", rd={f"v{LT[j]}"}, wr={"vcc"})
        br = Ins(f"s_cbranch_vccnz {lab_slow}\n{lab_slow}_r{st}:", "br",
                 rd=vset(sb, 32) | aset(O_BASE[j], 64) | {"vcc", f"%[m{j}]", f"%[l{j}]"},
                 wr=vset(pb, 16) | aset(O_BASE[j], 64) | {f"%[m{j}]", f"%[l{j}]", f"v{LT[j]}"} | vset(T0, 5)
                 | {f"v{t}" for pr in TEMPS[j] for t in pr},
                 name=f"sbr{j}")
        br.block = fix_block(slow_block(j, lab_slow))
        items += [chk, br]
        items.append(Ins(f"v_add_f32 %[l{j}], %[l{j}], v{LT[j]}", rd={f"%[l{j}]", f"v{LT[j]}"}, wr={f"%[l{j}]"}))
    return items


# ---------------------------------------------------------------- LDS / DMA
def kbase(st, kk):
    """Base register of K operand reads: even / odd k step (the row swizzle moves
    the two 32-byte halves of a 64-byte piece apart per row), stages 0-1 / 2-3."""
    return f"%[k{'o' if kk % 2 else 'e'}{st // 2}]"


def kofs(st, kb, kk):
    """Immediate offset of K operand (kb, kk) in stage st (rows of 320 bytes)."""
    return (st % 2) * KST + 32 * 320 * kb + 64 * (kk // 2)


def v_reads(st):
    items = []
    so = st * VST
    for u in range(16):
        kb, r = divmod(u, 8)
        jj, db = divmod(r, 4)
        reg = V_BASE + 16 * db + 8 * kb + 4 * jj
        base = f"%[v{'o' if jj else 'e'}{db}]"
        offs = (8192 * kb + 1024, 8192 * kb + 3072) if jj else (8192 * kb, 8192 * kb + 2048)
        for h in range(2):
            it = Ins(f"ds_read_b64_tr_b16 {ar(reg + 2 * h, 2)}, {base} offset:{so + offs[h]}", "lds",
                     wr=aset(reg + 2 * h, 2), after=16 + u + 2, name=f"V{u}.{h}")
            it.fixed_deadline = 36
            items.append(it)
    return items


def k_reads(st):
    nst = (st + 1) % 4
    so = nst * KST
    items = []
    for mm in range(16):
        kk, kb = divmod(mm, 2)
        reg = K_BASE + 32 * kb + 4 * kk
        items.append(Ins(f"ds_read_b128 {vr(reg, 4)}, {kbase(nst, kk)} offset:{kofs(nst, kb, kk)}", "lds",
                         wr=vset(reg, 4), after=32 + mm + 2, name=f"K{mm}"))
    return items


def dma(st):
    items = []
    items.append(Ins(f"s_add_u32 s{STMP}, s{SI}, 5\n\ts_cmp_eq_u32 s{STMP}, %[T]\n\t"
                     f"s_cselect_b32 s{STMP}, 0x80000000, 0\n\ts_add_u32 s{SINC}, s{STMP}, %[tstride]", "salu",
                     slots=4, name="sinc"))
    for jx in range(9):
        if jx < 5:
            off = st * KST + 4096 * jx
            lw = "%[lw]"
            rs = "%[rk]"
        else:
            off = V_REGION + st * VST + 4096 * (jx - 5)
            lw = "%[lw]"
            rs = "%[rv]"
        items.append(Ins(f"s_add_u32 m0, {lw}, {off}", "salu", wr={"m0"}, name=f"m0_{jx}"))
        items.append(Ins(f"buffer_load_dwordx4 %[cf{jx}], {rs}, 0 offen lds", "vmem",
                         rd={"m0", f"%[cf{jx}]"}, name=f"dma{jx}"))
    for jx in range(9):
        items.append(Ins(f"v_add_u32 %[cf{jx}], s{SINC}, %[cf{jx}]", rd={f"%[cf{jx}]"}, wr={f"%[cf{jx}]"},
                         name=f"inc{jx}"))
    return items


# ---------------------------------------------------------------- scheduler
def hazard_ws(emitted, c):
    """Wait states the candidate c still needs after the emitted sequence."""
    need = 0
    ws = 0
    mf_between = 0
    for p in reversed(emitted):
        if p.kind == "mfma":
            # MFMA result read / overwritten by a non-MFMA
            if c.kind != "mfma" and (c.rd | c.wr) & p.wr:
                need = max(need, 12 - ws)
            # register an MFMA still reads, overwritten
            if c.kind != "mfma" and c.wr & p.rd and mf_between < 2:
                return None
        elif p.kind in ("valu", "trans", "perm", "br"):
            if c.kind == "mfma" and c.rd & p.wr:
                need = max(need, 3 - ws)
            if p.kind == "trans" and c.kind not in ("trans",) and c.rd & p.wr:
                need = max(need, 1 - ws)
            if c.kind == "perm" and c.rd & p.wr:
                need = max(need, 2 - ws)
            if p.kind == "br" and c.kind != "mfma" and (c.rd & p.wr):
                need = max(need, 1 - ws)
        elif p.kind == "vmem":
            if c.wr & p.rd:
                need = max(need, 1 - ws)
        elif p.kind == "salu":
            if "m0" in p.wr and c.kind == "vmem" and "m0" in c.rd:
                need = max(need, 1 - ws)
        ws += p.ws()
        if p.kind == "mfma":
            mf_between += 1
        if ws > 24 and mf_between >= 2:
            break
    return max(0, need)


def schedule(mf, streams, prio_order, end_items):
    """streams: list of item lists (in-order within a stream). Greedy, cycle model:
    fill the 32-cycle shadow of each MFMA with ready items by deadline."""
    # deadlines: item must precede MFMA that reads what it writes (or explicit)
    for s in streams:
        for it in s:
            it.deadline = getattr(it, "fixed_deadline", 10 ** 9)
            for k, m in enumerate(mf):
                if (m.rd | m.wr) & it.wr or (it.kind == "vmem" and False):
                    if k > it.after:
                        it.deadline = min(it.deadline, k)
                        break
        # in-order: propagate deadlines backwards
        dl = 10 ** 9
        for it in reversed(s):
            dl = min(dl, it.deadline)
            it.deadline = dl
    heads = [0] * len(streams)
    out = []
    t = 0
    mfree = 0
    emitted_names = set()
    n_mfma = 0

    def ready(si, forced=False):
        s = streams[si]
        if heads[si] >= len(s):
            return None
        it = s[heads[si]]
        if it.after >= n_mfma:
            return None
        for d in it.deps:
            if d.name not in emitted_names:
                return None
        h = hazard_ws(out, it)
        if h is None:
            return None
        if h > 0 and not forced:
            return None
        return it, h

    gap_lds = [0]

    def emit(it):
        nonlocal t, mfree
        out.append(it)
        if it.kind == "lds":
            gap_lds[0] += 1
        emitted_names.add(it.name)
        if it.kind == "mfma":
            st = max(t, mfree)
            t = st + 4
            mfree = st + 32
        else:
            t += 4 * it.slots

    for k in range(len(mf) + 1):
        # fill the gap before MFMA k (or the tail)
        while True:
            # forced: items whose deadline is k
            cands = []
            for si in range(len(streams)):
                r = ready(si)
                if r:
                    cands.append((r[0].deadline, prio_order[si], si, r[0]))
            urgent = [s for s in range(len(streams)) if heads[s] < len(streams[s])
                      and streams[s][heads[s]].deadline <= k]
            if k < len(mf) and not urgent:
                cands = [c for c in cands if t + 4 * c[3].slots <= mfree]
            # at most LDS_PER_GAP LDS reads in one MFMA shadow: bursts fill the
            # CU's LDS command queue and stall issue
            if not urgent:
                cands = [c for c in cands if c[3].kind != "lds" or gap_lds[0] < LDS_PER_GAP]
            if not cands:
                if urgent:
                    # an urgent item waits for a hazard: pad
                    r = None
                    for si in sorted(urgent, key=lambda s: prio_order[s]):
                        r = ready(si, forced=True)
                        if r is not None:
                            break
                    if r is None:
                        for si in sorted(range(len(streams)), key=lambda s: prio_order[s]):
                            r = ready(si, forced=True)
                            if r is not None:
                                break
                    if r is None:
                        raise RuntimeError(f"deadlock before M{k}: {[streams[s][heads[s]] for s in urgent]}")
                    it, h = r
                    if h > 0:
                        emit(nop(h - 1))
                    emit(it)
                    heads[si] += 1
                    continue
                break
            cands.sort(key=lambda c: (c[0], c[1]))
            si = cands[0][2]
            emit(cands[0][3])
            heads[si] += 1
        if k == len(mf):
            break
        h = hazard_ws(out, mf[k])
        if h is None:
            raise RuntimeError(f"M{k} WAR")
        if h > 0:
            emit(nop(h - 1))
        emit(mf[k])
        gap_lds[0] = 0
        n_mfma += 1
    # drain leftovers (past the last MFMA)
    left = True
    while left:
        left = False
        for si in sorted(range(len(streams)), key=lambda s: prio_order[s]):
            r = ready(si, forced=True)
            if r:
                it, h = r
                if h > 0:
                    emit(nop(h - 1))
                emit(it)
                heads[si] += 1
                left = True
                break
    for si, s in enumerate(streams):
        if heads[si] < len(s):
            raise RuntimeError(f"stream {si} not drained: {s[heads[si]]}")
    for it in end_items:
        h = hazard_ws(out, it) or 0
        if h > 0:
            emit(nop(h - 1))
        emit(it)
    return out, t, mfree


def build_iteration(st, h_split, lab):
    """One tile iteration for LDS stage st (copy st of the unrolled loop)."""
    mf = mfmas()
    # barrier after all V reads have landed; DMA of tile i+4 into this stage and
    # the K(t+1) reads after it
    vr_ = v_reads(st)
    bar = Ins("s_waitcnt vmcnt(18) lgkmcnt(0)\n\ts_barrier", "sync", after=36, slots=2, name="bar")
    bar.deps = [vr_[-1]]
    bar.fixed_deadline = 40
    kr = k_reads(st)
    for it in kr:
        it.deps = [bar]
    dm = dma(st)
    for it in dm:
        if it.name.startswith("m0_") or it.name == "sinc":
            it.deps = [bar]
    # X: QB0 of this tile; Y: tail of QB1 of the previous tile, head of this tile
    x = stream_x_or_y(0, "L%=_mx", "L%=_sx", list(range(16)), [], "head", st) + \
        stream_x_or_y(0, "L%=_mx", "L%=_sx", list(range(16)), [], "tail", st)
    # (the tail part with no pairs: just the check)
    yt = stream_x_or_y(1, "L%=_my", "L%=_sy", list(range(h_split)), list(range(h_split, 16)), "tail", st)
    yh = stream_x_or_y(1, "L%=_my", "L%=_sy", list(range(h_split)), [], "head", st)
    for it in x:
        it.after = max(it.after, 15)
    for it in yh:
        it.after = max(it.after, 47)
    # the X check must precede PV0 (it may rewrite P0 / O0); Y tail before PV1
    streams = [yt, x, vr_, [bar], kr, dm, yh]
    prio = [0, 2, 1, 3, 4, 5, 6]
    start = [Ins("s_waitcnt lgkmcnt(0)", "sync", name="kwait")]
    loop = [Ins(f"s_add_u32 s{SI}, s{SI}, 1\n\ts_cmp_gt_u32 s{SI}, %[T]\n\ts_cbranch_scc1 L%=_fin", "salu",
                slots=3, name="loop")]
    out, t, mfree = schedule(mf, streams, prio, loop)
    return start + out, t


def verify(seq, ctx=""):
    """Re-check hazards over a straight-line sequence (with out-of-line blocks spliced)."""
    errs = []
    for i, c in enumerate(seq):
        h = hazard_ws(seq[:i], c)
        if h is None or h > 0:
            errs.append((i, c.text, h))
    return errs


def splice_checks(seq):
    errs = verify(seq)
    for i, it in enumerate(seq):
        if it.block:
            body = [b for b in it.block if b.kind != "label"]
            sp = seq[:i + 1] + body + seq[i + 1:]
            e = verify(sp)
            errs += [(x, y, z, it.name) for (x, y, z) in e]
    return errs


def fmt(seq):
    lines = []
    for it in seq:
        for ln in it.text.split("\n"):
            ln = ln.strip()
            if ln:
                lines.append(ln)
    return lines


def main():
    h_split = int(sys.argv[1]) if len(sys.argv) > 1 else 6
    total = 0
    allseq = []
    blocks = []
    for st in range(4):
        lab = f"L%=_{st}"
        seq, t = build_iteration(st, h_split, lab)
        errs = splice_checks(seq)
        if errs:
            for e in errs[:20]:
                print("HAZARD", st, e, file=sys.stderr)
            sys.exit(1)
        total = t
        allseq.append(seq)
        for it in seq:
            if it.block:
                blocks.append(it.block)
    nm = sum(1 for it in allseq[0] if it.kind == "mfma")
    print(f"// h_split={h_split} est cycles/iter={total} mfma={nm * 32} util={nm * 32 / total:.3f} "
          f"instrs={len(fmt(allseq[0]))}", file=sys.stderr)
    if "--stats" in sys.argv:
        return
    lines = []
    for st in range(4):
        lines.append(f"L%=_{st}_top:")
        lines += fmt(allseq[st])
    lines.append("s_branch L%=_0_top")
    seen = set()
    for b in blocks:
        key = b[0].text
        if key in seen:
            continue
        seen.add(key)
        lines += fmt(b)
    lines.append("L%=_fin:")
    dflt = __import__("pathlib").Path(__file__).resolve().parent / "attn_fwd128_stream.h"
    out = open(sys.argv[2] if len(sys.argv) > 2 and not sys.argv[2].startswith("--") else dflt, "w")
    out.write("// Generated by gen_fwd128_stream.py: the tile loop of attn_fwd128_kernel (attn_fwd.hip)\n"
              f"// as one instruction stream (QB1 split {h_split}). Regenerate rather than edit.\n"
              "#pragma once\n\n")
    out.write("#define SFA_FWD128_LOOP \\\n")
    for ln in lines:
        out.write(f'  "{ln}\\n" \\\n')
    out.write("\n")
    # the QB1 sum of the (absent) tile before the first: its tail part runs in
    # the first iteration on scores of -inf
    # Registers start as the state after a tile -1 with no admitted key: O, P1
    # and the V^T operands 0, the QB1 scores -inf (their exps in the first
    # tile's stream give 0), the QB1 partial sum 0. Tuples are filled by MFMAs
    # of constant operands (one issue slot per 16 registers): zeros times
    # zeros, and bf16 -inf times bf16 ones. The score MFMAs go first, so that
    # the first VALU reads of S1 / P1 lie more than 12 wait states later.
    z, ni, one = vr(T0, 4), vr(TEMPS[1][0][0], 4), vr(80, 4)
    pro = [f"s_mov_b32 s{SI}, 0", f"v_mov_b32 v{LT[1]}, 0"]
    pro += [f"v_mov_b32 v{T0 + x}, 0" for x in range(4)]
    pro += [f"v_mov_b32 v{TEMPS[1][0][0] + x}, 0xff80ff80" for x in range(4)]
    pro += [f"v_mov_b32 v{80 + x}, 0x3f803f80" for x in range(4)]
    pro += ["s_nop 2"]
    pro += [f"{MF} {vr(S_BASE[1], 16)}, {ni}, {one}, 0", f"{MF} {vr(S_BASE[1] + 16, 16)}, {ni}, {one}, 0",
            f"{MF} {vr(P_BASE[1], 16)}, {z}, {z}, 0"]
    kreads = []
    for mm in range(16):
        kk, kb = divmod(mm, 2)
        kreads.append(f"ds_read_b128 {vr(K_BASE + 32 * kb + 4 * kk, 4)}, {kbase(0, kk)} offset:{kofs(0, kb, kk)}")
    zero = [f"{MF} {ar(16 * x, 16)}, {z}, {z}, 0" for x in range(8)]
    zero += [f"{MF} {ar(V_BASE + 16 * x, 16)}, {z}, {z}, 0" for x in range(4)]
    for x in range(12):
        pro.append(zero[x])
        pro += kreads[x * 16 // 12:(x + 1) * 16 // 12]
    out.write("#define SFA_FWD128_PROLOGUE \\\n")
    for ln in pro:
        out.write(f'  "{ln}\\n" \\\n')
    out.write("\n")
    cv = ", ".join(f'"v{x}"' for x in range(80, 256))
    ca = ", ".join(f'"a{x}"' for x in range(V_BASE, 256))
    out.write(f"#define SFA_FWD128_CLOBBER_V {cv}\n")
    out.write(f"#define SFA_FWD128_CLOBBER_A {ca}\n")
    out.close()
    print(f"// {len(lines)} lines", file=sys.stderr)
    if "--show" in sys.argv:
        for ln in fmt(allseq[0]):
            print(ln)


if __name__ == "__main__":
    main()
