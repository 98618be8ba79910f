#!/usr/bin/env python3
"""Writes attn_dkdv128_stream.h: the step loop of bwd_dkdv128_kernel (attention
backward, dK and dV, d = 128, one wave per SIMD) as one inline-asm stream.

    python gen_dkdv128_stream.py [SPLIT] [OUT] [--stats] [--show]

Scheduling, wait states, LDS waits and checks as in gen_dq128_stream.py.

Per wave: 32 keys (K^T and V^T operands in AGPRs), accumulating dK^T and dV^T
over the steps of its work group: one step is one 64-query tile of one query
head (two blocks qb0, qb1 of 32 queries), the tiles from the last down, so
that the work groups of one XCD read the same tiles at about the same time. Per step t, 64 MFMAs:
  M0-15  G1: S(t, qb0) = Q K^T, dP(t, qb0) = dO V^T          (set A)
  M16-31 G2: dV^T += dO^T P, dK^T += Q^T dS  of (t-1, qb1)   (set B)
  M32-47 G3: S(t, qb1), dP(t, qb1)                           (set B)
  M48-63 G4: dV^T, dK^T of (t, qb0)                          (set A)
VALU streams: X = P and dS of (t, qb0) (after M15, before G4); Y = P and dS
of (t, qb1): head after M47, tail before M16 of step t+1 (SPLIT = its pairs
in the head). P = exp2(S c - lse2) and dS = P (dP - D), each rounded to bf16
pairs as the B operands of G2 / G4; lse2 and D per query come from LDS.
LDS (3 stages; Q tiles, then dO tiles, then the (lse2, D) pairs): Q and dO
tiles of 64 rows of 320 bytes (chunks swizzled by row quad), read as rows (A
operands of S and dP) and transposed (A operands of dV^T and dK^T). In step
t: the transposed reads of (t-1, qb1) (stage t-1) in G1, one barrier after
G2, then the DMA of step t+2 into stage t-1 and the rows of step t+1.
"""
import sys
from pathlib import Path

sys.path.insert(0, str(Path(__file__).resolve().parent))
from gen_fwd128_stream import (MF, NEG_INF, Ins, vr, ar, vset, aset, schedule, fix_block,  # noqa: E402
                               splice_checks, fmt)
from gen_dq128_stream import insert_lgkm_waits  # noqa: E402

# AGPRs
DK, DV = 0, 64           # dK^T[db], dV^T[db] at +16 db
KF, VF = 128, 160        # K^T / V^T B operands [kk] at +4 kk
TQ, TD = 192, 224        # Q^T / dO^T operands [db][jj] at +8 db + 4 jj
# VGPRs (fixed, v64-v255; v0-v63 are left to the compiler)
SETS = [dict(L=176, S=208, P=224, PP=240, DS=248),    # set A: qb0 of step t
        dict(L=96, S=128, P=144, PP=160, DS=168)]     # set B: qb1
# L: (lse2, D) of the 16 queries (32, pair k at +2 k); S: scores -> P (fp32,
# 16); P: dP -> dS (16); PP: P bf16 pairs (8, jj at +4); DS: dS bf16 pairs (8)
QR, DR = 64, 80          # Q / dO row rings: slot s at +4 s
_SIZES = dict(L=32, S=16, P=16, PP=8, DS=8)
_spans = [(QR, 16), (DR, 16)] + [(st[k], n) for st in SETS for k, n in _SIZES.items()]
assert sorted(x for b, n in _spans for x in range(b, b + n)) == list(range(64, 256)), "fixed VGPRs overlap"
# SGPRs
SI, SG, STI, SG2, STMP, SINC, SINCL, SLIM, SCMP = 84, 85, 86, 87, 88, 89, 90, 91, 92   # SCMP: s[92:93]

TILE = 20480             # bytes of a Q (or dO) tile: 64 rows of 320
D_REGION = 3 * TILE      # the dO tiles follow the 3 Q tiles
L_REGION = 6 * TILE      # then the (lse2, D) pairs: 4 KiB per stage, 1 KiB per wave
LST = 4096
NST = 3
LDS_LAT = int(__import__("os").environ.get("DK_LDS_LAT", "3"))
DMA_DEADLINE = int(__import__("os").environ.get("DK_DMA_DL", "40"))


# ---------------------------------------------------------------- MFMAs
def sdp_group(st):
    s = SETS[st]
    out = []
    for kk in range(8):
        slot = kk % 4
        q, d = QR + 4 * slot, DR + 4 * slot
        for (acc, a, b) in ((s["S"], q, KF + 4 * kk), (s["P"], d, VF + 4 * kk)):
            c = "0" if kk == 0 else vr(acc, 16)
            out.append(Ins(f"{MF} {vr(acc, 16)}, {vr(a, 4)}, {ar(b, 4)}, {c}", "mfma",
                           rd=vset(a, 4) | aset(b, 4) | (set() if kk == 0 else vset(acc, 16)), wr=vset(acc, 16)))
    return out


def dkdv_group(st):
    s = SETS[st]
    out = []
    for jj in range(2):
        for db in range(4):
            for (acc, a, b) in ((DV + 16 * db, TD + 8 * db + 4 * jj, s["PP"] + 4 * jj),
                                (DK + 16 * db, TQ + 8 * db + 4 * jj, s["DS"] + 4 * jj)):
                out.append(Ins(f"{MF} {ar(acc, 16)}, {ar(a, 4)}, {vr(b, 4)}, {ar(acc, 16)}", "mfma",
                               rd=aset(acc, 16) | aset(a, 4) | vset(b, 4), wr=aset(acc, 16)))
    return out


def mfmas():
    out = sdp_group(0) + dkdv_group(1) + sdp_group(1) + dkdv_group(0)
    for i, m in enumerate(out):
        m.name = f"M{i}"
    return out


# ---------------------------------------------------------------- P and dS
def pdsa(st, pairs):
    """P and dS of set st for register pairs p (registers 2p, 2p + 1)."""
    s = SETS[st]
    items = []
    for p in pairs:
        r0, r1 = 2 * p, 2 * p + 1
        s0, s1 = s["S"] + r0, s["S"] + r1
        d0, d1 = s["P"] + r0, s["P"] + r1
        l0, l1 = s["L"] + 2 * r0, s["L"] + 2 * r1          # lse2; D at +1
        pp, ds = s["PP"] + p, s["DS"] + p
        items.append(Ins(f"v_fma_f32 v{s0}, v{s0}, %[c], -v{l0}", rd={f"v{s0}", f"v{l0}"}, wr={f"v{s0}"}))
        items.append(Ins(f"v_fma_f32 v{s1}, v{s1}, %[c], -v{l1}", rd={f"v{s1}", f"v{l1}"}, wr={f"v{s1}"}))
        items.append(Ins(f"v_exp_f32 v{s0}, v{s0}", "trans", rd={f"v{s0}"}, wr={f"v{s0}"}, slots=2))
        items.append(Ins(f"v_exp_f32 v{s1}, v{s1}", "trans", rd={f"v{s1}"}, wr={f"v{s1}"}, slots=2))
        items.append(Ins(f"v_sub_f32 v{d0}, v{d0}, v{l0 + 1}", rd={f"v{d0}", f"v{l0 + 1}"}, wr={f"v{d0}"}))
        items.append(Ins(f"v_sub_f32 v{d1}, v{d1}, v{l1 + 1}", rd={f"v{d1}", f"v{l1 + 1}"}, wr={f"v{d1}"}))
        items.append(Ins(f"v_cvt_pk_bf16_f32 v{pp}, v{s0}, v{s1}", rd={f"v{s0}", f"v{s1}"}, wr={f"v{pp}"}))
        items.append(Ins(f"v_mul_f32 v{d0}, v{s0}, v{d0}", rd={f"v{s0}", f"v{d0}"}, wr={f"v{d0}"}))
        items.append(Ins(f"v_mul_f32 v{d1}, v{s1}, v{d1}", rd={f"v{s1}", f"v{d1}"}, wr={f"v{d1}"}))
        items.append(Ins(f"v_cvt_pk_bf16_f32 v{ds}, v{d0}, v{d1}", rd={f"v{d0}", f"v{d1}"}, wr={f"v{ds}"}))
    return items


def mask_block(st, lab):
    """Out of line: a block that is not full for every key of the wave. Score
    register r of lane (key vk, half hh) holds query q0b + e(r), e(r) =
    reg_key_offset(r / 4, hh) + r % 4 (the byte r / 4 of %[off] holds the first
    term), q0b = 64 qt + 32 qb for the step's query tile qt = (qtop - 64 STI) / 64;
    it stays when 0 <= q - vk < W (unsigned compare, W = 2^31 - 1 without a
    window) and q < Lv, else it becomes -inf. The step past the last (tile
    qt_begin - 1) has every query below every key."""
    s = SETS[st]
    t0, t1, t2, t3, t4 = (s["DS"] + x for x in range(5))     # free until this block's dS
    b = [Ins(f"{lab}:", "label"),
         Ins(f"s_lshl_b32 s{STMP}, s{STI}, 6\n\ts_sub_u32 s{STMP}, %[qtop], s{STMP}" +
             (f"\n\ts_add_u32 s{STMP}, s{STMP}, 32" if st else "") +
             f"\n\ts_sub_u32 s{SLIM}, %[Lv], s{STMP}", "salu"),
         Ins(f"v_sub_u32 v{t0}, s{STMP}, %[vk]", rd={"%[vk]"}, wr={f"v{t0}"}),
         Ins(f"v_mov_b32 v{t3}, {NEG_INF}", wr={f"v{t3}"})]
    for g in range(4):
        b.append(Ins(f"v_bfe_u32 v{t1}, %[off], {8 * g}, 8", rd={"%[off]"}, wr={f"v{t1}"}))
        for i in range(4):
            e = s["S"] + 4 * g + i
            q = t1
            if i:
                b.append(Ins(f"v_add_u32 v{t2}, {i}, v{t1}", rd={f"v{t1}"}, wr={f"v{t2}"}))
                q = t2
            b.append(Ins(f"v_add_u32 v{t4}, v{q}, v{t0}", rd={f"v{q}", f"v{t0}"}, wr={f"v{t4}"}))
            b.append(Ins(f"v_cmp_gt_u32 vcc, %[W], v{t4}", rd={f"v{t4}"}, wr={"vcc"}))
            b.append(Ins(f"v_cmp_gt_i32_e64 s[{SCMP}:{SCMP + 1}], s{SLIM}, v{q}\n\t"
                         f"s_and_b64 vcc, vcc, s[{SCMP}:{SCMP + 1}]", rd={f"v{q}", "vcc"}, wr={"vcc"}))
            b.append(Ins(f"v_cndmask_b32 v{e}, v{t3}, v{e}, vcc", rd={f"v{t3}", f"v{e}", "vcc"}, wr={f"v{e}"}))
    b.append(Ins(f"s_branch {lab}_r", "salu"))
    return b


def mask_check(st, lab):
    """Steps whose query tile is full for every key of the wave (processed
    indices fd .. fd + fc - 1) fall through; the rest, the step that closes the
    stream included, go out of line."""
    s = SETS[st]
    br = Ins(f"s_sub_u32 s{STMP}, s{STI}, %[fd]\n\ts_cmp_lt_u32 s{STMP}, %[fc]\n\ts_cbranch_scc0 {lab}\n{lab}_r:",
             "br", rd=vset(s["S"], 16), wr=vset(s["S"], 16) | {"vcc"} | vset(s["DS"], 5), slots=3,
             name=f"mchk{st}")
    br.block = fix_block(mask_block(st, lab))
    return br


# ---------------------------------------------------------------- LDS / DMA
def rows_read(stage, qb, kk, dout, after, name):
    reg = (DR if dout else QR) + 4 * (kk % 4)
    off = stage * TILE + 32 * 320 * qb + 64 * (kk // 2)
    base = f"%[{'g' if dout else 'q'}{'o' if kk % 2 else 'e'}]"
    return Ins(f"ds_read_b128 {vr(reg, 4)}, {base} offset:{off}", "lds", wr=vset(reg, 4), after=after, name=name)


def ring_reads(stage, qb, kks, prev_group, tag):
    """Rows kk into ring slot kk % 4, after the two MFMAs of the S/dP group at
    prev_group (None: the previous step) that read the slot's previous
    contents, and two more."""
    items = []
    for kk in kks:
        for dout in (False, True):
            after = 1 if prev_group is None else prev_group + 2 * ((kk + 4) % 8) + (1 if dout else 0) + 2
            items.append(rows_read(stage, qb, kk, dout, after, f"{tag}{'D' if dout else 'Q'}{kk}"))
    return items


def tr_reads(stage, qb, prev_group, tag):
    """Q^T and dO^T operands [db][jj] of block qb: two transposed reads each, from
    base <q|d><t><jj> at 64 db; each after the MFMA of the dV/dK group at
    prev_group (None: the previous step) that read the operand, and two more."""
    items = []
    for jj in range(2):
        for db in range(4):
            for dout in (True, False):
                reg = (TD if dout else TQ) + 8 * db + 4 * jj
                k = 8 * jj + 2 * db + (0 if dout else 1)
                after = 1 if prev_group is None else prev_group + k + 2
                for t in range(2):
                    off = stage * TILE + 32 * 320 * qb + 64 * db
                    items.append(Ins(f"ds_read_b64_tr_b16 {ar(reg + 2 * t, 2)}, %[{'d' if dout else 'q'}{t}{jj}] "
                                     f"offset:{off}", "lds", wr=aset(reg + 2 * t, 2), after=after,
                                     name=f"{tag}T{int(dout)}{db}{jj}{t}"))
    return items


def pair_reads(stage, st, qb, after, tag):
    """(lse2, D) of the 16 queries of the lane's registers: 8 broadcast reads
    (bases lp0 / lp1 hold the pair region and the lane half's 1 KiB)."""
    s = SETS[st]
    items = []
    for half in range(2):
        for k, off in enumerate((0, 16, 64, 80)):
            reg = s["L"] + 16 * half + 4 * k
            o = stage * LST + 2048 * qb + off
            items.append(Ins(f"ds_read_b128 {vr(reg, 4)}, %[lp{half}] offset:{o}", "lds", wr=vset(reg, 4),
                             after=after, name=f"{tag}L{half}{k}"))
    return items


def dma(dst):
    """Step t+2 into stage dst: 5 Q and 5 dO chunks and the wave's pair chunk;
    then the offsets advance to step t+3 (next head, or next tile after the
    last head; past the last step out of range)."""
    items = [Ins(f"s_add_u32 s{SG2}, s{SG2}, 1\n\ts_cmp_eq_u32 s{SG2}, %[G]\n\t"
                 f"s_cselect_b32 s{SINC}, %[incw], 256\n\ts_cselect_b32 s{SINCL}, %[inclw], %[inclh]\n\t"
                 f"s_cselect_b32 s{SG2}, 0, s{SG2}\n\ts_add_u32 s{STMP}, s{SI}, 3\n\ts_cmp_eq_u32 s{STMP}, %[T]\n\t"
                 f"s_cselect_b32 s{STMP}, 0x80000000, 0\n\ts_add_u32 s{SINC}, s{SINC}, s{STMP}\n\t"
                 f"s_add_u32 s{SINCL}, s{SINCL}, s{STMP}", "salu", slots=10, name="sinc")]
    for x in range(5):
        for dout in (False, True):
            off = (D_REGION if dout else 0) + dst * TILE + 4096 * x
            items.append(Ins(f"s_add_u32 m0, %[lw], {off}", "salu", wr={"m0"}, name=f"m0_{x}{int(dout)}"))
            items.append(Ins(f"buffer_load_dwordx4 %[cf{x}], %[{'rd' if dout else 'rq'}], 0 offen lds", "vmem",
                             rd={"m0", f"%[cf{x}]"}, name=f"dma{x}{int(dout)}"))
    items.append(Ins(f"s_add_u32 m0, %[lw], {L_REGION + dst * LST}", "salu", wr={"m0"}, name="m0_l"))
    items.append(Ins("buffer_load_dwordx4 %[cl], %[rl], 0 offen lds", "vmem", rd={"m0", "%[cl]"}, name="dmal"))
    for x in range(5):
        items.append(Ins(f"v_add_u32 %[cf{x}], s{SINC}, %[cf{x}]", rd={f"%[cf{x}]"}, wr={f"%[cf{x}]"},
                         name=f"inc{x}"))
    items.append(Ins(f"v_add_u32 %[cl], s{SINCL}, %[cl]", rd={"%[cl]"}, wr={"%[cl]"}, name="incl"))
    return items


def lds_deadlines(mf, items):
    for it in items:
        for k, m in enumerate(mf):
            if k > it.after and m.rd & it.wr:
                it.fixed_deadline = max(it.after + 1, k - LDS_LAT)
                break


def build_iteration(stage, h_split):
    mf = mfmas()
    prv, nxt = (stage - 1) % NST, (stage + 1) % NST
    lab = f"L%=_{stage}"
    trG1 = tr_reads(prv, 1, None, "a")            # (t-1, qb1) operands for G2
    rA = ring_reads(stage, 0, range(4, 8), 0, "a")  # qb0 rows kk 4-7 for G1
    lA = pair_reads(stage, 0, 0, -1, "a")         # (t, qb0) pairs for X
    rB0 = ring_reads(stage, 1, range(0, 4), 0, "b")   # qb1 rows kk 0-3 for G3
    rB1 = ring_reads(stage, 1, range(4, 8), 32, "c")  # qb1 rows kk 4-7
    lB = pair_reads(stage, 1, 1, 15, "b")         # (t, qb1) pairs for Y (after the Y tail of t-1)
    trG3 = tr_reads(stage, 0, 16, "e")            # (t, qb0) operands for G4
    rN = ring_reads(nxt, 0, range(0, 4), 32, "n")  # step t+1 qb0 rows kk 0-3
    bar = Ins("s_waitcnt vmcnt(0)\n\ts_barrier", "sync", after=31, slots=2, name="bar")
    bar.fixed_deadline = 36
    dm = dma(prv)
    for it in dm:
        if it.name.startswith("m0_") or it.name == "sinc":
            it.deps = [bar]
        it.fixed_deadline = DMA_DEADLINE + (6 if it.name.startswith("inc") else 0)
    for it in rN:
        it.deps = [bar]
    lds = trG1 + rA + lA + rB0 + rB1 + lB + trG3 + rN
    lds_deadlines(mf, lds)
    x = [mask_check(0, f"{lab}_mx")] + pdsa(0, range(8))
    for it in x:
        it.after = max(it.after, 15)
    yt = pdsa(1, range(h_split, 8))
    yh = [mask_check(1, f"{lab}_my")] + pdsa(1, range(h_split))
    for it in yh:
        it.after = max(it.after, 47)
    # the (t, qb1) pairs overwrite what the Y tail of t-1 still reads
    for it in lB:
        it.deps = [yt[-1]] if yt else []
    # vector consumers of the pairs come after their reads (the lgkm waits then
    # cover them); the reads issue a few MFMAs ahead of the first consumer
    for reads, items, first in ((lA, x, 15), (lB, yh, 47)):
        for it in reads:
            it.fixed_deadline = first - LDS_LAT
        for it in items:
            it.deps = it.deps + [r for r in reads if r.wr & it.rd]
    streams = [yt, x, trG1, rA, lA, rB0, rB1, lB, trG3, [bar], rN, dm, yh]
    prio = [0, 4, 1, 2, 3, 5, 6, 7, 8, 9, 10, 11, 12]
    loop = [Ins(f"s_add_u32 s{SI}, s{SI}, 1\n\ts_add_u32 s{SG}, s{SG}, 1\n\ts_cmp_eq_u32 s{SG}, %[G]\n\t"
                f"s_cselect_b32 s{SG}, 0, s{SG}\n\ts_cselect_b32 s{STMP}, 1, 0\n\ts_add_u32 s{STI}, s{STI}, s{STMP}\n\t"
                f"s_cmp_gt_u32 s{SI}, %[T]\n\ts_cbranch_scc1 L%=_fin", "salu", slots=8, name="loop")]
    out, t, mfree = schedule(mf, streams, prio, loop)
    return out, t


def main():
    h_split = int(sys.argv[1]) if len(sys.argv) > 1 and sys.argv[1].isdigit() else 0
    allseq, blocks = [], []
    total = 0
    for stage in range(NST):
        seq, t = build_iteration(stage, h_split)
        seq = insert_lgkm_waits(seq)
        errs = splice_checks(seq)
        if errs:
            for e in errs[:20]:
                print("HAZARD", stage, e, file=sys.stderr)
            sys.exit(1)
        total = t
        allseq.append(seq)
        blocks += [it.block for it in seq if it.block]
    nm = sum(1 for it in allseq[0] if it.kind == "mfma")
    nw = sum(1 for it in allseq[0] if it.name == "lgkm")
    print(f"// h_split={h_split} est cycles/iter={total} mfma={nm * 32} util={nm * 32 / total:.3f} "
          f"instrs={len(fmt(allseq[0]))} lgkm_waits={nw}", file=sys.stderr)
    if "--stats" in sys.argv:
        return
    lines = []
    for stage in range(NST):
        lines.append(f"L%=_{stage}_top:")
        lines += fmt(allseq[stage])
    lines.append("s_branch L%=_0_top")
    for b in blocks:
        lines += fmt(b)
    lines.append("L%=_fin:")

    # Prologue: dK^T = dV^T = 0; the state after a step -1 with no admitted
    # query: set B scores -inf, dP 0, pairs 0, its P / dS pairs 0 (so the first
    # G2 adds nothing); then the first step's qb0 rows kk 0-3.
    B = SETS[1]
    z, ni, one = vr(SETS[0]["DS"], 4), vr(SETS[0]["PP"], 4), vr(SETS[0]["PP"] + 4, 4)
    pro = [f"s_mov_b32 s{SI}, 0", f"s_mov_b32 s{SG}, 0", f"s_mov_b32 s{STI}, 0", f"s_mov_b32 s{SG2}, 2", "s_cmp_le_u32 %[G], 2", f"s_cselect_b32 s{SG2}, 0, s{SG2}"]   # 2 mod G
    pro += [f"v_mov_b32 v{SETS[0]['DS'] + x}, 0" for x in range(4)]
    pro += [f"v_mov_b32 v{SETS[0]['PP'] + x}, 0xff80ff80" for x in range(4)]
    pro += [f"v_mov_b32 v{SETS[0]['PP'] + 4 + x}, 0x3f803f80" for x in range(4)]
    pro += [f"v_mov_b32 v{B['PP'] + x}, 0" for x in range(8)]
    pro += [f"v_mov_b32 v{B['DS'] + x}, 0" for x in range(8)]
    pro += [f"v_mov_b32 v{B['L'] + x}, 0" for x in range(32)]
    pro += ["s_nop 2"]
    pro += [f"{MF} {vr(B['S'], 16)}, {ni}, {one}, 0", f"{MF} {vr(B['P'], 16)}, {z}, {z}, 0"]
    pro += [f"{MF} {ar(16 * x, 16)}, {z}, {z}, 0" for x in range(8)]
    for kk in range(4):
        for dout in (False, True):
            pro.append(fmt([rows_read(0, 0, kk, dout, -1, "p")])[0])
    pro += ["s_waitcnt lgkmcnt(0)", "s_nop 7", "s_nop 7"]

    dflt = Path(__file__).resolve().parent / "attn_dkdv128_stream.h"
    outp = sys.argv[2] if len(sys.argv) > 2 and not sys.argv[2].startswith("--") else dflt
    with open(outp, "w") as out:
        out.write("// Generated by gen_dkdv128_stream.py: the step loop of bwd_dkdv128_kernel (attn_bwd.hip)\n"
                  f"// as one instruction stream (Y split {h_split}). Regenerate rather than edit.\n"
                  "#pragma once\n\n")
        for name, body in (("SFA_DKDV128_PROLOGUE", pro), ("SFA_DKDV128_LOOP", lines)):
            out.write(f"#define {name} \\\n")
            for ln in body:
                out.write(f'  "{ln}\\n" \\\n')
            out.write("\n")
        cv = ", ".join(f'"v{x}"' for x in range(64, 256))
        out.write(f"#define SFA_DKDV128_CLOBBER_V {cv}\n")
        ca = ", ".join(f'"a{x}"' for x in range(TQ, 256))
        out.write(f"#define SFA_DKDV128_CLOBBER_A {ca}\n")
    print(f"// {len(lines)} lines", file=sys.stderr)
    if "--show" in sys.argv:
        for ln in fmt(allseq[0]):
            print(ln)


if __name__ == "__main__":
    main()
