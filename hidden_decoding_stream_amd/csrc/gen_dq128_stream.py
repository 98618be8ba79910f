#!/usr/bin/env python3
"""Writes attn_dq128_stream.h: the tile loop of bwd_dq128_kernel (attention
backward, dQ, d = 128, one wave per SIMD) as one inline-asm instruction stream.

    python gen_dq128_stream.py [SPLIT] [OUT] [--stats] [--show]

Scheduling, wait states and checks are those of gen_fwd128_stream.py (imported):
the MFMAs of a tile are fixed, every other instruction comes from in-order
streams placed greedily into the MFMA shadows, and each placement is checked
against the gfx950 wait states. New here: LDS reads land in register rings that
the MFMAs consume a few MFMAs later, so every consumer is preceded by the
s_waitcnt lgkmcnt that covers exactly its reads (LDS reads complete in order).

Per wave: 64 queries (QB0, QB1 of 32), one query head. Per 64-key tile t
(keys in two blocks kb0, kb1 of 32), 96 MFMAs:
  M0-31  A: S^T(t, kb0) = K Q^T, dP^T(t, kb0) = V dO^T, both QBs (v192-255)
  M32-47 B: dQ^T += K^T(t-1, kb1) dS^T(t-1, kb1)                   (a0-127)
  M48-79 C: S^T(t, kb1), dP^T(t, kb1)                              (v128-191)
  M80-95 D: dQ^T += K^T(t, kb0) dS^T(t, kb0)
VALU streams: X = dS of (t, kb0) (after M31, before D); Y = dS of (t, kb1):
head after M79 of iteration t, tail before M32 of iteration t+1 (SPLIT =
number of its 16 pairs in the head). dS = exp2(S c - lse2) (dP - D) in place,
rounded to bf16 pairs as the B operand of the dQ MFMAs.
LDS (3 stages, K then V regions): K and V tiles of 64 rows of 320 bytes with
the 16-byte chunks swizzled by row quad; K rows and V rows are read as MFMA A
operands (sigma order), K^T by transposed reads. In iteration t: the reads of
K^T(t-1, kb1) (stage t-1) in A, one barrier after B, then the DMA of tile t+2
into stage t-1 and the K / V rows of tile t+1 for the next A.
"""
import sys
from pathlib import Path

sys.path.insert(0, str(Path(__file__).resolve().parent))
from gen_fwd128_stream import (MF, NEG_INF, Ins, nop, vr, ar, vset, aset, hazard_ws, schedule,  # noqa: E402
                               fix_block, splice_checks, fmt)

# VGPRs (fixed; v0-v31 are left to the compiler for the asm's operands)
SX = [192, 208]     # S^T(kb0) of QB j
PX = [224, 240]     # dP^T(kb0)
SY = [128, 144]     # S^T(kb1)
PY = [160, 176]     # dP^T(kb1)
DS0 = 112           # dS^T(kb0) bf16: [j][jj] at DS0 + 8 j + 4 jj
DS1 = 96            # dS^T(kb1)
KT = 64             # K^T operands: [db][jj] at KT + 8 db + 4 jj
KR = 32             # K row ring: slot s at KR + 4 s
VRG = 48            # V row ring: slot s at VRG + 4 s
_spans = [(SX[0], 32), (PX[0], 32), (SY[0], 32), (PY[0], 32), (DS0, 16), (DS1, 16), (KT, 32), (KR, 16), (VRG, 16)]
assert sorted(x for b, n in _spans for x in range(b, b + n)) == list(range(32, 256)), "fixed VGPRs overlap"
# AGPRs
DQ = 0              # dQ^T[j][db] at DQ + 64 j + 16 db
QA = 128            # Q^T operands [j][kk] at QA + 32 j + 4 kk
DOA = 192           # dO^T operands [j][kk] at DOA + 32 j + 4 kk
# SGPRs
SI, STMP, SINC = 84, 85, 86

KST = 20480         # bytes per K (or V) stage: 64 rows of 320
V_REGION = 3 * KST  # the V stages follow the 3 K stages
NST = 3
LDS_LAT = int(__import__("os").environ.get("DQ_LDS_LAT", "3"))      # MFMAs from an LDS read to its first consumer
DMA_DEADLINE = int(__import__("os").environ.get("DQ_DMA_DL", "60"))  # the DMA of tile t+2 issues before this MFMA


def tr_temps(kb):
    """Mask temporaries: the dS registers of that key block are free while its mask applies."""
    b = DS0 if kb == 0 else DS1
    return b, b + 1, b + 2, b + 3


# ---------------------------------------------------------------- MFMAs
def sdp_group(kb, base_idx):
    """S^T and dP^T of key block kb for both QBs: 8 k-steps x (S0, S1, P0, P1)."""
    S = SX if kb == 0 else SY
    P = PX if kb == 0 else PY
    out = []
    for kk in range(8):
        slot = kk % 4
        k, v = KR + 4 * slot, VRG + 4 * slot
        for j in range(2):
            d = S[j]
            c = "0" if kk == 0 else vr(d, 16)
            q = QA + 32 * j + 4 * kk
            out.append(Ins(f"{MF} {vr(d, 16)}, {vr(k, 4)}, {ar(q, 4)}, {c}", "mfma",
                           rd=vset(k, 4) | aset(q, 4) | (set() if kk == 0 else vset(d, 16)), wr=vset(d, 16)))
        for j in range(2):
            d = P[j]
            c = "0" if kk == 0 else vr(d, 16)
            q = DOA + 32 * j + 4 * kk
            out.append(Ins(f"{MF} {vr(d, 16)}, {vr(v, 4)}, {ar(q, 4)}, {c}", "mfma",
                           rd=vset(v, 4) | aset(q, 4) | (set() if kk == 0 else vset(d, 16)), wr=vset(d, 16)))
    return out


def dq_group(ds):
    out = []
    for jj in range(2):
        for db in range(4):
            for j in range(2):
                o = DQ + 64 * j + 16 * db
                a = KT + 8 * db + 4 * jj
                b = ds + 8 * j + 4 * jj
                out.append(Ins(f"{MF} {ar(o, 16)}, {vr(a, 4)}, {vr(b, 4)}, {ar(o, 16)}", "mfma",
                               rd=aset(o, 16) | vset(a, 4) | vset(b, 4), wr=aset(o, 16)))
    return out


def mfmas():
    out = sdp_group(0, 0) + dq_group(DS1) + sdp_group(1, 48) + dq_group(DS0)
    for i, m in enumerate(out):
        m.name = f"M{i}"
    return out


# ---------------------------------------------------------------- dS pieces
def ds_pairs(kb, pairs):
    """dS of key block kb for pair indices p (0..15: QB p // 8, registers 2 (p % 8), +1)."""
    S = SX if kb == 0 else SY
    P = PX if kb == 0 else PY
    DS = DS0 if kb == 0 else DS1
    items = []
    for p in pairs:
        j, q = divmod(p, 8)
        s0, s1 = S[j] + 2 * q, S[j] + 2 * q + 1
        p0, p1 = P[j] + 2 * q, P[j] + 2 * q + 1
        dst = DS + 8 * j + q
        lse, dd = f"%[l{j}]", f"%[d{j}]"
        items.append(Ins(f"v_fma_f32 v{s0}, v{s0}, %[c], -{lse}", rd={f"v{s0}", lse}, wr={f"v{s0}"}))
        items.append(Ins(f"v_fma_f32 v{s1}, v{s1}, %[c], -{lse}", rd={f"v{s1}", lse}, wr={f"v{s1}"}))
        items.append(Ins(f"v_exp_f32 v{s0}, v{s0}", "trans", rd={f"v{s0}"}, wr={f"v{s0}"}, slots=2))
        items.append(Ins(f"v_exp_f32 v{s1}, v{s1}", "trans", rd={f"v{s1}"}, wr={f"v{s1}"}, slots=2))
        items.append(Ins(f"v_sub_f32 v{p0}, v{p0}, {dd}", rd={f"v{p0}", dd}, wr={f"v{p0}"}))
        items.append(Ins(f"v_sub_f32 v{p1}, v{p1}, {dd}", rd={f"v{p1}", dd}, wr={f"v{p1}"}))
        items.append(Ins(f"v_mul_f32 v{p0}, v{s0}, v{p0}", rd={f"v{s0}", f"v{p0}"}, wr={f"v{p0}"}))
        items.append(Ins(f"v_mul_f32 v{p1}, v{s1}, v{p1}", rd={f"v{s1}", f"v{p1}"}, wr={f"v{p1}"}))
        items.append(Ins(f"v_cvt_pk_bf16_f32 v{dst}, v{p0}, v{p1}", rd={f"v{p0}", f"v{p1}"}, wr={f"v{dst}"}))
    return items


def mask_block(kb, lab):
    """Out of line: a tile that is not full for every query of the wave. Score
    register r of lane (query vq, half hh) holds key key0 + o(r), o(r) =
    reg_key_offset(r / 4, hh) + r % 4 (the byte r / 4 of %[off] holds the first
    term); it stays when vq - key < W (unsigned: 0 <= vq - key < W, W = 2^31 - 1
    without a window), else it becomes -inf."""
    S = SX if kb == 0 else SY
    t0, t1, t2, t3 = tr_temps(kb)
    b = [Ins(f"{lab}:", "label"),
         Ins(f"s_lshl_b32 s{STMP}, s{SI}, 6\n\ts_add_u32 s{STMP}, s{STMP}, %[kb0]" +
             (f"\n\ts_add_u32 s{STMP}, s{STMP}, 32" if kb else ""), "salu"),
         Ins(f"v_mov_b32 v{t3}, {NEG_INF}", wr={f"v{t3}"})]
    for j in range(2):
        b.append(Ins(f"v_subrev_u32 v{t0}, s{STMP}, %[vq{j}]", rd={f"%[vq{j}]"}, wr={f"v{t0}"}))
        for g in range(4):
            b.append(Ins(f"v_bfe_u32 v{t1}, %[off], {8 * g}, 8", rd={"%[off]"}, wr={f"v{t1}"}))
            b.append(Ins(f"v_sub_u32 v{t1}, v{t0}, v{t1}", rd={f"v{t0}", f"v{t1}"}, wr={f"v{t1}"}))
            for i in range(4):
                e = S[j] + 4 * g + i
                d = t1
                if i:
                    b.append(Ins(f"v_sub_u32_e64 v{t2}, v{t1}, {i}", rd={f"v{t1}"}, wr={f"v{t2}"}))
                    d = t2
                b.append(Ins(f"v_cmp_gt_u32 vcc, %[W], v{d}", rd={f"v{d}"}, wr={"vcc"}))
                b.append(Ins(f"v_cndmask_b32 v{e}, v{t3}, v{e}, vcc", rd={f"v{t3}", f"v{e}", "vcc"}, wr={f"v{e}"}))
    b.append(Ins(f"s_branch {lab}_r", "salu"))
    return b


def mask_check(kb, lab):
    """Tiles in the wave's full range (every key of the tile admitted for every
    query of the wave: relative tile index fd .. fd + fc - 1) fall through; the
    rest, the extra tile that closes the stream included, go out of line."""
    S = SX if kb == 0 else SY
    br = Ins(f"s_sub_u32 s{STMP}, s{SI}, %[fd]\n\ts_cmp_lt_u32 s{STMP}, %[fc]\n\ts_cbranch_scc0 {lab}\n{lab}_r:",
             "br", rd=vset(S[0], 16) | vset(S[1], 16), wr=vset(S[0], 16) | vset(S[1], 16) | {"vcc"}
             | set(f"v{x}" for x in tr_temps(kb)), slots=3, name=f"mchk{kb}")
    br.block = fix_block(mask_block(kb, lab))
    return br


# ---------------------------------------------------------------- LDS / DMA
def kbase(kk, v=False):
    return f"%[{'v' if v else 'k'}{'o' if kk % 2 else 'e'}]"


def rows_read(st, kb, kk, v, after, name):
    reg = (VRG if v else KR) + 4 * (kk % 4)
    off = st * KST + 32 * 320 * kb + 64 * (kk // 2)
    return Ins(f"ds_read_b128 {vr(reg, 4)}, {kbase(kk, v)} offset:{off}", "lds", wr=vset(reg, 4), after=after,
               name=name)


def ring_reads(st, kb, kks, prev_group, tag):
    """Rows kk of key block kb into ring slot kk % 4, each after the MFMAs that
    read the slot's previous contents (k-step kk +- 4 of the S/dP group starting
    at MFMA prev_group; None: the previous iteration) and two more."""
    items = []
    for kk in kks:
        for v in (False, True):
            if prev_group is None:
                after = 1
            else:
                pk = (kk + 4) % 8
                after = prev_group + 4 * pk + (3 if v else 1) + 2
            items.append(rows_read(st, kb, kk, v, after, f"{tag}{'V' if v else 'K'}{kk}"))
    return items


def kt_reads(st, kb, prev_group, tag):
    """K^T operands [db][jj] of key block kb in stage st: two transposed reads each
    (t = 0, 1), from base tr<t><jj> at 64 db; each after the two dQ MFMAs that
    read the operand's previous contents (group starting at MFMA prev_group;
    None: the previous iteration) and two more."""
    items = []
    for jj in range(2):
        for db in range(4):
            reg = KT + 8 * db + 4 * jj
            after = 1 if prev_group is None else prev_group + 8 * jj + 2 * db + 1 + 2
            for t in range(2):
                off = st * KST + 32 * 320 * kb + 64 * db
                items.append(Ins(f"ds_read_b64_tr_b16 {vr(reg + 2 * t, 2)}, %[t{t}{jj}] offset:{off}", "lds",
                                 wr=vset(reg + 2 * t, 2), after=after, name=f"{tag}T{db}{jj}{t}"))
    return items


def dma(st_dst):
    items = [Ins(f"s_add_u32 s{STMP}, s{SI}, 3\n\ts_cmp_eq_u32 s{STMP}, %[T]\n\t"
                 f"s_cselect_b32 s{STMP}, 0x80000000, 0\n\ts_add_u32 s{SINC}, s{STMP}, %[tstride]", "salu",
                 slots=4, name="sinc")]
    for x in range(5):
        for v in (False, True):
            off = (V_REGION if v else 0) + st_dst * KST + 4096 * x
            items.append(Ins(f"s_add_u32 m0, %[lw], {off}", "salu", wr={"m0"}, name=f"m0_{x}{int(v)}"))
            items.append(Ins(f"buffer_load_dwordx4 %[cf{x}], %[{'rv' if v else 'rk'}], 0 offen lds", "vmem",
                             rd={"m0", f"%[cf{x}]"}, name=f"dma{x}{int(v)}"))
    for x in range(5):
        items.append(Ins(f"v_add_u32 %[cf{x}], s{SINC}, %[cf{x}]", rd={f"%[cf{x}]"}, wr={f"%[cf{x}]"},
                         name=f"inc{x}"))
    return items


def lds_deadlines(mf, items):
    """An LDS read must issue at least LDS_LAT MFMAs before the first MFMA reading it."""
    for it in items:
        for k, m in enumerate(mf):
            if k > it.after and m.rd & it.wr:
                it.fixed_deadline = max(it.after + 1, k - LDS_LAT)
                break


def build_iteration(st, h_split):
    """One tile iteration with tile t in stage st (copy st of the unrolled loop)."""
    mf = mfmas()
    prv, nxt = (st - 1) % NST, (st + 1) % NST
    lab = f"L%=_{st}"
    ktA = kt_reads(prv, 1, None, "a")                         # K^T(t-1, kb1) for B
    kvA = ring_reads(st, 0, range(4, 8), 0, "a")              # rows kk 4-7 for A
    kvC0 = ring_reads(st, 1, range(0, 4), 0, "c")             # rows kk 0-3 for C
    kvC1 = ring_reads(st, 1, range(4, 8), 48, "d")            # rows kk 4-7 for C
    ktC = kt_reads(st, 0, 32, "e")                            # K^T(t, kb0) for D
    kvN = ring_reads(nxt, 0, range(0, 4), 48, "n")            # rows kk 0-3 of tile t+1 for the next A
    bar = Ins("s_waitcnt vmcnt(0)\n\ts_barrier", "sync", after=47, slots=2, name="bar")
    bar.fixed_deadline = 60
    dm = dma(prv)
    for it in dm:
        if it.name.startswith("m0_") or it.name == "sinc":
            it.deps = [bar]
        # issued right after the barrier: the next barrier waits for it
        it.fixed_deadline = DMA_DEADLINE + (6 if it.name.startswith("inc") else 0)
    for it in kvN:
        it.deps = [bar]
    lds = ktA + kvA + kvC0 + kvC1 + ktC + kvN
    lds_deadlines(mf, lds)
    # X: dS(t, kb0); Y: dS(t, kb1), tail of the previous tile first
    x = [mask_check(0, f"{lab}_mx")] + ds_pairs(0, range(16))
    for it in x:
        it.after = max(it.after, 31)
    yt = ds_pairs(1, range(h_split, 16))
    yh = [mask_check(1, f"{lab}_my")] + ds_pairs(1, range(h_split))
    for it in yh:
        it.after = max(it.after, 79)
    streams = [yt, x, ktA, kvA, kvC0, kvC1, ktC, [bar], kvN, dm, yh]
    prio = [0, 3, 1, 2, 4, 5, 6, 7, 8, 9, 10]
    loop = [Ins(f"s_add_u32 s{SI}, s{SI}, 1\n\ts_cmp_gt_u32 s{SI}, %[T]\n\ts_cbranch_scc1 L%=_fin", "salu",
                slots=3, name="loop")]
    out, t, mfree = schedule(mf, streams, prio, loop)
    return out, t


LGKM_AHEAD = int(__import__("os").environ.get("LGKM_AHEAD", "4"))   # MFMAs a wait also covers


def insert_lgkm_waits(seq, ahead=None):
    """Before each instruction that reads (or overwrites) registers an outstanding
    LDS read writes, wait until that read has completed; the wait also covers
    the reads already issued that the instructions up to `ahead` MFMAs further
    need (fewer waits, each a little earlier). The sequence is one iteration;
    it runs after a copy of itself, so reads issued late in the previous
    iteration are outstanding at the start."""
    ahead = LGKM_AHEAD if ahead is None else ahead

    def run(prefix_outstanding, body, emit):
        outstanding = list(prefix_outstanding)    # in issue order: sets of written registers
        out = []
        for pos, it in enumerate(body):
            if it.kind in ("label",):
                out.append(it)
                continue
            regs = it.rd | it.wr
            need = -1
            for i, w in enumerate(outstanding):
                if w & regs:
                    need = i
            if need >= 0 and it.kind != "lds" and ahead > 0:
                nm = 0
                for nxt in body[pos + 1:]:
                    if nxt.kind == "mfma":
                        nm += 1
                        if nm > ahead:
                            break
                    for i, w in enumerate(outstanding):
                        if w & (nxt.rd | nxt.wr):
                            need = max(need, i)
            if need >= 0 and it.kind != "lds":
                keep = len(outstanding) - need - 1
                out.append(Ins(f"s_waitcnt lgkmcnt({min(keep, 15)})", "sync", name="lgkm"))
                outstanding = outstanding[need + 1:]
            elif need >= 0:
                raise RuntimeError(f"LDS read {it} overwrites a register of a read in flight")
            if it.kind == "lds":
                outstanding.append(it.wr)
            if it.block:
                for b in it.block:
                    if b.kind != "label" and (b.rd | b.wr) & set().union(*outstanding) if outstanding else False:
                        raise RuntimeError(f"out-of-line block of {it.name} touches a register in flight")
            out.append(it)
        return out, outstanding
    _, tail = run([], seq, False)
    out, tail2 = run(tail, seq, True)
    assert [sorted(x) for x in tail] == [sorted(x) for x in tail2], "outstanding reads differ between iterations"
    return out


def main():
    h_split = int(sys.argv[1]) if len(sys.argv) > 1 and sys.argv[1].isdigit() else 8
    allseq, blocks = [], []
    total = 0
    for st in range(NST):
        seq, t = build_iteration(st, h_split)
        seq = insert_lgkm_waits(seq)
        errs = splice_checks(seq)
        if errs:
            for e in errs[:20]:
                print("HAZARD", st, e, file=sys.stderr)
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
    for st in range(NST):
        lines.append(f"L%=_{st}_top:")
        lines += fmt(allseq[st])
    lines.append("s_branch L%=_0_top")
    for b in blocks:
        lines += fmt(b)
    lines.append("L%=_fin:")

    # Prologue: dQ^T = 0; the state after a tile -1 with no admitted key: the kb1
    # scores -inf and dP 0 (their dS, formed in the first iteration's Y tail, are 0),
    # the dS^T(kb1) pairs of the Y head 0; then the first tile's kb0 rows kk 0-3.
    z, ni, one = vr(DS0, 4), vr(KT, 4), vr(KT + 4, 4)
    pro = [f"s_mov_b32 s{SI}, 0"]
    pro += [f"v_mov_b32 v{DS0 + x}, 0" for x in range(4)]
    pro += [f"v_mov_b32 v{KT + x}, 0xff80ff80" for x in range(4)]
    pro += [f"v_mov_b32 v{KT + 4 + x}, 0x3f803f80" for x in range(4)]
    pro += [f"v_mov_b32 v{DS1 + x}, 0" for x in range(16)]
    pro += ["s_nop 2"]
    pro += [f"{MF} {vr(SY[j], 16)}, {ni}, {one}, 0" for j in range(2)]
    pro += [f"{MF} {vr(PY[j], 16)}, {z}, {z}, 0" for j in range(2)]
    pro += [f"{MF} {ar(DQ + 16 * x, 16)}, {z}, {z}, 0" for x in range(8)]
    for kk in range(4):
        for v in (False, True):
            pro.append(fmt([rows_read(0, 0, kk, v, -1, "p")])[0])
    pro += ["s_waitcnt lgkmcnt(0)", "s_nop 7", "s_nop 7"]

    dflt = Path(__file__).resolve().parent / "attn_dq128_stream.h"
    outp = sys.argv[2] if len(sys.argv) > 2 and not sys.argv[2].startswith("--") else dflt
    with open(outp, "w") as out:
        out.write("// Generated by gen_dq128_stream.py: the tile loop of bwd_dq128_kernel (attn_bwd.hip)\n"
                  f"// as one instruction stream (Y split {h_split}). Regenerate rather than edit.\n"
                  "#pragma once\n\n")
        for name, body in (("SFA_DQ128_PROLOGUE", pro), ("SFA_DQ128_LOOP", lines)):
            out.write(f"#define {name} \\\n")
            for ln in body:
                out.write(f'  "{ln}\\n" \\\n')
            out.write("\n")
        cv = ", ".join(f'"v{x}"' for x in range(32, 256))
        out.write(f"#define SFA_DQ128_CLOBBER_V {cv}\n")
    print(f"// {len(lines)} lines", file=sys.stderr)
    if "--show" in sys.argv:
        for ln in fmt(allseq[0]):
            print(ln)


if __name__ == "__main__":
    main()
