"""Summaries of rocprofv3 counter runs of the library's kernels (measurement
tooling; not used by the library itself).

    python -m hidden_decoding_stream_amd.profile_summary prefill DIR [DIR ...]
    python -m hidden_decoding_stream_amd.profile_summary decode DIR
    python -m hidden_decoding_stream_amd.profile_summary data DIR [DIR ...]
    python -m hidden_decoding_stream_amd.profile_summary kernels PATTERN DIR [DIR ...]

Each DIR holds the CSV output of one `rocprofv3 --pmc ... --kernel-trace
--output-format csv` run of `bench.py --profile-prefill`, which launches the
four full-size prefill workloads three times each, in a fixed order. The
prefill kernel dispatches (attn_fwd128_kernel, attn_fwd_kernel) are assigned to
the workloads in dispatch order.
For each workload it prints the counters averaged over its launches and what
follows from them. GRBM_GUI_ACTIVE is reported summed over the chip's 8 XCDs
(one instance each, counting that XCD's active cycles), so one XCD's active
cycles are the sum / 8:

  mfma_busy        SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE/8 x 1024 SIMDs): the
                   share of SIMD cycles the matrix core was busy
  effective clock  (GUI_ACTIVE/8) / kernel duration
  cu_busy          SQ_BUSY_CU_CYCLES / (GUI_ACTIVE/8 x 256 CUs): the share of
                   CU cycles with a wave resident, 1 - (ramp + tail + gaps
                   between work groups). The counter is read as cycles: read
                   as quad-cycles, as its description has it, it would exceed
                   100% on every kernel here.
  executed flops   SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, against the useful
                   (admitted-pair) flops
  valu_busy        SQ_ACTIVE_INST_VALU x 4 / (GUI_ACTIVE/8 x 1024): VALU
                   issue cycles per SIMD cycle (the counter is per wave, in
                   quad-cycles)
  coexec           SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES: the
                   share of MFMA-busy cycles in which a VALU op also issued
  lds_*            LDS counters per CU cycle (SQ_LDS_IDX_ACTIVE: LDS busy;
                   SQ_LDS_BANK_CONFLICT: cycles stalled by bank conflicts)
  hbm_bytes        (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0) KiB per launch: the
                   factors are what the counters read for a 1 GiB device copy
                   (bench.py --copy-calibration), against the compulsory
                   bytes (read Q, K, V once; write O once)
"""
from __future__ import annotations

import csv
import hashlib
import pathlib
import re
import sys

from . import counts as C
from . import inputs as I

PKG = pathlib.Path(__file__).resolve().parent
ORDER = ("intra_16k", "cross_window_16k", "cross_full_32k", "intra_32k")
REPS = 3
SIMDS = 1024
CUS = 256
XCDS = 8
# HBM counters against a 1 GiB device copy: FETCH_SIZE reads half the bytes, WRITE_SIZE all of them
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0


def _sha16(paths) -> str:
    """First 16 hex digits of the SHA-256 of the given files' bytes, in order."""
    h = hashlib.sha256()
    for path in paths:
        h.update(pathlib.Path(path).read_bytes())
    return h.hexdigest()[:16]



def _read_dir(d: pathlib.Path):
    """{dispatch id: {"name", "ns", counters...}} from one run's CSV files."""
    rows = {}
    for f in sorted(d.rglob("*counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            did = int(r["Dispatch_Id"])
            rec = rows.setdefault(did, {"name": r["Kernel_Name"]})
            rec[r["Counter_Name"]] = rec.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                rec["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    counted = bool(rows)
    for f in sorted(d.rglob("*kernel_trace.csv")):
        for r in csv.DictReader(open(f)):
            did = int(r["Dispatch_Id"])
            if did in rows or not counted:
                rows.setdefault(did, {"name": r["Kernel_Name"]})["ns"] = int(r["End_Timestamp"]) - int(
                    r["Start_Timestamp"])
    return rows


def prefill(dirs) -> str:
    by_name = {w.name: w for w in I.PREFILL_WORKLOADS}
    per = {name: {} for name in ORDER}
    counters_seen = []
    for d in dirs:
        rows = _read_dir(pathlib.Path(d))
        fwd = [rows[k] for k in sorted(rows) if re.search(r"attn_fwd(128)?_kernel<", rows[k]["name"])]
        if len(fwd) != len(ORDER) * REPS:
            raise SystemExit(f"{d}: expected {len(ORDER) * REPS} prefill dispatches, found {len(fwd)}")
        for i, name in enumerate(ORDER):
            for rec in fwd[i * REPS:(i + 1) * REPS]:
                for key, val in rec.items():
                    if key == "name":
                        per[name]["kernel"] = val
                        continue
                    per[name].setdefault(key, []).append(val)
        for key in fwd[0]:
            if key not in ("name", "ns") and key not in counters_seen:
                counters_seen.append(key)
    out = []
    sha = _sha16([PKG / "csrc" / "attn_fwd.hip", PKG / "csrc" / "attn_fwd128_stream.h"])
    for name in ORDER:
        w = by_name[name]
        rec = per[name]
        avg = {k: sum(v) / len(v) for k, v in rec.items() if k != "kernel"}
        useful = C.prefill_flops(w.mode, w.n, w.L, w.batch, w.hq, w.d, w.window)
        out.append(f"{name}: {rec['kernel']}  (n={w.n} L={w.L} batch={w.batch} hq={w.hq} hkv={w.hkv} d={w.d}"
                   f"{' W=' + str(w.window) if w.window else ''})")
        ns = avg.get("ns")
        gui = avg.get("GRBM_GUI_ACTIVE")
        if ns:
            out.append(f"  duration under counters, mean of {REPS}: {ns / 1e3:.1f} us "
                       f"({useful / ns / 1e3:.1f} useful TFLOP/s)")
        for key in counters_seen:
            if key in avg:
                out.append(f"  {key}: {avg[key]:.6g}")
        if gui:
            gx = gui / XCDS
            clk = gx / ns if ns else float("nan")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                busy = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gx * SIMDS)
                out.append(f"mfma_busy[{name}]: {busy:.2f} effective_clock_ghz: {clk:.3f}")
            if "SQ_BUSY_CU_CYCLES" in avg:
                out.append(f"  cu_busy: {100.0 * avg['SQ_BUSY_CU_CYCLES'] / (gx * CUS):.2f} %")
            if "SQ_ACTIVE_INST_VALU" in avg:
                out.append(f"  valu_busy: {100.0 * 4 * avg['SQ_ACTIVE_INST_VALU'] / (gx * SIMDS):.2f} %")
            for key, label in (("SQ_LDS_IDX_ACTIVE", "lds_busy"), ("SQ_LDS_BANK_CONFLICT", "lds_bank_conflict")):
                if key in avg:
                    out.append(f"  {label}: {100.0 * avg[key] / (gx * CUS):.2f} % of CU cycles")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            ex = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            out.append(f"  executed bf16 MFMA flops: {ex:.4e} (useful {useful:.4e}, useful/executed "
                       f"{useful / ex:.4f})")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            out.append(f"  coexec: {100.0 * avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.2f} "
                       "% of MFMA-busy cycles")
        if "FETCH_SIZE" in avg and "WRITE_SIZE" in avg:
            # KiB per dispatch, scaled by what the counters read for a plain 1 GiB copy
            total = (avg["FETCH_SIZE"] * FETCH_FACTOR + avg["WRITE_SIZE"] * WRITE_FACTOR) * 1024
            compulsory = w.batch * w.S * (2 * w.hq + 2 * w.hkv) * w.d * 2   # read Q, K, V; write O
            out.append(f"hbm_bytes[{name}]: {total:.4e} (compulsory {compulsory:.4e}, ratio {total / compulsory:.2f})")
        out.append("")
    out.append(f"kernel_source_sha256_16: {sha}")
    return "\n".join(out)


def decode(d) -> str:
    """The kernel trace of `bench.py --profile-decode`: every dispatch of the
    library's decode kernels and of the plain read, in order, with its
    duration and the idle gap since the previous dispatch ended; then per
    call (split kernel start to combine kernel end, or the split kernel
    alone) and per kernel averages."""
    rows = []
    for f in sorted(pathlib.Path(d).rglob("*kernel_trace.csv")):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            short = ("split" if "decode_split_kernel" in name else "combine" if "decode_combine_kernel" in name
                     else "cfused" if "chain_split_kernel<true>" in name
                     else "csplit" if "chain_split_kernel<false>" in name
                     else "ccomb" if "chain_combine_kernel" in name
                     else "read" if "read_kernel" in name else "slices" if "slices_kernel" in name
                     else "ring" + re.search(r"slices_lds_kernel<(\d+)", name).group(1)
                     if "slices_lds_kernel" in name else None)
            if short:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short, name,
                             r.get("Grid_Size") or r.get("Grid_Size_X") or ""))
    rows.sort()
    out = ["dispatch  kernel   grid      us     gap_before_us"]
    prev_end = None
    calls = []
    for i, (st, en, short, name, grid) in enumerate(rows):
        gap = (st - prev_end) / 1e3 if prev_end is not None else float("nan")
        out.append(f"{i:8d}  {short:7s}  {grid:>8s}  {(en - st) / 1e3:7.2f}  {gap:7.2f}")
        if short == "split":
            calls.append([st, en, en - st, 0, 0.0])
        elif short == "combine" and calls:
            calls[-1][1] = en
            calls[-1][3] = en - st
            calls[-1][4] = gap
        prev_end = en
    out.append("")
    out.append("per call: split us, combine us, gap split->combine us, call span us")
    for c in calls:
        out.append(f"  {c[2] / 1e3:7.2f}  {c[3] / 1e3:7.2f}  {c[4]:7.2f}  {(c[1] - c[0]) / 1e3:7.2f}")
    reads = [(en - st) / 1e3 for st, en, short, _, _ in rows if short == "read"]
    if reads:
        out.append(f"plain read of the same bytes, 256 groups: mean {sum(reads) / len(reads):.2f} us, "
                   f"min {min(reads):.2f} us over {len(reads)} launches")
    for short, what in (("slices", "16-byte loads into registers"), ("ring2", "DMA, ring of 2 stages of 32 rows"),
                        ("ring4", "DMA, ring of 4 stages of 16 rows"), ("ring8", "DMA, ring of 8 stages of 8 rows")):
        ts = [(en - st) / 1e3 for st, en, s, _, _ in rows if s == short]
        if ts:
            out.append(f"the same bytes in the decode's pattern, {what}: mean {sum(ts) / len(ts):.2f} us, "
                       f"min {min(ts):.2f} us over {len(ts)} launches")
    chain = [(st, en) for st, en, s, _, _ in rows if s == "csplit"]
    spans = []
    for st, en in chain:
        nxt = [e2 for s2, e2, k2, _, _ in rows if k2 == "ccomb" and s2 >= en]
        if nxt:
            spans.append((min(nxt) - st) / 1e3)
    if spans:
        out.append(f"the same stream with decode-sized partials and a combine kernel, no arithmetic (split start to "
                   f"combine end): mean {sum(spans) / len(spans):.2f} us, min {min(spans):.2f} us over {len(spans)} calls")
    ts = [(en - st) / 1e3 for st, en, s, _, _ in rows if s == "cfused"]
    if ts:
        out.append(f"the same in one launch, the last group of each kv head merging: mean {sum(ts) / len(ts):.2f} us, "
                   f"min {min(ts):.2f} us over {len(ts)} calls")
    return "\n".join(out)


def kernels(pattern: str, dirs) -> str:
    """Durations and counters of every kernel whose name contains `pattern`
    (a run with only --kernel-trace gives the durations alone), averaged
    over its dispatches in the run directories, with the derived lines of
    prefill(); FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are also given
    in bytes, scaled by the 1 GiB copy calibration of
    FETCH_FACTOR and WRITE_FACTOR)."""
    per = {}
    for d in dirs:
        rows = _read_dir(pathlib.Path(d))
        for k in sorted(rows):
            rec = rows[k]
            if pattern not in rec["name"]:
                continue
            name = rec["name"].replace("void ", "").replace("sfa::(anonymous namespace)::", "").split("(")[0]
            agg = per.setdefault(name, {})
            for key, val in rec.items():
                if key != "name":
                    agg.setdefault(key, []).append(val)
    out = []
    for name, agg in per.items():
        avg = {k: sum(v) / len(v) for k, v in agg.items()}
        ns = avg.get("ns")
        out.append(f"{name}: {len(agg.get('ns', []))} dispatches" + (f", mean {ns / 1e3:.1f} us" if ns else ""))
        if "ns" in agg:
            out.append("  durations (us, in order): " + " ".join(f"{x / 1e3:.1f}" for x in agg["ns"]))
        for key in sorted(avg):
            if key != "ns":
                out.append(f"  {key}: {avg[key]:.6g}")
        gui = avg.get("GRBM_GUI_ACTIVE")
        if gui:
            gx = gui / XCDS
            if ns:
                out.append(f"  effective clock: {gx / ns:.3f} GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                out.append(f"  mfma_busy: {100.0 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (gx * SIMDS):.2f} %")
            if "SQ_BUSY_CU_CYCLES" in avg:
                out.append(f"  cu_busy: {100.0 * avg['SQ_BUSY_CU_CYCLES'] / (gx * CUS):.2f} %")
            if "SQ_ACTIVE_INST_VALU" in avg:
                out.append(f"  valu_busy: {100.0 * 4 * avg['SQ_ACTIVE_INST_VALU'] / (gx * SIMDS):.2f} %")
            for key, label in (("SQ_LDS_IDX_ACTIVE", "lds_busy"), ("SQ_LDS_BANK_CONFLICT", "lds_bank_conflict")):
                if key in avg:
                    out.append(f"  {label}: {100.0 * avg[key] / (gx * CUS):.2f} % of CU cycles")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and avg.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            out.append(f"  coexec: {100.0 * avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.2f} "
                       "% of MFMA-busy cycles")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            out.append(f"  executed bf16 MFMA flops: {avg['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4e}")
        if "FETCH_SIZE" in avg:
            out.append(f"  HBM read bytes (FETCH_SIZE x 1024 x {FETCH_FACTOR}): {avg['FETCH_SIZE'] * 1024 * FETCH_FACTOR:.4e}")
        if "WRITE_SIZE" in avg:
            out.append(f"  HBM write bytes (WRITE_SIZE x 1024 x {WRITE_FACTOR}): {avg['WRITE_SIZE'] * 1024 * WRITE_FACTOR:.4e}")
        out.append("")
    return "\n".join(out)


DATA_ORDER = ("randn", "v_zero", "q_zero", "all_zero")
DATA_REPS = 5


def data(dirs) -> str:
    """Counter runs of `bench.py --prefill-data`: the cross_full 32k prefill
    launched DATA_REPS times on each data set of DATA_ORDER after one warm-up
    launch. Per data set: duration, effective clock, MFMA busy and CU busy,
    averaged over its launches (the warm-up launch is left out)."""
    w = I.CROSS_32K
    useful = C.prefill_flops(w.mode, w.n, w.L, w.batch, w.hq, w.d, w.window)
    per = {name: {} for name in DATA_ORDER}
    for d in dirs:
        rows = _read_dir(pathlib.Path(d))
        fwd = [rows[k] for k in sorted(rows) if re.search(r"attn_fwd128_kernel<", rows[k]["name"])]
        if len(fwd) != 1 + len(DATA_ORDER) * DATA_REPS:
            raise SystemExit(f"{d}: expected {1 + len(DATA_ORDER) * DATA_REPS} prefill dispatches, found {len(fwd)}")
        for i, name in enumerate(DATA_ORDER):
            for rec in fwd[1 + i * DATA_REPS:1 + (i + 1) * DATA_REPS]:
                for key, val in rec.items():
                    if key != "name":
                        per[name].setdefault(key, []).append(val)
    out = [f"{'data':9s} {'us':>8s} {'TFLOP/s':>8s} {'clock_GHz':>9s} {'mfma_busy_%':>11s} {'cu_busy_%':>9s}"]
    for name in DATA_ORDER:
        avg = {k: sum(v) / len(v) for k, v in per[name].items()}
        ns = avg.get("ns", float("nan"))
        gx = avg.get("GRBM_GUI_ACTIVE", float("nan")) / XCDS
        busy = 100.0 * avg.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (gx * SIMDS)
        cu = 100.0 * avg.get("SQ_BUSY_CU_CYCLES", float("nan")) / (gx * CUS)
        out.append(f"{name:9s} {ns / 1e3:8.1f} {useful / ns / 1e3:8.1f} {gx / ns:9.3f} {busy:11.2f} {cu:9.2f}")
    out.append("")
    out.append("kernel_source_sha256_16: " + _sha16([PKG / "csrc" / "attn_fwd.hip", PKG / "csrc" / "attn_fwd128_stream.h"]))
    return "\n".join(out)


def main(argv):
    if len(argv) >= 2 and argv[0] == "prefill":
        print(prefill(argv[1:]))
    elif len(argv) >= 2 and argv[0] == "data":
        print(data(argv[1:]))
    elif len(argv) == 2 and argv[0] == "decode":
        print(decode(argv[1]))
    elif len(argv) >= 3 and argv[0] == "kernels":
        print(kernels(argv[1], argv[2:]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
