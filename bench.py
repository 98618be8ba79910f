#!/usr/bin/env python3
"""Benchmark of the stream-factorized attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over the 32k workload
(n = 4 streams, L = 8192 tokens, S = 32768 expanded positions, batch 1,
32 query / 8 key-value heads, d = 128, bf16):
  1. interleave the per-stream Q, K, V into the expanded sequence;
  2. cross_full prefill attention (causal over all 32768 positions);
  3. intra prefill attention on the same tensors (one causal pass per stream);
  4. de-interleave K and V into the per-stream KV cache;
  5. decode of token L-1's four stream queries against that cache (cross_full).
The reported value is the useful attention throughput of the step: the flops of
the admitted (query, key) pairs of steps 2, 3 and 5 divided by the step time.
The line also carries the roofline of the dominant kernel (the cross_full
prefill, timed with HIP events around its own launches, with the hardware
MFMA-busy share from the committed counter summary), every prefill workload
timed on its own (tiny, intra 16k, cross_window 16k, cross_full and intra
32k), a decode bandwidth sweep (batch 1, 8, 64; intra and cross_full) and the
CPU oracle timed on a bounded sample of the same workload.

Inputs are synthetic (seeded N(0,1), rounded to bf16) and resident in HBM
before timing starts. Only one GPU is used.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import pathlib
import re
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
METRIC = "SF-attention useful TFLOP/s + MFMA% at n=4 nL=32k; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PROFILE_COUNTERS = ROOT / "profiles" / "attn_fwd_prefill_counters.txt"
# the prefill kernels' sources: the counter summary is used only if taken on these
FWD_SOURCES = (ROOT / "hidden_decoding_stream_amd" / "csrc" / "attn_fwd.hip",
               ROOT / "hidden_decoding_stream_amd" / "csrc" / "attn_fwd128_stream.h")
# launches per workload in --profile-prefill (counter runs read them in this order)
PROFILE_PREFILL_ORDER = ("intra_16k", "cross_window_16k", "cross_full_32k", "intra_32k")
PROFILE_PREFILL_REPS = 3
# --prefill-data: the cross_full 32k launch on the workload's N(0,1) inputs and on the same inputs with
# operands zeroed (one warm-up launch, then this many per data set, in this order)
PREFILL_DATA_ORDER = ("randn", "v_zero", "q_zero", "all_zero")
PREFILL_DATA_REPS = 5


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode-sweep", action="store_true", help="skip the decode bandwidth sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters), then exit")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only run decode calls for trace and counter runs (batch 1 and 8, cross_full and "
                         "intra, 3 calls each on distinct caches; then 24 plain reads of the batch-1 "
                         "cache's bytes on the decode's 256-group grid), then exit")
    ap.add_argument("--decode-splits", action="store_true",
                    help="time decode at small batch over explicit split counts (one JSON line per case) and exit")
    ap.add_argument("--trace-prefill", action="store_true",
                    help="only run the four full-size prefill workloads on the trace build of the library "
                         "(libsfattn_trace.so) and print each launch's timeline statistics, then exit")
    ap.add_argument("--profile-backward", action="store_true",
                    help="only run sf_attn_bwd on the 32k workload for counter runs (cross_full then intra, "
                         "2 calls each after the forward that gives the LSE), then exit")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="only run the four full-size prefill workloads for counter runs "
                         f"({', '.join(PROFILE_PREFILL_ORDER)}; {PROFILE_PREFILL_REPS} launches each, "
                         "in that order), then exit")
    ap.add_argument("--prefill-data", action="store_true",
                    help="only run the cross_full 32k prefill on its N(0,1) inputs and with operands zeroed "
                         f"({', '.join(PREFILL_DATA_ORDER)}; one warm-up launch, then {PREFILL_DATA_REPS} "
                         "launches each, timed with HIP events), then exit")
    return ap.parse_args()


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        h.update(path.read_bytes())
    return h.hexdigest()[:16]


def _stored_counters():
    """The committed prefill counter summary, if it was taken on the current
    kernel source; else None."""
    if not PROFILE_COUNTERS.exists():
        return None
    text = PROFILE_COUNTERS.read_text()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_sha or m_sha.group(1) != source_sha(FWD_SOURCES):
        return None
    return text


def stored_mfma_busy():
    """Hardware MFMA-busy share (SQ_VALU_MFMA_BUSY_CYCLES over one XCD's
    GRBM_GUI_ACTIVE x 1024 SIMDs) and effective clock per prefill workload,
    from the committed counter summary (only if taken on the current kernel
    source); else {}."""
    text = _stored_counters()
    if text is None:
        return {}
    out = {}
    for name, busy, clk in re.findall(r"^mfma_busy\[(\w+)\]:\s*([0-9.]+)\s+effective_clock_ghz:\s*([0-9.]+)",
                                      text, flags=re.M):
        out[name] = {"mfma_busy": float(busy), "clock_ghz": float(clk)}
    return out


def stored_traffic():
    """HBM bytes of one cross_full 32k prefill launch (FETCH_SIZE and
    WRITE_SIZE, calibrated against a plain copy), from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    text = _stored_counters()
    m = re.search(r"^hbm_bytes\[cross_full_32k\]:\s*([0-9.eE+]+)", text or "", flags=re.M)
    return float(m.group(1)) if m else None


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.trace_prefill:
        # the measurement build of the library, with the prefill's timeline compiled in
        os.environ["SFATTN_LIB"] = str(ROOT / "hidden_decoding_stream_amd" / "libsfattn_trace.so")
    import torch

    import hidden_decoding_stream_amd as sfa
    import hidden_decoding_stream_amd.counts as C
    import hidden_decoding_stream_amd.inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        nbytes = 1 << 30
        a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}))
        return
    if args.profile_decode:
        for batch in (1, 8):
            for mode in ("cross_full", "intra"):
                wd = I.decode_workload(batch, mode)
                g = torch.Generator(device=dev).manual_seed(3)
                q = torch.randn((batch, wd.n, wd.hq, wd.d), generator=g, device=dev).to(torch.bfloat16)
                caches = [tuple(torch.randn((batch, wd.n, wd.T, wd.hkv, wd.d), generator=g, device=dev)
                                .to(torch.bfloat16) for _ in range(2)) for _ in range(3)]
                for kc, vc in caches:
                    sfa.sf_attn_decode(q, kc, vc, wd.T, mode, scale=wd.scale)
                torch.cuda.synchronize()
                print(json.dumps({"profile_decode": mode, "batch": batch, "calls": 3}), flush=True)
                del caches
                torch.cuda.empty_cache()
        # the floor for the batch-1 stream: one plain read of the same 134,217,728 bytes on the same
        # 256-group grid, from 8 distinct buffers (1 GiB, beyond the Infinity Cache), 3 rounds
        import hidden_decoding_stream_amd.peaks as P
        nbytes = 2 * 4 * 8192 * 8 * 128 * 2
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(8)]
        sink = torch.empty(256, dtype=torch.int32, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            for b in bufs:
                if P.lib().sfp_read(b.data_ptr(), nbytes, sink.data_ptr(), 256, st) != 0:
                    raise RuntimeError("sfp_read launch failed")
        torch.cuda.synchronize()
        print(json.dumps({"profile_read": nbytes, "blocks": 256, "launches": 24}), flush=True)
        # the same bytes in the decode's pattern (8 heads x 32 key ranges, each head's 256-byte slice of
        # every K and V row): 16-byte loads into registers, then buffer->LDS DMA through rings of 2, 4
        # and 8 stages per wave; 8 cache pairs (1 GiB) rotated, 3 rounds each
        rows = 4 * 8192
        pairs = [(bufs[i], bufs[i + 4]) for i in range(4)] + [(bufs[i + 4], bufs[i]) for i in range(4)]
        sink = torch.empty(8 * 32, dtype=torch.int32, device=dev)
        for ring in (0, 2, 4, 8):
            for _ in range(3):
                for kb, vb in pairs:
                    rc = (P.lib().sfp_read_slices(kb.data_ptr(), vb.data_ptr(), rows, 8, 32, sink.data_ptr(), st)
                          if ring == 0 else
                          P.lib().sfp_read_slices_lds(kb.data_ptr(), vb.data_ptr(), rows, 8, 32, ring, st))
                    if rc != 0:
                        raise RuntimeError("sfp_read_slices launch failed")
            torch.cuda.synchronize()
            print(json.dumps({"profile_read_slices": ring or "registers", "launches": 24}), flush=True)
        # the batch-1 call's structure with no arithmetic: the same stream, decode-sized partials and
        # their merge, by a second kernel (two launches per call) or in one launch; 24 calls each
        part = torch.empty(8 * 16 * 32 * 130, dtype=torch.float32, device=dev)
        ticket = torch.zeros(8, dtype=torch.int32, device=dev)
        outb = torch.empty(8 * 16 * 128, dtype=torch.bfloat16, device=dev)
        for fused in (0, 1):
            for _ in range(3):
                for kb, vb in pairs:
                    if P.lib().sfp_decode_chain(kb.data_ptr(), vb.data_ptr(), rows, 8, 32, part.data_ptr(),
                                                ticket.data_ptr(), outb.data_ptr(), fused, st) != 0:
                        raise RuntimeError("sfp_decode_chain launch failed")
            torch.cuda.synchronize()
            print(json.dumps({"profile_decode_chain": "one launch" if fused else "split + combine",
                              "calls": 24}), flush=True)
        return

    if args.decode_splits:
        decode_split_sweep(torch, sfa, C, dev)
        return
    if args.trace_prefill:
        trace_prefill(torch, sfa, I, dev)
        return
    if args.profile_backward:
        wb = I.CROSS_32K
        q, k, v = I.workload_qkv(wb, device=dev)
        g = torch.Generator(device=dev).manual_seed(1053)
        dout = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
        for mode in ("cross_full", "intra"):
            o, lse = sfa.sf_attn_fwd(q, k, v, mode, wb.n, scale=wb.scale, lse=True)
            for _ in range(2):
                sfa.sf_attn_bwd(q, k, v, o, dout, lse, mode, wb.n, scale=wb.scale)
            torch.cuda.synchronize()
            print(json.dumps({"profile_backward": mode, "calls": 2}), flush=True)
        return
    if args.profile_prefill:
        by_name = {x.name: x for x in I.PREFILL_WORKLOADS}
        for name in PROFILE_PREFILL_ORDER:
            wp = by_name[name]
            q, k, v = I.workload_qkv(wp, device=dev)
            o = torch.empty_like(q)
            for _ in range(PROFILE_PREFILL_REPS):
                sfa.sf_attn_fwd(q, k, v, wp.mode, wp.n, window=wp.window, scale=wp.scale, out=o)
            torch.cuda.synchronize()
            print(json.dumps({"profile_prefill": name, "launches": PROFILE_PREFILL_REPS}), flush=True)
            del q, k, v, o
            torch.cuda.empty_cache()
        return

    if args.prefill_data:
        # Same kernel, same shapes and masks, different operand values: the matrix core's switching
        # activity depends on the data, and with it the clock the chip holds under this load.
        wp = I.CROSS_32K
        q, k, v = I.workload_qkv(wp, device=dev)
        o = torch.empty_like(q)
        data = {"randn": (q, k, v), "v_zero": (q, k, torch.zeros_like(v)),
                "q_zero": (torch.zeros_like(q), k, v),
                "all_zero": (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v))}
        st = torch.cuda.current_stream()
        useful = C.prefill_flops(wp.mode, wp.n, wp.L, wp.batch, wp.hq, wp.d, wp.window)
        sfa.sf_attn_fwd(q, k, v, wp.mode, wp.n, scale=wp.scale, out=o)
        for name in PREFILL_DATA_ORDER:
            qq, kk, vv = data[name]
            ev = []
            for _ in range(PREFILL_DATA_REPS):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                sfa.sf_attn_fwd(qq, kk, vv, wp.mode, wp.n, scale=wp.scale, out=o)
                e1.record(st)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in ev)
            med = ms[len(ms) // 2]
            print(json.dumps({"prefill_data": name, "workload": wp.name, "launches": PREFILL_DATA_REPS,
                              "ms_median": round(med, 4), "ms_min": round(ms[0], 4),
                              "useful_tflops": round(useful / med / 1e9, 1)}), flush=True)
        return

    w = I.CROSS_32K
    n, L, B, hq, hkv, d, S = w.n, w.L, w.batch, w.hq, w.hkv, w.d, w.S
    scale = w.scale

    # ---- inputs, resident in HBM ----
    qs, ks, vs = I.stream_qkv(n, L, B, hq, hkv, d, seed=w.seed, device=dev)   # [n][B][L][H][d]
    Q = torch.empty((B, S, hq, d), dtype=torch.bfloat16, device=dev)
    K = torch.empty((B, S, hkv, d), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    Oc = torch.empty_like(Q)
    Oi = torch.empty_like(Q)
    kc = torch.empty((n, B, L, hkv, d), dtype=torch.bfloat16, device=dev)     # == [B][n][L][hkv][d] at B=1
    vc = torch.empty_like(kc)
    assert B == 1, "the per-stream cache view below relies on batch 1"
    q_new = qs[:, 0, L - 1].unsqueeze(0).contiguous()                          # [1][n][hq][d]
    od = torch.empty_like(q_new)
    ws_bytes = sfa.sf_attn_decode_workspace_bytes(B, n, L, hq, hkv, d, "cross_full")
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    flops_cross = C.prefill_flops("cross_full", n, L, B, hq, d)
    flops_intra = C.prefill_flops("intra", n, L, B, hq, d)
    flops_dec = C.decode_flops("cross_full", n, L, B, hq, d)
    step_flops = flops_cross + flops_intra + flops_dec

    ev = {k: [] for k in ("cross", "intra", "ilv", "dec")}

    def step(record: bool):
        def mark(name):
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                ev[name].append((e0, e1))
                return e0, e1
            return None, None

        a0, a1 = mark("ilv")
        if a0: a0.record(stream)
        sfa.sf_interleave_multi([qs, ks, vs], n, outs=[Q, K, V])
        if a1: a1.record(stream)
        e0, e1 = mark("cross")
        if e0: e0.record(stream)
        sfa.sf_attn_fwd(Q, K, V, "cross_full", n, scale=scale, out=Oc)
        if e1: e1.record(stream)
        i0, i1 = mark("intra")
        if i0: i0.record(stream)
        sfa.sf_attn_fwd(Q, K, V, "intra", n, scale=scale, out=Oi)
        if i1: i1.record(stream)
        sfa.sf_interleave_multi([K, V], n, inverse=True, outs=[kc.view(n, B, L, hkv, d), vc.view(n, B, L, hkv, d)])
        d0, d1 = mark("dec")
        if d0: d0.record(stream)
        sfa.sf_attn_decode(q_new, kc.view(B, n, L, hkv, d), vc.view(B, n, L, hkv, d), L, "cross_full",
                           scale=scale, out=od, workspace=ws)
        if d1: d1.record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = step_flops / (elapsed / args.steps) / 1e12

    def avg_ms(name):
        return sum(a.elapsed_time(b) for a, b in ev[name]) / len(ev[name])

    cross_ms, intra_ms, ilv_ms, dec_ms = avg_ms("cross"), avg_ms("intra"), avg_ms("ilv"), avg_ms("dec")
    achieved = flops_cross / (cross_ms * 1e-3) / 1e12
    traffic = stored_traffic()
    hw = stored_mfma_busy()
    print(f"[bench] step {ms_per_step:.3f} ms; cross_full {cross_ms:.3f} ms ({achieved:.1f} TFLOP/s), "
          f"intra {intra_ms:.3f} ms, interleave x3 {ilv_ms:.3f} ms, decode {dec_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    # sanity: decode of token L-1 equals the last n rows of the cross_full prefill
    torch.cuda.synchronize()
    dev_err = (od[0].float() - Oc[0, (L - 1) * n:].float()).abs().max().item()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "sfa_step_32k: interleave Q,K,V + cross_full prefill + intra prefill + "
                        "de-interleave K,V to the per-stream cache + cross_full decode of token L-1",
            "n": n, "L": L, "S": S, "batch": B, "hq": hq, "hkv": hkv, "d": d,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "attn_fwd128_kernel<1> (cross_full) 32k",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "mfma_busy": (hw.get("cross_full_32k") or {}).get("mfma_busy"),
            "clock_ghz": (hw.get("cross_full_32k") or {}).get("clock_ghz"),
            "useful_flop_per_launch": flops_cross,
            "avg_launch_ms": round(cross_ms, 4),
        },
        "breakdown_ms": {
            "interleave_qkv": round(ilv_ms, 4),
            "cross_full_prefill": round(cross_ms, 4),
            "intra_prefill": round(intra_ms, 4),
            "decode_b1_cross_full": round(dec_ms, 4),
            "intra_tflops": round(flops_intra / (intra_ms * 1e-3) / 1e12, 2),
        },
        "decode_vs_prefill_max_abs": dev_err,
    }

    line["prefill"] = prefill_configs(torch, sfa, C, I, dev, stream, hw,
                                      {"cross_full_32k": cross_ms, "intra_32k": intra_ms})
    line["last_stream"] = last_stream_timing(torch, sfa, C, Q, K, V, n, L, B, hq, d, scale, stream)
    line["front_end"] = front_end_timing(torch, sfa, C, n, L, B, hq, d, dev, stream)
    line["backward"] = backward_timing(torch, sfa, C, Q, K, V, Oc, n, L, B, hq, hkv, d, scale, dev, stream)
    if not args.no_decode_sweep:
        line["decode"] = decode_sweep(torch, sfa, C, I, dev)
        line["serving"] = serving_sweep(torch, sfa, C, I, dev)
    line["attainable"] = attainable_peaks(line)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, C, I, qs, ks, vs, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def trace_prefill(torch, sfa, I, dev, reps=3):
    """Timeline of the prefill's work groups, from the trace build: for each
    full-size workload, `reps` launches after 2 untimed ones. Per launch, with
    every item's start, first-tiles-landed, tile-loop end and end (100 MHz
    s_memrealtime), and the CU (HW_ID) and XCD (XCC_ID) that ran it:
      busy_share     sum of item durations / (CUs x span)
      gap_share      idle time between consecutive items on a CU / (CUs x span)
      tail_share     idle time after a CU's last item / (CUs x span)
      prologue_share (first tiles landed - start) / busy: Q load and the first tiles' DMA
      epilogue_share (end - tile loop end) / busy: normalisation and the output stores
      fit_us_per_tile, fit_us_fixed: least squares of item duration against its key tiles.
    Printed as one JSON line per launch."""
    import numpy as np
    L = sfa.lib()
    L.sf_trace_prefill.argtypes = [ctypes.c_void_p]
    L.sf_trace_prefill.restype = None
    by_name = {x.name: x for x in I.PREFILL_WORKLOADS}
    for name in PROFILE_PREFILL_ORDER:
        w = by_name[name]
        q, k, v = I.workload_qkv(w, device=dev)
        o = torch.empty_like(q)
        call = lambda: sfa.sf_attn_fwd(q, k, v, w.mode, w.n, window=w.window, scale=w.scale, out=o)  # noqa: E731
        L.sf_trace_prefill(None)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        # work items of the launch (the kernel's own count): query blocks x head groups per unit
        G = w.hq // w.hkv
        HG = 1
        while HG * 2 <= 8 and G % (HG * 2) == 0:
            HG *= 2
        nseq, Lv = (w.n, w.L) if w.mode == "intra" else (1, w.S)
        items = w.batch * nseq * w.hkv * -(-Lv // ((8 // HG) * 32)) * (G // HG)
        for rep in range(reps):
            buf = torch.zeros(items * 8, dtype=torch.int64, device=dev)
            L.sf_trace_prefill(buf.data_ptr())
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            L.sf_trace_prefill(None)
            tr = buf.view(-1, 8).cpu().numpy()
            tr = tr[tr[:, 0] != 0]
            start, landed, loop_end, end, hw, xcc, _, tiles = (tr[:, i].astype(np.int64) for i in range(8))
            t0, span = start.min(), end.max() - start.min()
            cu = xcc * 256 + ((hw >> 8) & 0xFF)      # HW_ID bits 8-15: CU, SH and SE of the work group
            per = {}
            for i in range(len(tr)):
                per.setdefault(int(cu[i]), []).append((int(start[i]), int(end[i])))
            gaps, tails = 0, 0
            for lst in per.values():
                lst.sort()
                gaps += sum(b[0] - a[1] for a, b in zip(lst, lst[1:]))
                tails += t0 + span - lst[-1][1]
            busy = int((end - start).sum())
            cap = len(per) * span
            fit = np.linalg.lstsq(np.vstack([tiles, np.ones(len(tiles))]).T.astype(np.float64),
                                  (end - start).astype(np.float64), rcond=None)[0]
            print(json.dumps({
                "trace_prefill": name, "launch": rep, "event_ms": round(e0.elapsed_time(e1), 4),
                "items": int(len(tr)), "cus": len(per), "span_us": span / 100.0,
                "busy_share": round(busy / cap, 4), "gap_share": round(gaps / cap, 4),
                "tail_share": round(tails / cap, 4),
                "prologue_share": round(float((landed - start).sum()) / busy, 4),
                "epilogue_share": round(float((end - loop_end).sum()) / busy, 4),
                "prologue_us_mean": round(float((landed - start).mean()) / 100, 2),
                "epilogue_us_mean": round(float((end - loop_end).mean()) / 100, 2),
                "fit_us_per_tile": round(fit[0] / 100, 4), "fit_us_fixed": round(fit[1] / 100, 2)}), flush=True)
        del q, k, v, o
        torch.cuda.empty_cache()


def warm_up(torch, call, min_s=0.05):
    """Untimed launches of `call` until about min_s seconds of it have run.
    The clock the chip holds under a new load settles over several
    milliseconds: after a pause (inputs drawn, tensors freed) the first
    launches of a 1 ms kernel run up to 15% slower than the steady state."""
    torch.cuda.synchronize()
    t = time.perf_counter()
    call()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t, 1e-5)
    for _ in range(max(1, int(min_s / one))):
        call()
    torch.cuda.synchronize()


def prefill_configs(torch, sfa, C, I, dev, stream, hw, step_ms, reps=10):
    """Every prefill workload on its own: the tiny problem (intra and
    cross_full, attention on the bf16 rounding of its fp32 draws), intra 16k
    (batch 2), cross_window 16k (batch 2, W = 4096 positions) and the 32k
    cross_full and intra passes (their times are the step's own launches).
    Useful TFLOP/s counts admitted pairs only; `frac` is of 2.5 PFLOP/s dense
    bf16; `mfma_busy` and `clock_ghz` come from the committed counter summary
    (null unless it was taken on the current kernel source)."""
    out = {}
    for w in I.PREFILL_WORKLOADS:
        fl = C.prefill_flops(w.mode, w.n, w.L, w.batch, w.hq, w.d, w.window)
        if w.name in step_ms:
            ms = step_ms[w.name]
        else:
            q, k, v = I.workload_qkv(w, device=dev)
            if q.dtype != torch.bfloat16:
                q, k, v = (I.to_bf16(x) for x in (q, k, v))
            o = torch.empty_like(q)
            call = lambda: sfa.sf_attn_fwd(q, k, v, w.mode, w.n, window=w.window, scale=w.scale,  # noqa: E731
                                           out=o)
            warm_up(torch, call)
            pairs = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call()
                e1.record(stream)
                pairs.append((e0, e1))
            torch.cuda.synchronize()
            ms = sum(a.elapsed_time(b) for a, b in pairs) / reps
            del q, k, v, o
        tf = fl / (ms * 1e-3) / 1e12
        rec = {"mode": w.mode, "n": w.n, "L": w.L, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "d": w.d,
               "window": w.window, "ms": round(ms, 4), "useful_flop": fl, "tflops": round(tf, 2),
               "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        h = hw.get(w.name) or {}
        rec["mfma_busy"] = h.get("mfma_busy")
        rec["clock_ghz"] = h.get("clock_ghz")
        out[w.name] = rec
        print(f"[bench] prefill {w.name}: {ms:.4f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    return out


def attainable_peaks(line):
    """The chip's attainable peaks measured on this GPU (back-to-back dense
    bf16 MFMAs on fixed operands and on random ones; a streaming read of
    2 GiB, beyond the Infinity Cache), and the headline prefill and the
    decode sweep as fractions of them, beside the published peaks that
    `roofline` uses."""
    import hidden_decoding_stream_amd.peaks as P
    mfma = P.mfma_bf16_flops() / 1e12
    mfma_rnd = P.mfma_bf16_random_flops() / 1e12
    read = P.read_bandwidth() / 1e9
    out = {"mfma_bf16_tflops": round(mfma, 1), "mfma_bf16_random_tflops": round(mfma_rnd, 1),
           "hbm_read_GBps": round(read, 1),
           "prefill_cross_full_frac": round(line["roofline"]["achieved"] / mfma, 4),
           "prefill_cross_full_frac_random": round(line["roofline"]["achieved"] / mfma_rnd, 4)}
    for key, rec in (line.get("decode") or {}).items():
        out[f"decode_{key}_frac"] = round(rec["GBps"] / read, 4)
    # the floor of the batch-1 decode call: its bytes in its pattern with no arithmetic, read alone,
    # then with the split + combine hand-over (two launches) and with a one-launch merge
    fl = P.decode_structure_floor()
    out["decode_b1_floor"] = fl
    print(f"[bench] batch-1 decode floor: read {fl['read_us']} us, split+combine chain {fl['chain_us']} us, "
          f"one-launch chain {fl['fused_us']} us", file=sys.stderr, flush=True)
    print(f"[bench] attainable: {mfma:.0f} TFLOP/s bf16 (random operands {mfma_rnd:.0f}), {read:.0f} GB/s read",
          file=sys.stderr, flush=True)
    return out


def last_stream_timing(torch, sfa, C, Q, K, V, n, L, B, hq, d, scale, stream, reps=10):
    """Attention of stream n-1's queries only (one per token) against all
    streams' K/V of the same 32k workload: useful TFLOP/s per mode."""
    ql = Q[:, n - 1::n].contiguous()
    o = torch.empty_like(ql)
    out = {}
    for mode in ("cross_full", "intra"):
        warm_up(torch, lambda: sfa.sf_attn_fwd_last_stream(ql, K, V, mode, n, scale=scale, out=o))
        pairs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sfa.sf_attn_fwd_last_stream(ql, K, V, mode, n, scale=scale, out=o)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in pairs) / reps
        fl = C.last_stream_flops(mode, n, L, B, hq, d)
        out[mode] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "useful_flop": fl}
        print(f"[bench] last-stream {mode}: {ms:.3f} ms, {fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    return out


def front_end_timing(torch, sfa, C, n, L, B, hq, d, dev, stream, vocab=32000, reps=10):
    """The expansion front-end at the 32k workload: the gather of the n
    embedding tables (vocab x hq*d bf16 each) into the expanded sequence, and
    the rotary encoding of Q in place. HBM GB/s of their algorithmic bytes."""
    hidden = hq * d
    g = torch.Generator(device=dev).manual_seed(1005)
    tables = torch.randn((n, vocab, hidden), generator=g, device=dev).to(torch.bfloat16)
    ids = torch.randint(0, vocab, (B, L), generator=g, device=dev, dtype=torch.int32)
    x = torch.empty((B, n * L, hidden), dtype=torch.bfloat16, device=dev)
    q = torch.randn((B, n * L, hq, d), generator=g, device=dev).to(torch.bfloat16)

    def timed(fn):
        for _ in range(2):
            fn()
        pairs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in pairs) / reps

    out = {}
    ms = timed(lambda: sfa.sf_expand_embed(ids, tables, out=x))
    by = C.expand_embed_bytes(B, n, L, hidden * 2)
    out["expand_embed"] = {"us": round(ms * 1e3, 1), "GBps": round(by / (ms * 1e-3) / 1e9, 1),
                           "hbm_frac": round(by / (ms * 1e-3) / 8e12, 4), "bytes": by}
    ms = timed(lambda: sfa.sf_rope(q, base=10000.0))
    by = C.rope_bytes(q.numel() * 2)
    out["rope_q"] = {"us": round(ms * 1e3, 1), "GBps": round(by / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(by / (ms * 1e-3) / 8e12, 4), "bytes": by}
    for k2, v2 in out.items():
        print(f"[bench] {k2}: {v2['us']} us, {v2['GBps']} GB/s", file=sys.stderr, flush=True)
    del tables, x, q
    torch.cuda.empty_cache()
    return out


def backward_timing(torch, sfa, C, Q, K, V, Oc, n, L, B, hq, hkv, d, scale, dev, stream, reps=5):
    """sf_attn_bwd (all three of its kernels) on the 32k workload: useful
    TFLOP/s for cross_full and intra."""
    g = torch.Generator(device=dev).manual_seed(1053)
    dout = torch.randn(Q.shape, generator=g, device=dev).to(torch.bfloat16)
    dq, dk, dv = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ws = torch.empty(int(sfa.lib().sf_attn_bwd_workspace_bytes(B, n, L, hq, hkv, d, 1, 0)) + 16,
                     dtype=torch.uint8, device=dev)
    out = {}
    for mode in ("cross_full", "intra"):
        o, lse = sfa.sf_attn_fwd(Q, K, V, mode, n, scale=scale, lse=True)
        call = lambda: sfa.sf_attn_bwd(Q, K, V, o, dout, lse, mode, n, scale=scale, out=(dq, dk, dv),  # noqa: E731
                                       workspace=ws)
        warm_up(torch, call)
        pairs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in pairs) / reps
        fl = C.backward_flops(mode, n, L, B, hq, d)
        out[mode] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "useful_flop": fl}
        print(f"[bench] backward {mode}: {ms:.3f} ms, {fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        del o, lse
    return out


def decode_sweep(torch, sfa, C, I, dev):
    """Decode bandwidth at batch 1, 8 and 64. Caches are rotated over >= 1 GiB
    of distinct memory so the 256 MiB Infinity Cache cannot serve repeats."""
    out = {}
    reps = 20
    for batch in (1, 8, 64):
        for mode in ("intra", "cross_full"):
            w = I.decode_workload(batch, mode)
            per_cache = 2 * batch * w.n * w.T * w.hkv * w.d * 2
            copies = max(1, math.ceil((1 << 30) / per_cache))
            g = torch.Generator(device=dev).manual_seed(w.seed)
            q = torch.randn((batch, w.n, w.hq, w.d), generator=g, device=dev).to(torch.bfloat16)
            caches = []
            for _ in range(copies):
                kc = torch.randn((batch, w.n, w.T, w.hkv, w.d), generator=g, device=dev).to(torch.bfloat16)
                vc = torch.randn((batch, w.n, w.T, w.hkv, w.d), generator=g, device=dev).to(torch.bfloat16)
                caches.append((kc, vc))
            o = torch.empty_like(q)
            ws = torch.empty(sfa.sf_attn_decode_workspace_bytes(batch, w.n, w.T, w.hq, w.hkv, w.d, mode) + 16,
                             dtype=torch.uint8, device=dev)
            for i in range(3):
                kc, vc = caches[i % copies]
                sfa.sf_attn_decode(q, kc, vc, w.T, mode, scale=w.scale, out=o, workspace=ws)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                kc, vc = caches[i % copies]
                sfa.sf_attn_decode(q, kc, vc, w.T, mode, scale=w.scale, out=o, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            nbytes = C.decode_bytes(mode, w.n, w.T, batch, w.hq, w.hkv, w.d)
            gbps = nbytes / (us * 1e-6) / 1e9
            out[f"b{batch}_{mode}"] = {"us": round(us, 2), "GBps": round(gbps, 1),
                                       "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4), "bytes": nbytes,
                                       "caches_rotated": copies}
            print(f"[bench] decode b={batch} {mode}: {us:.1f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
            del caches, q, o, ws
            torch.cuda.empty_cache()
    return out


def _rotated_time(torch, calls, reps=20):
    """Mean microseconds per call, cycling through `calls` (one per distinct
    copy of the data) after 3 untimed calls."""
    for i in range(3):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        calls[i % len(calls)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def decode_split_sweep(torch, sfa, C, dev):
    """Decode at small batch against the split count: the library's plan (0)
    and explicit counts 4 ... 128, each the best of 3 rotated timings of 20
    calls, after ~50 ms of warm-up calls on the case. Cases: cross_window W = 4096 at batch 1 and 8, cross_full and intra
    at batch 1 (n = 4, T = 8192), cross_full at n = 8, T = 4096, batch 1;
    32/8 heads, d = 128."""
    g = torch.Generator(device=dev).manual_seed(1010)

    def bf16(*shape):
        return torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)

    hq, hkv, d = 32, 8, 128
    for tag, n, T, mode, W, batch in (("window4096", 4, 8192, "cross_window", 4096, 1),
                                      ("window4096", 4, 8192, "cross_window", 4096, 8),
                                      ("cross_full", 4, 8192, "cross_full", 0, 1),
                                      ("intra", 4, 8192, "intra", 0, 1),
                                      ("n8_cross_full", 8, 4096, "cross_full", 0, 1)):
        nbytes = C.decode_bytes(mode, n, T, batch, hq, hkv, d, window=W)
        cache_bytes = 2 * batch * n * T * hkv * d * 2
        copies = max(1, min(math.ceil((1 << 30) / nbytes), (12 << 30) // cache_bytes))
        q = bf16(batch, n, hq, d)
        caches = [(bf16(batch, n, T, hkv, d), bf16(batch, n, T, hkv, d)) for _ in range(copies)]
        o = torch.empty_like(q)
        scale = 1.0 / math.sqrt(d)
        res = {}
        # warm the chip on this case first: the count timed first would otherwise carry the clock's ramp
        ws0 = torch.empty(sfa.sf_attn_decode_workspace_bytes(batch, n, T, hq, hkv, d, mode, W) + 16,
                          dtype=torch.uint8, device=dev)
        warm_up(torch, lambda: [sfa.sf_attn_decode(q, kc, vc, T, mode, window=W, scale=scale, out=o, workspace=ws0)
                                for kc, vc in caches])
        for ns in (0, 4, 8, 16, 32, 64, 128):
            ws = torch.empty(sfa.sf_attn_decode_workspace_bytes(batch, n, T, hq, hkv, d, mode, W, num_splits=ns) + 16,
                             dtype=torch.uint8, device=dev)
            calls = [lambda kc=kc, vc=vc: sfa.sf_attn_decode(q, kc, vc, T, mode, window=W, scale=scale, out=o,
                                                             workspace=ws, num_splits=ns) for kc, vc in caches]
            res[str(ns)] = round(min(_rotated_time(torch, calls) for _ in range(3)), 2)
        print(json.dumps({"decode_splits": f"{tag}_b{batch}", "bytes": nbytes, "us_by_splits": res}), flush=True)
        del caches, q, o
        torch.cuda.empty_cache()


def serving_sweep(torch, sfa, C, I, dev, budget=16 << 30):
    """Decode in its serving variants: the cross_window mask (W = 4096
    positions), n = 8 streams (32 query rows per kv head), and the paged cache
    with per-sequence lengths. Every call's data is rotated over >= 1 GiB of
    distinct reads (within `budget` bytes of caches)."""
    out = {}

    def record(key, us, nbytes, copies):
        gbps = nbytes / (us * 1e-6) / 1e9
        out[key] = {"us": round(us, 2), "GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "bytes": nbytes, "copies_rotated": copies}
        print(f"[bench] serving {key}: {us:.1f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)

    g = torch.Generator(device=dev).manual_seed(1007)

    def bf16(*shape):
        return torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)

    # contiguous cache: windowed decode and n = 8
    for tag, n, T, mode, W in (("window4096", 4, 8192, "cross_window", 4096),
                               ("n8_cross_full", 8, 4096, "cross_full", 0),
                               ("n8_intra", 8, 4096, "intra", 0)):
        for batch in (1, 8, 64):
            hq, hkv, d = 32, 8, 128
            nbytes = C.decode_bytes(mode, n, T, batch, hq, hkv, d, window=W)
            cache_bytes = 2 * batch * n * T * hkv * d * 2
            copies = max(1, min(math.ceil((1 << 30) / nbytes), budget // cache_bytes))
            q = bf16(batch, n, hq, d)
            caches = [(bf16(batch, n, T, hkv, d), bf16(batch, n, T, hkv, d)) for _ in range(copies)]
            o = torch.empty_like(q)
            ws = torch.empty(sfa.sf_attn_decode_workspace_bytes(batch, n, T, hq, hkv, d, mode, W) + 16,
                             dtype=torch.uint8, device=dev)
            scale = 1.0 / math.sqrt(d)
            calls = [lambda kc=kc, vc=vc: sfa.sf_attn_decode(q, kc, vc, T, mode, window=W, scale=scale, out=o,
                                                             workspace=ws) for kc, vc in caches]
            record(f"{tag}_b{batch}", _rotated_time(torch, calls), nbytes, copies)
            del caches, calls, q, o, ws
            torch.cuda.empty_cache()

    # paged cache, pages of 256 tokens: every sequence at 8192 tokens, and a
    # batch of lengths drawn uniformly from 1..8192
    n, hq, hkv, d, page = 4, 32, 8, 128, 256
    lg = torch.Generator().manual_seed(1008)
    for tag, batch, lens in (("paged_b8_8192", 8, [8192] * 8), ("paged_b64_8192", 64, [8192] * 64),
                             ("paged_b64_mixed", 64, torch.randint(1, 8193, (64,), generator=lg).tolist())):
        for mode in ("intra", "cross_full"):
            w = I.PagedDecodeWorkload(tag, n, tuple(lens), page, hq, hkv, d, mode, seed=1009, spare_pages=0)
            q, kp, vp, table, sl = I.paged_decode_inputs(w, device=dev)
            nbytes = sum(C.decode_bytes(mode, n, T, 1, hq, hkv, d) for T in lens)
            o = torch.empty_like(q)
            ws = torch.empty(sfa.sf_attn_decode_paged_workspace_bytes(batch, n, 8192, hq, hkv, d, mode) + 16,
                             dtype=torch.uint8, device=dev)
            call = lambda: sfa.sf_attn_decode_paged(q, kp, vp, table, sl, mode, max_T=8192,  # noqa: E731
                                                    scale=w.scale, out=o, workspace=ws)
            record(f"{tag}_{mode}", _rotated_time(torch, [call]), nbytes, 1)
            del q, kp, vp, table, sl, o, ws
            torch.cuda.empty_cache()
    return out


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, C, I, qs, ks, vs, target_s):
    """The fp64 oracle, as it stands, on evenly spaced query rows of the same
    32k cross_full workload (all heads). The rows are split into blocks that
    a pool of one worker thread per core of this process's affinity mask (at
    most its OMP_NUM_THREADS share) computes, each with one BLAS thread (NumPy
    releases the interpreter lock inside its matrix products, exponentials and
    comparisons). Scaled to useful TFLOP/s with the same pair count the GPU
    figure uses."""
    import concurrent.futures

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle.sfa as orc
    w = I.CROSS_32K
    n, L, S = w.n, w.L, w.S
    # the process's affinity mask, at most its OMP_NUM_THREADS share (16 on a one-GPU machine)
    cores = max(1, min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS") or 16)))
    # the oracle reads the expanded layout; build it on the CPU by its own interleave
    q = orc.interleave(qs.to("cpu", torch.float64).numpy())
    k = orc.interleave(ks.to("cpu", torch.float64).numpy())
    v = orc.interleave(vs.to("cpu", torch.float64).numpy())

    def run(nrows):
        rows = np.unique(np.linspace(0, S - 1, nrows).astype(np.int64))
        parts = [r for r in np.array_split(rows, 4 * cores) if len(r)]
        t = time.perf_counter()
        with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(cores) as ex:
            list(ex.map(lambda r: orc.attn_fwd(q, k, v, "cross_full", n, scale=w.scale, rows=r), parts))
        dt = time.perf_counter() - t
        pairs = int(np.sum(rows + 1))          # causal: row p admits p+1 keys
        return rows, dt, 4 * w.d * pairs * w.batch * w.hq

    rows, dt, fl = run(16 * cores)
    for _ in range(2):     # the time is not quite linear in the rows: calibrate twice
        if dt >= 0.6 * target_s or len(rows) >= S:
            break
        rows, dt, fl = run(int(min(S, len(rows) * target_s / max(dt, 1e-3))))
    blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                     if p.get("user_api") == "blas") or "unknown"
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{len(rows)} evenly spaced query rows of the cross_full 32k workload, all {w.hq} heads, "
                  f"fp64 NumPy, {cores} worker threads with one BLAS thread each, {dt:.1f} s",
        "seconds": round(dt, 2),
        "cpu_model": _cpu_model(),
        "numpy": np.__version__,
        "blas": blas,
    }


if __name__ == "__main__":
    main()
