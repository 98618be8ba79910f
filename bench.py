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
prefill, timed with HIP events around its own launches), a decode bandwidth
sweep (batch 1, 8, 64; intra and cross_full) and the CPU oracle timed on a
bounded sample of the same workload.

Inputs are synthetic (seeded N(0,1), rounded to bf16) and resident in HBM
before timing starts. Only one GPU is used.
"""
from __future__ import annotations

import argparse
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
PROFILE_PMC = ROOT / "profiles" / "attn_fwd_cross_full_32k_pmc.txt"
FWD_SOURCE = ROOT / "hidden_decoding_stream_amd" / "csrc" / "attn_fwd.hip"


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
                    help="only run decode calls for counter runs (batch 1 and 8, cross_full and intra, "
                         "3 calls each on distinct caches), then exit")
    return ap.parse_args()


def source_sha(path: pathlib.Path) -> str:
    return hashlib.sha256(path.read_bytes()).hexdigest()[:16]


def stored_traffic():
    """HBM traffic of one cross_full 32k prefill launch, from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    if not PROFILE_PMC.exists():
        return None
    text = PROFILE_PMC.read_text()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(FWD_SOURCE):
        return None
    return float(m_b.group(1))


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

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
            "kernel": "attn_fwd_kernel<128, 1, false> (cross_full) 32k",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
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


def attainable_peaks(line):
    """The chip's attainable peaks measured on this GPU (back-to-back dense
    bf16 MFMAs; a streaming read of 2 GiB, beyond the Infinity Cache), and the
    headline prefill and the decode sweep as fractions of them, beside the
    published peaks that `roofline` uses."""
    import hidden_decoding_stream_amd.peaks as P
    mfma = P.mfma_bf16_flops() / 1e12
    read = P.read_bandwidth() / 1e9
    out = {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_GBps": round(read, 1),
           "prefill_cross_full_frac": round(line["roofline"]["achieved"] / mfma, 4)}
    for key, rec in (line.get("decode") or {}).items():
        out[f"decode_{key}_frac"] = round(rec["GBps"] / read, 4)
    print(f"[bench] attainable: {mfma:.0f} TFLOP/s bf16, {read:.0f} GB/s read", file=sys.stderr, flush=True)
    return out


def last_stream_timing(torch, sfa, C, Q, K, V, n, L, B, hq, d, scale, stream, reps=10):
    """Attention of stream n-1's queries only (one per token) against all
    streams' K/V of the same 32k workload: useful TFLOP/s per mode."""
    ql = Q[:, n - 1::n].contiguous()
    o = torch.empty_like(ql)
    out = {}
    for mode in ("cross_full", "intra"):
        for _ in range(2):
            sfa.sf_attn_fwd_last_stream(ql, K, V, mode, n, scale=scale, out=o)
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
        call()
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


def cpu_baseline(torch, C, I, qs, ks, vs, target_s):
    """The fp64 oracle, as it stands, on evenly spaced query rows of the same
    32k cross_full workload (all heads). Scaled to useful TFLOP/s with the
    same pair count the GPU figure uses."""
    import numpy as np

    import oracle.sfa as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    w = I.CROSS_32K
    n, L, S = w.n, w.L, w.S
    # the oracle reads the expanded layout; build it on the CPU by its own interleave
    q = orc.interleave(qs.to("cpu", torch.float64).numpy())
    k = orc.interleave(ks.to("cpu", torch.float64).numpy())
    v = orc.interleave(vs.to("cpu", torch.float64).numpy())

    def run(nrows):
        rows = np.unique(np.linspace(0, S - 1, nrows).astype(np.int64))
        t = time.perf_counter()
        orc.attn_fwd(q, k, v, "cross_full", n, scale=w.scale, rows=rows)
        dt = time.perf_counter() - t
        pairs = int(np.sum(rows + 1))          # causal: row p admits p+1 keys
        return rows, dt, 4 * w.d * pairs * w.batch * w.hq

    rows, dt, fl = run(64)
    nrows = int(min(S, max(64, 64 * target_s / max(dt, 1e-3))))
    rows, dt, fl = run(nrows)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(rows)} evenly spaced query rows of the cross_full 32k workload, all {w.hq} heads, "
                  f"fp64 NumPy, {dt:.1f} s",
        "seconds": round(dt, 2),
    }


if __name__ == "__main__":
    main()
