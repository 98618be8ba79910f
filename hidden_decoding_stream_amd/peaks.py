"""ctypes binding of libsfpeaks.so: attainable HBM read / copy bandwidth and
dense bf16 MFMA rate on the current GPU, timed with HIP events on the launch
stream. Measurement only; the attention path does not use it."""
from __future__ import annotations

import ctypes
import pathlib

import torch

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libsfpeaks.so"
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: run python -m hidden_decoding_stream_amd.build")
        L = ctypes.CDLL(str(LIB_PATH))
        c = ctypes
        L.sfp_read.argtypes = [c.c_void_p, c.c_size_t, c.c_void_p, c.c_int, c.c_void_p]
        L.sfp_copy.argtypes = [c.c_void_p, c.c_void_p, c.c_size_t, c.c_int, c.c_void_p]
        L.sfp_mfma.argtypes = [c.c_void_p, c.c_int, c.c_int, c.c_int, c.c_void_p]
        L.sfp_mfma_random.argtypes = [c.c_void_p, c.c_int, c.c_int, c.c_void_p]
        L.sfp_read_slices.argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int, c.c_int, c.c_void_p, c.c_void_p]
        L.sfp_read_slices_lds.argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int, c.c_int, c.c_int, c.c_void_p]
        L.sfp_decode_chain.argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int, c.c_int, c.c_void_p, c.c_void_p,
                                       c.c_void_p, c.c_int, c.c_void_p]
        for f in (L.sfp_read, L.sfp_copy, L.sfp_mfma, L.sfp_mfma_random, L.sfp_read_slices, L.sfp_read_slices_lds,
                  L.sfp_decode_chain):
            f.restype = c.c_int
        _lib = L
    return _lib


def _time(fn, reps: int) -> float:
    """Median seconds of fn() over reps launches, events on the current stream."""
    s = torch.cuda.current_stream()
    fn()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    times.sort()
    return times[len(times) // 2]


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} launch failed (hipError {rc})")


def read_bandwidth(nbytes: int = 2 << 30, blocks: int = 256 * 8, reps: int = 10) -> float:
    """Bytes/s of one streaming read of nbytes (larger than the 256 MiB
    Infinity Cache, so it comes from HBM)."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().sfp_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, st), "sfp_read"),
              reps)
    return nbytes / t


def copy_bandwidth(nbytes: int = 1 << 30, blocks: int = 256 * 8, reps: int = 10) -> float:
    """Bytes/s moved (read + write) by a device copy of nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().sfp_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, st), "sfp_copy"),
              reps)
    return 2 * nbytes / t


def mfma_bf16_flops(blocks: int = 256, iters: int = 32768, chains: int = 8, reps: int = 5) -> float:
    """Dense bf16 flop/s of back-to-back 32x32x16 MFMAs, one wave per SIMD
    with `chains` independent accumulators. The default launch runs about
    4 ms, as long as the 32k prefill: the clock under this load settles over
    a few milliseconds, and launches of under a millisecond read 10-15%
    high or low."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().sfp_mfma(out.data_ptr(), blocks, iters, chains, st), "sfp_mfma"), reps)
    return blocks * 4 * chains * iters * 32768 / t


def mfma_bf16_random_flops(blocks: int = 256, iters: int = 32768, reps: int = 5) -> float:
    """As mfma_bf16_flops with 8 chains, the operands rotating over four
    pairs of random bf16 values (the matrix core's inputs switch as on
    random data)."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().sfp_mfma_random(out.data_ptr(), blocks, iters, st), "sfp_mfma_random"), reps)
    return blocks * 4 * 8 * iters * 32768 / t


# batch-1 decode of the 32k workload: 4 streams x 8192 tokens of 8 kv heads, d = 128, bf16
DECODE_B1_ROWS, DECODE_B1_HEADS, DECODE_B1_SPLITS = 4 * 8192, 8, 32


def decode_structure_floor(rounds: int = 3, pairs: int = 8) -> dict:
    """Microseconds per call (median) of the batch-1 decode's bytes, in its
    pattern and grid (8 kv heads x 32 key ranges, each head's 256-byte slice
    of every K and V row, 134,217,728 bytes), with no arithmetic:
      read   the stream alone (DMA ring of 2 stages of 32 rows per wave);
      chain  the stream, a decode-sized partial per work group, and a second
             kernel merging the partials per output row (the library's
             split + combine structure);
      fused  the same in one launch, the last work group of each kv head
             merging its rows after a release fence and an atomic ticket.
    Each timed with HIP events around the call; `pairs` distinct K/V buffer
    pairs (1 GiB at 8) rotated so the 256 MiB Infinity Cache cannot serve
    repeats."""
    rows, heads, splits = DECODE_B1_ROWS, DECODE_B1_HEADS, DECODE_B1_SPLITS
    half = rows * heads * 256
    bufs = [torch.ones(half // 4, dtype=torch.int32, device="cuda") for _ in range(2 * pairs)]
    part = torch.empty(heads * 16 * splits * 130, dtype=torch.float32, device="cuda")
    ticket = torch.zeros(heads, dtype=torch.int32, device="cuda")
    out = torch.empty(heads * 16 * 128, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream()
    st = s.cuda_stream
    calls = {
        "read": lambda kb, vb: lib().sfp_read_slices_lds(kb, vb, rows, heads, splits, 2, st),
        "chain": lambda kb, vb: lib().sfp_decode_chain(kb, vb, rows, heads, splits, part.data_ptr(),
                                                       ticket.data_ptr(), out.data_ptr(), 0, st),
        "fused": lambda kb, vb: lib().sfp_decode_chain(kb, vb, rows, heads, splits, part.data_ptr(),
                                                       ticket.data_ptr(), out.data_ptr(), 1, st),
    }
    res = {}
    for name, fn in calls.items():
        _check(fn(bufs[0].data_ptr(), bufs[1].data_ptr()), f"decode floor {name}")
        ev = []
        for _ in range(rounds):
            for i in range(pairs):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(s)
                _check(fn(bufs[2 * i].data_ptr(), bufs[2 * i + 1].data_ptr()), f"decode floor {name}")
                b.record(s)
                ev.append((a, b))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        res[name + "_us"] = round(t[len(t) // 2], 2)
        res[name + "_min_us"] = round(t[0], 2)
    if int(ticket.abs().sum().item()) != 0:
        raise RuntimeError("decode floor: fused tickets not reset")
    res["bytes"] = 2 * half
    return res
