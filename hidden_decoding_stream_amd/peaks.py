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
        for f in (L.sfp_read, L.sfp_copy, L.sfp_mfma):
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


def mfma_bf16_flops(blocks: int = 256, iters: int = 4096, chains: int = 8, reps: int = 5) -> float:
    """Dense bf16 flop/s of back-to-back 32x32x16 MFMAs, one wave per SIMD
    with `chains` independent accumulators."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().sfp_mfma(out.data_ptr(), blocks, iters, chains, st), "sfp_mfma"), reps)
    return blocks * 4 * chains * iters * 32768 / t
