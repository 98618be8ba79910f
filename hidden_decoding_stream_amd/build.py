"""Build libsfattn.so in-tree with hipcc for gfx950.

    python -m hidden_decoding_stream_amd.build

Compiles the HIP sources under csrc/ to objects in _build/ (at the repository
root) and links them into hidden_decoding_stream_amd/libsfattn.so (the
attention library), hidden_decoding_stream_amd/libsfpeaks.so (attainable-
peak microbenchmarks) and hidden_decoding_stream_amd/libsfattn_trace.so (the
attention library with the prefill's per-work-group timeline compiled in,
SFA_PREFILL_TRACE). The last two are used only for measurement. Always
recompiles: it is the "does it build" check as well as the build.
"""
from __future__ import annotations

import concurrent.futures
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libsfattn.so"
SOURCES = ["api.hip", "interleave.hip", "frontend.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip"]
PEAKS_LIB = PKG / "libsfpeaks.so"
PEAKS_SOURCES = ["peaks.hip"]
TRACE_LIB = PKG / "libsfattn_trace.so"

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled: the compiler would otherwise form them
# from ordinary float code on its own.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsfattn)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _link(cc, objs, lib):
    tmp = lib.with_name(lib.name + ".tmp")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)])
    os.replace(tmp, lib)


def build(verbose: bool = False, extra_flags=()) -> pathlib.Path:
    cc = hipcc()
    BUILD.mkdir(exist_ok=True)
    cmds = []
    for src in SOURCES + PEAKS_SOURCES:
        obj = BUILD / (pathlib.Path(src).stem + ".o")
        cmds.append((obj, [cc, *FLAGS, *extra_flags, "-c", str(CSRC / src), "-o", str(obj)]))
    trace_obj = BUILD / "attn_fwd_trace.o"
    cmds.append((trace_obj, [cc, *FLAGS, *extra_flags, "-DSFA_PREFILL_TRACE", "-c", str(CSRC / "attn_fwd.hip"),
                             "-o", str(trace_obj)]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        for (_, cmd), r in zip(cmds, ex.map(_run, [c for _, c in cmds])):
            if verbose:
                print(" ".join(cmd))
                sys.stdout.write(r.stderr)
    objs = {pathlib.Path(o).stem: o for o, _ in cmds}
    _link(cc, [objs[pathlib.Path(s).stem] for s in SOURCES], LIB)
    _link(cc, [objs[pathlib.Path(s).stem] for s in PEAKS_SOURCES], PEAKS_LIB)
    _link(cc, [objs["attn_fwd_trace"] if s == "attn_fwd.hip" else objs[pathlib.Path(s).stem] for s in SOURCES],
          TRACE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
