"""Helpers shared by the GPU parity tests (comparison, sampling, probes)."""
from __future__ import annotations

import concurrent.futures
import os
import sys

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import oracle.sfa as orc

# Accuracy bar for bf16 inputs with fp32 accumulation against the fp64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(got, ref, what="", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    say(f"{what}: max|err| {mx:.3e} mean|err| {mn:.3e}")
    assert mx <= max_abs, f"{what}: max abs error {mx} > {max_abs}"
    assert mn <= mean_abs, f"{what}: mean abs error {mn} > {mean_abs}"


def sample_rows(S: int, seed: int = 0, extra: int = 8, tile: int = 64, window: int = 0):
    """Query rows at tile edges, window edges, both ends, and a few random."""
    rows = {0, 1, 2, 3, tile - 1, tile, tile + 1, 2 * tile - 1, 255, 256, S // 2, S - 4, S - 3, S - 2, S - 1}
    for base in (1024, 4096, 4097, 8191, 8192, 16383, 16384):
        rows.add(base)
    if window:
        for w in (window - 1, window, window + 1, window + tile):
            rows.add(w)
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, S, size=extra))
    return np.array(sorted(r for r in rows if 0 <= r < S))


def probe_values(S: int, hkv: int, d: int, cols, batch: int = 1, device="cuda"):
    """V one-hot on chosen key columns: V[b][cols[j]][h][j] = 1."""
    v = torch.zeros((batch, S, hkv, d), dtype=torch.bfloat16)
    for j, c in enumerate(cols):
        v[:, c, :, j] = 1.0
    return v.to(device)


def oracle_mask_cols(mode, n, L, window, rows, cols, block=1024):
    """Mask entries [rows][cols] and row popcounts, from the oracle's mask."""
    sub = np.empty((len(rows), len(cols)), dtype=bool)
    cnt = np.empty(len(rows), dtype=np.int64)
    for r0 in range(0, len(rows), block):
        M = orc.mask(mode, n, L, window, rows[r0:r0 + block])
        sub[r0:r0 + block] = M[:, cols]
        cnt[r0:r0 + block] = M.sum(axis=1)
    return sub, cnt


def cpu_share() -> int:
    """Worker threads for oracle runs: the cores of this process's affinity
    mask, at most its OMP_NUM_THREADS share (16 on a one-GPU machine)."""
    cap = int(os.environ.get("OMP_NUM_THREADS") or 16)
    return max(1, min(len(os.sched_getaffinity(0)), cap))


def pooled(fn, items, blas_threads: int = 1):
    """fn over items on cpu_share() threads, each with `blas_threads` BLAS
    threads (NumPy releases the interpreter lock in its array work)."""
    with threadpool_limits(blas_threads), concurrent.futures.ThreadPoolExecutor(cpu_share()) as ex:
        return list(ex.map(fn, items))


def oracle_fwd_head(q, k, v, mode, n, window, scale, rows=None, block=512):
    """The oracle's attention of one head over all (or the given) query rows:
    q [S][D], k, v [S][D] (float64). Row blocks go to a thread pool; each
    block is one plain call of the oracle. Returns (o [R][D], lse [R])."""
    S = q.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    q4, k4, v4 = q[None, :, None], k[None, :, None], v[None, :, None]
    parts = [rows[i:i + block] for i in range(0, len(rows), block)]
    res = pooled(lambda r: orc.attn_fwd(q4, k4, v4, mode, n, window=window, scale=scale, rows=r, with_lse=True),
                 parts)
    o = np.concatenate([x[0][0, :, 0] for x in res])
    lse = np.concatenate([x[1][0, 0] for x in res])
    return o, lse


def assert_close_rows(got, ref, what, rel_max=2e-2, rel_mean=2e-3):
    """Gradient comparison normalised per row: each row r (last axis = d)
    must have max |err| <= rel_max * max(1, max_d |ref[r]|), and the mean of
    |err| / max(1, max_d |ref[r]|) over every element must be <= rel_mean.
    A gradient's size grows with the number of queries (or keys) that reach
    it, so a bar scaled by the whole tensor's largest row would be loose for
    every small row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    norm = np.maximum(1.0, np.abs(ref).max(axis=-1, keepdims=True))
    rel = np.abs(got - ref) / norm
    mx, mn = float(rel.max()), float(rel.mean())
    say(f"{what}: max|err|/rownorm {mx:.3e} mean {mn:.3e} (largest row norm {float(norm.max()):.3e})")
    assert mx <= rel_max, f"{what}: max row-normalised error {mx} > {rel_max}"
    assert mn <= rel_mean, f"{what}: mean row-normalised error {mn} > {rel_mean}"
