"""sf_attn_decode on the GPU against the fp64 oracle, and against the last n
rows of the GPU prefill over the same tokens."""
import math

import numpy as np
import pytest
import torch

import hidden_decoding_stream_amd as sfa
import hidden_decoding_stream_amd.inputs as I
import oracle.sfa as orc
from gpu_util import assert_close, np64, pooled, say

pytestmark = pytest.mark.gpu


def _scale(d):
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


SMALL = [
    # B, n, T, T_max, hq, hkv, d, mode, window
    (2, 4, 37, 50, 8, 2, 128, "cross_full", 0),
    (2, 4, 37, 50, 8, 2, 128, "intra", 0),
    (2, 4, 37, 50, 8, 2, 128, "cross_window", 33),
    (1, 4, 37, 37, 8, 2, 128, "cross_window", 1),
    (1, 4, 300, 300, 4, 4, 64, "cross_window", 10),
    (3, 2, 129, 200, 8, 1, 64, "intra", 0),
    (1, 3, 1, 4, 6, 2, 128, "cross_full", 0),          # a single token
    (1, 1, 500, 512, 16, 1, 128, "cross_full", 0),     # n = 1, G = 16
    (2, 4, 1000, 1000, 32, 8, 128, "cross_full", 0),
    # more query rows per kv head than one 16-row block: n = 8 (the pages' probe), larger G
    (1, 8, 70, 80, 16, 4, 128, "cross_full", 0),         # 32 rows
    (1, 8, 70, 80, 16, 4, 128, "cross_window", 100),
    (2, 8, 40, 40, 8, 1, 64, "cross_full", 0),           # 64 rows
    (1, 16, 33, 40, 8, 2, 128, "cross_full", 0),         # n = 16: 64 rows
    (1, 3, 50, 60, 16, 2, 128, "cross_full", 0),         # 24 rows: second block half used
    (1, 6, 45, 50, 16, 2, 64, "cross_window", 40),       # 48 rows
    (1, 4, 60, 64, 64, 2, 128, "intra", 0),              # G = 32 under intra
    (1, 2, 60, 64, 64, 1, 64, "intra", 0),               # G = 64 under intra
    (2, 4, 200, 210, 12, 4, 128, "cross_full", 0),       # G = 3: 12 rows
    (1, 4, 150, 150, 6, 1, 64, "intra", 0),              # G = 6 under intra
]


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_vs_oracle(case, splits):
    B, n, T, Tm, hq, hkv, d, mode, W = case
    say("decode small", case, "splits", splits)
    w = I.DecodeWorkload("t", n, T, Tm, B, hq, hkv, d, mode, window=W, seed=T + 7)
    q, kc, vc = I.decode_inputs(w)
    o = sfa.sf_attn_decode(q.cuda(), kc.cuda(), vc.cuda(), T, mode, window=W, scale=_scale(d), num_splits=splits)
    torch.cuda.synchronize()
    ref = orc.decode(np64(q), np64(kc), np64(vc), T, mode, window=W or None, scale=_scale(d))
    assert_close(np64(o), ref, f"{case} splits={splits}")


@pytest.mark.parametrize("n,hq,hkv", [(4, 8, 2), (8, 16, 2)])
@pytest.mark.parametrize("mode,W", [("intra", 0), ("cross_full", 0), ("cross_window", 45)])
def test_decode_is_last_rows_of_prefill(mode, W, n, hq, hkv):
    B, T, d = 1, 300, 128
    say("decode vs prefill", mode, n)
    w = I.DecodeWorkload("t", n, T, T, B, hq, hkv, d, mode, window=W, seed=3)
    q, kc, vc = (t.cuda() for t in I.decode_inputs(w))
    o = sfa.sf_attn_decode(q, kc, vc, T, mode, window=W, scale=_scale(d))
    # expanded sequence: [B][n][T][hkv][d] -> [n][B][T][hkv*d] -> interleave -> [B][n*T][hkv][d]
    K = sfa.sf_interleave(kc.permute(1, 0, 2, 3, 4).contiguous(), n).view(B, n * T, hkv, d)
    V = sfa.sf_interleave(vc.permute(1, 0, 2, 3, 4).contiguous(), n).view(B, n * T, hkv, d)
    Q = torch.zeros((B, n * T, hq, d), dtype=torch.bfloat16, device="cuda")
    Q[:, (T - 1) * n:] = q
    full = sfa.sf_attn_fwd(Q, K, V, mode, n, window=W, scale=_scale(d))
    torch.cuda.synchronize()
    assert_close(np64(o), np64(full[:, (T - 1) * n:]), f"decode vs prefill {mode}", max_abs=1e-2, mean_abs=1e-3)


@pytest.mark.parametrize("mode", ["intra", "cross_full"])
@pytest.mark.parametrize("batch", [1, 8, 64])
def test_full_size(batch, mode):
    """The decode workload (8192 tokens x 4 streams, 32/8 heads, d=128) in the
    benchmark's launch configuration; every output element against the
    oracle (one oracle call per batch element, in parallel threads)."""
    w = I.decode_workload(batch, mode)
    say("decode full size", w.name)
    q, kc, vc = I.decode_inputs(w, device="cuda")
    o = sfa.sf_attn_decode(q, kc, vc, w.T, mode, scale=w.scale)
    o2 = sfa.sf_attn_decode(q, kc, vc, w.T, mode, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "decode must be deterministic"
    ref = pooled(lambda b: orc.decode(np64(q[b:b + 1]), np64(kc[b:b + 1]), np64(vc[b:b + 1]), w.T, mode,
                                      scale=w.scale)[0], list(range(batch)))
    assert_close(np64(o), np.stack(ref), f"{w.name} all {batch} batch elements")
    del q, kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [1, 8])
def test_full_size_window(batch):
    """Windowed decode at the serving size (8192 tokens x 4 streams, W = 4096
    positions, 32/8 heads, d = 128) with the library's plan (32 splits of one
    step per wave at batch 1): every output element against the oracle."""
    w = I.DecodeWorkload("window4096", 4, 8192, 8192, batch, 32, 8, 128, "cross_window", window=4096, seed=1011)
    say("decode full size window", batch)
    q, kc, vc = I.decode_inputs(w, device="cuda")
    o = sfa.sf_attn_decode(q, kc, vc, w.T, w.mode, window=w.window, scale=_scale(w.d))
    o2 = sfa.sf_attn_decode(q, kc, vc, w.T, w.mode, window=w.window, scale=_scale(w.d))
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "decode must be deterministic"
    ref = pooled(lambda b: orc.decode(np64(q[b:b + 1]), np64(kc[b:b + 1]), np64(vc[b:b + 1]), w.T, w.mode,
                                      window=w.window, scale=_scale(w.d))[0], list(range(batch)))
    assert_close(np64(o), np.stack(ref), f"window4096 all {batch} batch elements")
    del q, kc, vc
    torch.cuda.empty_cache()


def test_workspace_reused_across_calls():
    """One workspace, its contents left over from earlier calls, serves
    consecutive calls of different shapes, split counts and masks; each
    result matches the oracle."""
    ws = torch.full((1 << 22,), 0x7f, dtype=torch.uint8, device="cuda")    # not zero on purpose
    calls = [
        # B, n, T, T_max, hq, hkv, d, mode, window, splits
        (2, 4, 1000, 1000, 32, 8, 128, "cross_full", 0, 7),
        (1, 4, 300, 320, 8, 2, 64, "intra", 0, 5),
        (2, 4, 1000, 1000, 32, 8, 128, "cross_full", 0, 7),     # same shape again
        (1, 2, 777, 800, 8, 1, 128, "cross_window", 300, 2),
        (1, 4, 8192, 8192, 32, 8, 128, "cross_full", 0, 0),     # library-chosen splits
        (3, 4, 129, 129, 8, 2, 128, "cross_full", 0, 3),        # smaller after larger
    ]
    for i, (B, n, T, Tm, hq, hkv, d, mode, W, splits) in enumerate(calls):
        say("decode workspace reuse", i, mode, "splits", splits)
        w = I.DecodeWorkload("t", n, T, Tm, B, hq, hkv, d, mode, window=W, seed=100 + i)
        q, kc, vc = I.decode_inputs(w)
        need = sfa.sf_attn_decode_workspace_bytes(B, n, T, hq, hkv, d, mode, W, splits)
        assert need <= ws.numel()
        o = sfa.sf_attn_decode(q.cuda(), kc.cuda(), vc.cuda(), T, mode, window=W, scale=_scale(d),
                               num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        ref = orc.decode(np64(q), np64(kc), np64(vc), T, mode, window=W or None, scale=_scale(d))
        assert_close(np64(o), ref, f"reuse call {i}")
