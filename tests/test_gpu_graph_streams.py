"""Serving-side use of the library on the GPU: calls captured in a HIP graph
(torch.cuda.CUDAGraph) and replayed on new inputs, and calls on two streams
at once. The kernels are deterministic and the library allocates and clears
nothing itself, so every replay and every concurrent call must equal the
eager, sequential result bit for bit."""
import math

import pytest
import torch

import hidden_decoding_stream_amd as sfa
import hidden_decoding_stream_amd.inputs as I
from gpu_util import say

pytestmark = pytest.mark.gpu


def _scale(d):
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _fill(t, g):
    t.copy_(torch.randn(t.shape, generator=g, device=t.device).to(t.dtype))


def test_graph_replay_prefill_and_decode():
    n, L, B, hq, hkv, d, T = 4, 300, 2, 8, 2, 128, 700
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(11)
    q = torch.empty((B, n * L, hq, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((B, n * L, hkv, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((B, hq, n * L), dtype=torch.float32, device=dev)
    qn = torch.empty((B, n, hq, d), dtype=torch.bfloat16, device=dev)
    kc = torch.empty((B, n, T, hkv, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    on = torch.empty_like(qn)
    ws = torch.empty(sfa.sf_attn_decode_workspace_bytes(B, n, T, hq, hkv, d, "cross_full", 0, 3) + 16,
                     dtype=torch.uint8, device=dev)
    inputs = (q, k, v, qn, kc, vc)
    for t in inputs:
        _fill(t, g)

    def work():
        sfa.sf_attn_fwd(q, k, v, "cross_full", n, scale=_scale(d), out=o, lse=lse)
        sfa.sf_attn_decode(qn, kc, vc, T, "cross_full", scale=_scale(d), num_splits=3, out=on, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()                                   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for replay in range(4):
        say("graph replay", replay)
        for t in inputs:
            _fill(t, g)
        graph.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone(), on.clone())
        # eager work between replays, then the same inputs eagerly
        scratch = torch.randn((1 << 20,), device=dev).sum()
        work()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(got[0], o) and torch.equal(got[1], lse) and torch.equal(got[2], on), replay


def test_two_streams_at_once():
    """A prefill on one stream and a decode on another, overlapping, each
    equal to the same call run alone."""
    dev = torch.device("cuda")
    w = I.CROSS_32K
    q, k, v = I.workload_qkv(w, device=dev)
    wd = I.decode_workload(8, "cross_full")
    qn, kc, vc = I.decode_inputs(wd, device=dev)
    say("two streams")
    ref_o = sfa.sf_attn_fwd(q, k, v, w.mode, w.n, scale=w.scale)
    ref_d = sfa.sf_attn_decode(qn, kc, vc, wd.T, wd.mode, scale=wd.scale)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o = torch.empty_like(ref_o)
    od = torch.empty_like(ref_d)
    ws = torch.empty(sfa.sf_attn_decode_workspace_bytes(8, wd.n, wd.T, wd.hq, wd.hkv, wd.d, wd.mode) + 16,
                     dtype=torch.uint8, device=dev)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        sfa.sf_attn_fwd(q, k, v, w.mode, w.n, scale=w.scale, out=o)
    with torch.cuda.stream(s2):
        for _ in range(5):
            sfa.sf_attn_decode(qn, kc, vc, wd.T, wd.mode, scale=wd.scale, out=od, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o)
    assert torch.equal(od, ref_d)


def test_graph_replay_whole_step():
    """The whole hot path as one captured graph: Q, K, V interleaved in one
    launch, cross_full and intra prefill, K and V de-interleaved in one launch
    into the per-stream cache, and the decode of the last token's n streams
    from it. Every replay on refilled inputs equals the eager step bit for
    bit."""
    n, L, B, hq, hkv, d = 4, 200, 1, 8, 2, 128
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(12)
    qs = torch.empty((n, B, L, hq, d), dtype=torch.bfloat16, device=dev)
    ks = torch.empty((n, B, L, hkv, d), dtype=torch.bfloat16, device=dev)
    vs = torch.empty_like(ks)
    Q = torch.empty((B, n * L, hq, d), dtype=torch.bfloat16, device=dev)
    K = torch.empty((B, n * L, hkv, d), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    Oc, Oi = torch.empty_like(Q), torch.empty_like(Q)
    kc = torch.empty((n, B, L, hkv, d), dtype=torch.bfloat16, device=dev)   # == [B][n][L][hkv][d] at B = 1
    vc = torch.empty_like(kc)
    q_new = torch.empty((B, n, hq, d), dtype=torch.bfloat16, device=dev)
    od = torch.empty_like(q_new)
    ws = torch.zeros(sfa.sf_attn_decode_workspace_bytes(B, n, L, hq, hkv, d, "cross_full") + 16,
                     dtype=torch.uint8, device=dev)
    s = _scale(d)

    def refill():
        for t in (qs, ks, vs):
            _fill(t, g)

    def step():
        sfa.sf_interleave_multi([qs, ks, vs], n, outs=[Q, K, V])
        sfa.sf_attn_fwd(Q, K, V, "cross_full", n, scale=s, out=Oc)
        sfa.sf_attn_fwd(Q, K, V, "intra", n, scale=s, out=Oi)
        sfa.sf_interleave_multi([K, V], n, inverse=True, outs=[kc, vc])
        q_new.copy_(qs[:, 0, L - 1].unsqueeze(0))
        sfa.sf_attn_decode(q_new, kc.view(B, n, L, hkv, d), vc.view(B, n, L, hkv, d), L, "cross_full",
                           scale=s, out=od, workspace=ws)

    refill()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    outs = (Q, K, V, Oc, Oi, kc, vc, od)
    for replay in range(3):
        say("whole-step graph replay", replay)
        refill()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        step()
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a, b), replay
        assert torch.equal(kc, ks) and torch.equal(vc, vs)
