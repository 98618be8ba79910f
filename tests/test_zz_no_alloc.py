"""sf_attn_decode_noalloc: the decode without a workspace argument, its split
partials in the library's fixed per-GPU scratch array.

Through the C ABI (the binding only marshals arguments), two calls in a row
(the second smaller, so it runs over what the first left in the scratch) are
compared with sf_attn_decode on the same inputs, bitwise (same kernels and
split plan), and with the fp64 oracle at the accuracy bar. A plan that needs
more scratch than the array holds is refused before any launch."""
import math

import numpy as np
import pytest
import torch

import hidden_decoding_stream_amd as sfa
import hidden_decoding_stream_amd.inputs as I
import oracle.sfa as orc
from gpu_util import assert_close, np64, say

pytestmark = pytest.mark.gpu


def _scale(d):
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


CALLS = [
    # B, n, T, T_max, hq, hkv, d, mode, window, splits
    (1, 4, 8192, 8192, 32, 8, 128, "cross_full", 0, 0),     # the batch-1 decode workload: 32 splits
    (2, 4, 1000, 1024, 8, 2, 64, "intra", 0, 3),            # smaller, after it
]


def test_noalloc_matches_workspace_decode_twice():
    for i, (B, n, T, Tm, hq, hkv, d, mode, W, splits) in enumerate(CALLS):
        say("decode noalloc call", i, (B, n, T, Tm, hq, hkv, d, mode, W, splits))
        need = sfa.sf_attn_decode_workspace_bytes(B, n, T, hq, hkv, d, mode, W, splits)
        assert 0 < need <= 16 << 20, "the case must use the scratch, within its size"
        w = I.DecodeWorkload("t", n, T, Tm, B, hq, hkv, d, mode, window=W, seed=200 + i)
        q, kc, vc = (t.cuda() for t in I.decode_inputs(w))
        o_ref = sfa.sf_attn_decode(q, kc, vc, T, mode, window=W, scale=_scale(d), num_splits=splits)
        o = torch.full_like(q, float("nan"))
        sfa.sf_attn_decode_noalloc(q, kc, vc, T, mode, window=W, scale=_scale(d), num_splits=splits, out=o)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {i}: differs from sf_attn_decode"
        ref = orc.decode(np64(q), np64(kc), np64(vc), T, mode, window=W or None, scale=_scale(d))
        assert_close(np64(o), ref, f"noalloc call {i}")


def test_noalloc_refuses_oversized_plan():
    say("decode noalloc oversized plan")
    B, n, T, hq, hkv, d = 4, 4, 8192, 32, 8, 128
    need = sfa.sf_attn_decode_workspace_bytes(B, n, T, hq, hkv, d, "cross_full", 0, 1024)
    assert need > (16 << 20)
    q = torch.zeros((B, n, hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, n, T, hkv, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    with pytest.raises(sfa.SFError, match="scratch"):
        sfa.sf_attn_decode_noalloc(q, kc, kc, T, "cross_full", num_splits=1024, out=o)
    assert not torch.any(o), "a refused call must launch nothing"
