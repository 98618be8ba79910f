"""Expansion front-end on the GPU against the oracle: sf_expand_embed (gather
from n embedding tables + interleave, bit-exact) and sf_rope (rotary encoding
at continuous expanded positions)."""
import numpy as np
import pytest
import torch

import hidden_decoding_stream_amd as sfa
import hidden_decoding_stream_amd.inputs as I
import oracle.sfa as orc
from gpu_util import assert_close, np64, say

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.detach().cpu().view(view).numpy()


@pytest.mark.parametrize("n,L,B,vocab,row,dtype", [
    (4, 64, 1, 100, 128, torch.bfloat16),
    (4, 37, 2, 50, 4096, torch.bfloat16),
    (3, 11, 2, 9, 7, torch.int16),          # 14-byte rows: 2-byte vectors
    (2, 5, 3, 4, 3, torch.uint8),           # 3-byte rows
    (1, 20, 1, 30, 24, torch.float32),      # n = 1: a plain gather
])
def test_expand_embed_small(n, L, B, vocab, row, dtype):
    say("expand_embed", n, L, B, vocab, row, dtype)
    g = torch.Generator().manual_seed(5 + L)
    tables = torch.randint(-1000, 1000, (n, vocab, row), generator=g).to(dtype)
    ids = torch.randint(0, vocab, (B, L), generator=g, dtype=torch.int32)
    ids[0, 0] = -3                    # out of range: zero rows
    ids[-1, -1] = vocab
    out = sfa.sf_expand_embed(ids.cuda(), tables.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), orc.expand_embed(ids.numpy(), _bits(tables)))


def test_expand_embed_full_size():
    """n = 4 tables of 32000 x 4096 bf16 (1 GiB), 8192 tokens: sampled tokens,
    all streams, bit-exact."""
    n, L, vocab, hidden = 4, 8192, 32000, 4096
    say("expand_embed full size")
    g = torch.Generator(device="cuda").manual_seed(1005)
    tables = torch.randn((n, vocab, hidden), generator=g, device="cuda").to(torch.bfloat16)
    ids = torch.randint(0, vocab, (1, L), generator=g, device="cuda", dtype=torch.int32)
    out = sfa.sf_expand_embed(ids, tables)
    torch.cuda.synchronize()
    toks = np.array(sorted({0, 1, 2, 63, 64, 1000, 4095, 4096, L - 2, L - 1}))
    ids_s = ids[:, toks].cpu().numpy()
    used = np.unique(ids_s)
    sub = tables[:, torch.from_numpy(used).cuda().long()]
    remap = np.searchsorted(used, ids_s).astype(np.int32)
    ref = orc.expand_embed(remap, _bits(sub))                          # [1][n*len(toks)][hidden]
    rows = (toks[:, None] * n + np.arange(n)[None, :]).reshape(-1)
    assert np.array_equal(_bits(out[:, rows]), ref)


@pytest.mark.parametrize("S,H,d,base,pos0", [
    (64, 4, 128, 10000.0, 0),
    (300, 2, 64, 10000.0, 1000),
    (17, 3, 256, 500000.0, 32760),
    (50, 1, 8, 10000.0, 7),
    (40, 2, 24, 10000.0, 3),                # d a multiple of 8 but not of 16
    (2, 32, 128, 10000.0, (1 << 31) - 5),   # positions past 2^31
])
def test_rope_small(S, H, d, base, pos0):
    say("rope", S, H, d, base, pos0)
    g = torch.Generator().manual_seed(S + d)
    x = I.to_bf16(torch.randn((2, S, H, d), generator=g))
    y = sfa.sf_rope(x.cuda(), base=base, pos0=pos0)
    torch.cuda.synchronize()
    ref = orc.rope(np64(x), base, pos0)
    got = np64(y)
    assert_close(got, ref, f"rope S={S} d={d} pos0={pos0}")
    # one bf16 rounding of the exact value: half an ulp, plus fp32 arithmetic
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4), "beyond one bf16 rounding"


def test_rope_rows_8_byte_aligned():
    # rows only 8-byte aligned, the least the call accepts; nothing outside the tensor is written
    S, H, d = 33, 3, 128
    g = torch.Generator().manual_seed(77)
    x = I.to_bf16(torch.randn((1, S, H, d), generator=g))
    buf = torch.zeros(S * H * d + 4, dtype=torch.bfloat16, device="cuda")
    xv = buf[4:].view(1, S, H, d)
    xv.copy_(x.cuda())
    assert xv.data_ptr() % 16 == 8
    y = sfa.sf_rope(xv, base=10000.0, pos0=5)
    torch.cuda.synchronize()
    assert_close(np64(y), orc.rope(np64(x), 10000.0, 5), "rope 8-byte aligned rows")
    assert torch.equal(buf[:4].cpu(), torch.zeros(4, dtype=torch.bfloat16)), "wrote before the tensor"


def test_rope_full_size_q():
    """Q of the 32k workload (32768 positions, 32 heads, d=128): sampled rows."""
    w = I.CROSS_32K
    say("rope full size")
    q, _, _ = I.workload_qkv(w, device="cuda")
    y = sfa.sf_rope(q.clone(), base=10000.0)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 4095, 4096, 16383, 16384, w.S - 2, w.S - 1}))
    # each sampled row at its own position
    ref = np.concatenate([orc.rope(np64(q[:, r:r + 1]), 10000.0, int(r)) for r in rows], axis=1)
    got = np64(y[:, rows])
    assert_close(got, ref, "rope 32k")
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)
