"""sf_interleave on the GPU: bit-exact against the oracle's interleave."""
import numpy as np
import pytest
import torch

import hidden_decoding_stream_amd as sfa
import hidden_decoding_stream_amd.inputs as I
import oracle.sfa as orc
from gpu_util import say

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    """The raw bytes of a tensor as a numpy array of the same shape."""
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.detach().cpu().view(view).numpy()


def test_tiny_fp32_forward_and_inverse():
    say("interleave tiny fp32")
    q, _, _ = I.stream_qkv(4, 64, 1, 4, 64, 64, seed=1000, dtype="fp32")  # [4][1][64][4][64]
    x = q.cuda()
    y = sfa.sf_interleave(x, 4)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), orc.interleave(_bits(q)))
    back = sfa.sf_interleave(y, 4, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), q)


@pytest.mark.parametrize("n,L,B,row_elems,dtype", [
    (1, 37, 2, 24, torch.bfloat16),       # n = 1 is a copy
    (3, 5, 2, 7, torch.int16),             # 14-byte rows: 2-byte vectors
    (4, 9, 3, 3, torch.uint8),             # 3-byte rows: byte vectors
    (2, 33, 1, 6, torch.int32),            # 24-byte rows: 8-byte vectors
    (5, 17, 2, 1000, torch.bfloat16),      # ragged tails, many tiles
])
def test_ragged_shapes(n, L, B, row_elems, dtype):
    say("interleave ragged", n, L, B, row_elems, dtype)
    g = torch.Generator().manual_seed(7)
    src = torch.randint(-100, 100, (n, B, L, row_elems), generator=g).to(dtype)
    y = sfa.sf_interleave(src.cuda(), n)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), orc.interleave(_bits(src)))
    back = sfa.sf_interleave(y, n, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back), _bits(src))


def test_unaligned_pointers():
    say("interleave unaligned")
    n, L, B, R = 4, 11, 2, 16
    buf = torch.randint(0, 255, (n * B * L * R + 1,), dtype=torch.uint8)
    src = buf[1:].view(n, B, L, R)
    # misaligned device pointers (offset views of one allocation)
    dbuf = torch.zeros(n * B * L * R + 8, dtype=torch.uint8, device="cuda")
    dbuf[3:3 + src.numel()] = src.reshape(-1).cuda()
    dout = torch.zeros(B * n * L * R + 8, dtype=torch.uint8, device="cuda")
    st = sfa.lib().sf_interleave(dbuf.data_ptr() + 3, dout.data_ptr() + 5, n, L, B, R, 0,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    got = dout[5:5 + src.numel()].cpu().numpy().reshape(B, n * L, R)
    assert np.array_equal(got, orc.interleave(src.numpy()))


@pytest.mark.parametrize("w", [I.INTRA_16K, I.CROSS_32K], ids=lambda w: w.name)
def test_full_size_qkv(w):
    say("interleave full size", w.name)
    q, k, v = I.stream_qkv(w.n, w.L, w.batch, w.hq, w.hkv, w.d, seed=w.seed, device="cuda")
    for name, t in (("q", q), ("k", k), ("v", v)):
        y = sfa.sf_interleave(t, w.n)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), orc.interleave(_bits(t))), name
    back = sfa.sf_interleave(sfa.sf_interleave(k, w.n), w.n, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back, k)


@pytest.mark.parametrize("n,L,B,rows", [
    # (elements per row, dtype) of each tensor
    (4, 37, 2, [(8 * 64, torch.bfloat16), (2 * 64, torch.bfloat16), (2 * 64, torch.bfloat16)]),  # Q, K, V
    (3, 129, 1, [(7, torch.int16), (32, torch.bfloat16)]),        # 14-byte rows: 2-byte vectors for both
    (2, 50, 3, [(3, torch.uint8), (5, torch.int32), (1, torch.int16), (16, torch.bfloat16)]),   # four tensors
    (4, 1000, 1, [(1000, torch.bfloat16)]),                      # one tensor, many blocks
])
def test_multi_matches_single_and_oracle(n, L, B, rows):
    """One launch over several tensors moves each exactly as sf_interleave
    does, forward and back, with the vector width all of them allow."""
    say("interleave multi", n, L, B, [r for r, _ in rows])
    g = torch.Generator().manual_seed(11)
    srcs = [torch.randint(-100, 100, (n, B, L, r), generator=g).to(dt) for r, dt in rows]
    outs = sfa.sf_interleave_multi([x.cuda() for x in srcs], n)
    torch.cuda.synchronize()
    for x, y in zip(srcs, outs):
        assert np.array_equal(_bits(y), orc.interleave(_bits(x)))
        assert torch.equal(y, sfa.sf_interleave(x.cuda(), n))
    backs = sfa.sf_interleave_multi(outs, n, inverse=True)
    torch.cuda.synchronize()
    for x, z in zip(srcs, backs):
        assert np.array_equal(_bits(z), _bits(x))


def test_multi_full_size_qkv():
    """The 32k step's Q, K and V in one launch, and K, V back into the
    per-stream layout in another: bitwise equal to one call per tensor."""
    say("interleave multi full size")
    w = I.CROSS_32K
    qs, ks, vs = I.stream_qkv(w.n, w.L, w.batch, w.hq, w.hkv, w.d, seed=5, device="cuda")
    Q, K, V = sfa.sf_interleave_multi([qs, ks, vs], w.n)
    torch.cuda.synchronize()
    assert torch.equal(Q, sfa.sf_interleave(qs, w.n))
    assert torch.equal(K, sfa.sf_interleave(ks, w.n))
    assert torch.equal(V, sfa.sf_interleave(vs, w.n))
    kc, vc = sfa.sf_interleave_multi([K, V], w.n, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(kc, ks) and torch.equal(vc, vs)
