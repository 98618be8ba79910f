"""The Python binding rejects caller-supplied tensors whose shape or device
does not match the call before anything reaches the library.

The C ABI sees raw pointers only, so a short output, LSE, gradient or cache
tensor would become an out-of-bounds device access. These checks run before
any pointer is taken, so CPU tensors exercise them without a GPU; with every
shape right the binding then refuses CPU tensors, which shows the shape check
came first.
"""
import pytest
import torch

import hidden_decoding_stream_amd as sfa

bf = torch.bfloat16
B, n, L, hq, hkv, d = 1, 4, 16, 8, 2, 64
S = n * L


def qkv():
    return (torch.zeros(B, S, hq, d, dtype=bf), torch.zeros(B, S, hkv, d, dtype=bf),
            torch.zeros(B, S, hkv, d, dtype=bf))


def test_fwd_short_out_and_lse():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out must have shape"):
        sfa.sf_attn_fwd(q, k, v, "cross_full", n, out=torch.zeros(B, S - 1, hq, d, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        sfa.sf_attn_fwd(q, k, v, "cross_full", n, lse=torch.zeros(B, hq, S - 4))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        sfa.sf_attn_fwd(q, k, v, "cross_full", n, out=torch.zeros_like(q), lse=torch.zeros(B, hq, S))


def test_fwd_last_stream_short_out_and_lse():
    _, k, v = qkv()
    ql = torch.zeros(B, L, hq, d, dtype=bf)
    with pytest.raises(ValueError, match="out must have shape"):
        sfa.sf_attn_fwd_last_stream(ql, k, v, "cross_full", n, out=torch.zeros(B, L, hq, d - 8, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        sfa.sf_attn_fwd_last_stream(ql, k, v, "cross_full", n, lse=torch.zeros(B, hq, S))


@pytest.mark.parametrize("which", ["v", "o", "dout", "lse", "dq", "dk", "dv"])
def test_bwd_every_tensor_checked(which):
    q, k, v = qkv()
    args = dict(q=q, k=k, v=v, o=torch.zeros_like(q), dout=torch.zeros_like(q), lse=torch.zeros(B, hq, S))
    grads = [torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)]
    if which in args:
        t = args[which]
        args[which] = t[..., :-1] if t.dim() == 4 else t[:, :, :-1]
    else:
        i = ("dq", "dk", "dv").index(which)
        grads[i] = grads[i][:, :-1]
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        sfa.sf_attn_bwd(args["q"], args["k"], args["v"], args["o"], args["dout"], args["lse"], "cross_full", n,
                        out=tuple(grads))


def test_decode_short_out():
    q = torch.zeros(B, n, hq, d, dtype=bf)
    kc = torch.zeros(B, n, L, hkv, d, dtype=bf)
    with pytest.raises(ValueError, match="out must have shape"):
        sfa.sf_attn_decode(q, kc, kc.clone(), L, "cross_full", out=torch.zeros(B, n - 1, hq, d, dtype=bf))
    with pytest.raises(ValueError, match="caches must be"):
        sfa.sf_attn_decode(q, kc, kc[:, :, :-1].contiguous(), L, "cross_full")


def test_decode_paged_short_out():
    q = torch.zeros(B, n, hq, d, dtype=bf)
    pages = torch.zeros(4, 32, hkv, d, dtype=bf)
    table = torch.zeros(B, n, 1, dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        sfa.sf_attn_decode_paged(q, pages, pages.clone(), table, lens, "cross_full",
                                 out=torch.zeros(B, n, hq, d // 2, dtype=bf))


def test_interleave_and_expand_out():
    src = torch.zeros(n, B, L, 3)
    with pytest.raises(ValueError, match="out must have shape"):
        sfa.sf_interleave(src, n, out=torch.zeros(B, S - 1, 3))
    ids = torch.zeros(B, L, dtype=torch.int32)
    tables = torch.zeros(n, 10, 6, dtype=bf)
    with pytest.raises(ValueError, match="out must have shape"):
        sfa.sf_expand_embed(ids, tables, out=torch.zeros(B, S, 5, dtype=bf))
