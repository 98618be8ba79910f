"""The closed-form work counts used by the benchmark, against the oracle's
mask popcounts (no GPU)."""
import numpy as np
import pytest

import hidden_decoding_stream_amd.counts as C
import oracle.sfa as orc


@pytest.mark.parametrize("n,L", [(1, 7), (2, 16), (4, 33), (3, 50)])
@pytest.mark.parametrize("mode,W", [("intra", 0), ("cross_full", 0), ("cross_window", 1), ("cross_window", 9),
                                    ("cross_window", 64), ("cross_window", 10 ** 6)])
def test_prefill_pairs(n, L, mode, W):
    assert C.prefill_pairs(mode, n, L, W) == orc.pair_count(mode, n, L, W or None)


@pytest.mark.parametrize("n,T", [(1, 5), (4, 9), (3, 20)])
@pytest.mark.parametrize("mode,W", [("intra", 0), ("cross_full", 0), ("cross_window", 1), ("cross_window", 7),
                                    ("cross_window", 1000)])
def test_decode_pairs(n, T, mode, W):
    rows = (T - 1) * n + np.arange(n)
    want = int(orc.mask(mode, n, T, W or None, rows).sum())
    assert C.decode_pairs(mode, n, T, W) == want


@pytest.mark.parametrize("n,T,W", [(4, 9, 5), (4, 9, 1), (4, 9, 36), (4, 9, 100), (2, 30, 17)])
def test_decode_bytes_window_rows(n, T, W):
    """Cache rows admitted by at least one of the n queries."""
    rows = (T - 1) * n + np.arange(n)
    used = int(orc.mask("cross_window", n, T, W, rows).any(axis=0).sum())
    per_row = 2 * 1 * 1 * 2   # K and V, hkv=1, d=1, 2 bytes
    qo = 2 * n * 1 * 1 * 2
    assert C.decode_bytes("cross_window", n, T, 1, 1, 1, 1, W) == used * per_row + qo


def test_headline_numbers():
    # 32k cross_full prefill: n=4, L=8192, B=1, 32 query heads, d=128
    assert C.prefill_pairs("cross_full", 4, 8192) == 536_887_296
    assert C.prefill_flops("cross_full", 4, 8192, 1, 32, 128) == 8_796_361_457_664
    assert C.prefill_pairs("intra", 4, 8192) == 134_234_112
    # decode cache: 2 * n * T * hkv * d * 2 bytes per batch element
    assert C.decode_bytes("cross_full", 4, 8192, 1, 32, 8, 128) == 134_217_728 + 2 * 4 * 32 * 128 * 2


@pytest.mark.parametrize("mode,W", [("intra", None), ("cross_full", None), ("cross_window", 7), ("cross_window", 1),
                                    ("cross_window", 400)])
@pytest.mark.parametrize("n,L", [(4, 9), (3, 17), (1, 12)])
def test_last_stream_pairs_match_oracle_mask(mode, W, n, L):
    rows = np.arange(L) * n + (n - 1)
    want = int(orc.mask(mode, n, L, W, rows).sum())
    assert C.last_stream_pairs(mode, n, L, W or 0) == want


def test_front_end_bytes():
    # n=4 tables, L=8192 tokens, 8 KiB rows: read + write of 32768 rows, plus the ids
    assert C.expand_embed_bytes(1, 4, 8192, 8192) == 2 * 32768 * 8192 + 4 * 8192
    assert C.rope_bytes(1 << 28) == 1 << 29


def test_backward_flops_is_two_and_a_half_forwards():
    for mode, W in (("intra", 0), ("cross_full", 0), ("cross_window", 4096)):
        assert 2 * C.backward_flops(mode, 4, 4096, 2, 32, 128, W) == 5 * C.prefill_flops(mode, 4, 4096, 2, 32, 128, W)
