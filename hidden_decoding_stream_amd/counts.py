"""Algorithmic work of stream-factorized attention, in closed form.

Useful work counts only the (query, key) pairs the mask admits: the n^2 growth
of dense attention over the expanded sequence is what the factorised masks
avoid (page "微信WeLM提出Hidden Decoding：大模型推理新范式", section
规模化落地的工程优化: dense attention grows 16x at n=4, the factorised form adds
about n times). Each admitted pair costs 2*d flops for q.k and 2*d for p*v.
"""
from __future__ import annotations


def prefill_pairs(mode: str, n: int, L: int, window: int = 0) -> int:
    """Admitted (query, key) pairs of one head over S = n*L positions."""
    S = n * L
    if mode == "intra":
        return n * L * (L + 1) // 2          # n causal problems of length L
    if mode == "cross_full" or window >= S:
        return S * (S + 1) // 2              # causal over S
    if mode == "cross_window":
        return window * (window + 1) // 2 + (S - window) * window
    raise ValueError(mode)


def prefill_flops(mode: str, n: int, L: int, batch: int, hq: int, d: int, window: int = 0) -> int:
    return 4 * d * prefill_pairs(mode, n, L, window) * batch * hq


def last_stream_pairs(mode: str, n: int, L: int, window: int = 0) -> int:
    """Admitted pairs of one head when only stream n-1 queries: token i's
    query sits at position i*n + n-1 and sees that many + 1 positions
    (cross), at most `window` of them (cross_window), or i + 1 keys of its
    own stream (intra)."""
    if mode == "intra":
        return L * (L + 1) // 2
    if mode == "cross_full" or window >= n * L:
        return n * L * (L + 1) // 2
    if mode == "cross_window":
        return sum(min(i * n + n, window) for i in range(L))
    raise ValueError(mode)


def last_stream_flops(mode: str, n: int, L: int, batch: int, hq: int, d: int, window: int = 0) -> int:
    return 4 * d * last_stream_pairs(mode, n, L, window) * batch * hq


def decode_pairs(mode: str, n: int, T: int, window: int = 0) -> int:
    """Admitted pairs of the n queries of token T-1 for one head."""
    total = 0
    for k in range(n):
        p = (T - 1) * n + k
        if mode == "intra":
            total += T
        else:
            seen = p + 1
            if mode == "cross_window":
                seen = min(seen, window)
            total += seen
    return total


def decode_flops(mode: str, n: int, T: int, batch: int, hq: int, d: int, window: int = 0) -> int:
    return 4 * d * decode_pairs(mode, n, T, window) * batch * hq


def decode_bytes(mode: str, n: int, T: int, batch: int, hq: int, hkv: int, d: int, window: int = 0,
                 elem: int = 2) -> int:
    """HBM bytes a decode step must move: every cache row (K and V) that some
    query admits, plus the queries and the outputs."""
    if mode == "cross_window" and window < n * T:
        oldest = (T - 1) * n - window + 1          # oldest position any query sees
        rows = n * T - max(0, oldest)
    else:
        rows = n * T
    kv = 2 * rows * hkv * d * elem
    qo = 2 * n * hq * d * elem
    return batch * (kv + qo)


def interleave_bytes(tensor_bytes: int) -> int:
    """A copy reads and writes every byte once."""
    return 2 * tensor_bytes


def expand_embed_bytes(batch: int, n: int, L: int, row_bytes: int) -> int:
    """Every output row is read once from its table and written once, plus
    the token ids."""
    return 2 * batch * n * L * row_bytes + 4 * batch * L


def rope_bytes(tensor_bytes: int) -> int:
    """In place: the tensor is read and written once."""
    return 2 * tensor_bytes


def backward_flops(mode: str, n: int, L: int, batch: int, hq: int, d: int, window: int = 0) -> int:
    """Useful work of the backward: dV = P^T dO, dP = dO V^T, dQ = dS K and
    dK = dS^T Q, plus recomputing S = Q K^T: five products of 2*d flops per
    admitted pair, 2.5 times the forward's."""
    return 10 * d * prefill_pairs(mode, n, L, window) * batch * hq
