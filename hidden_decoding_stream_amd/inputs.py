"""Seeded synthetic inputs for stream-factorized attention (SFA) workloads.

This module only draws random numbers and names workload sizes. It holds none
of the method's arithmetic (no index maps, masks or softmax), so the GPU path
and the CPU oracle can both take their inputs from it without sharing any
computation.

Recipe:
  * a ``torch.Generator`` seeded with ``seed``, on the CPU by default (the
    same values on every machine) or on the GPU for the large workloads
    (``device="cuda"``: much faster to draw; the oracle then consumes exact
    copies of the GPU tensors, so parity does not depend on the stream);
  * tensors are drawn in a fixed order (Q, K, V for prefill; q_new, K cache,
    V cache for decode), each as float32 N(0, 1);
  * attention inputs are then rounded to bfloat16 (round-to-nearest-even).
    The oracle consumes exactly these rounded values, upcast to float64, so
    input quantisation is never counted as kernel error.

The workloads follow the pages' setting: n = 4 streams per token (the "HD4"
models, page "微信WeLM提出Hidden Decoding：大模型推理新范式", section
实验效果与成本分析), a 32k expanded training sequence (same page, section
规模化落地的工程优化, the KV-mirror paragraph) and grouped-query attention
(aiflownews.com page, section "Tencent's ecosystem first scaling strategy").
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes only.

    n: streams per token; L: tokens; batch: sequences; hq/hkv: query / key-value
    heads; d: head dimension; mode: "intra" | "cross_full" | "cross_window";
    window: positions a cross_window query may look back (self included).
    """
    name: str
    n: int
    L: int
    batch: int
    hq: int
    hkv: int
    d: int
    mode: str
    window: int = 0
    seed: int = 0
    dtype: str = "bf16"

    @property
    def S(self) -> int:
        return self.n * self.L

    @property
    def scale(self) -> float:
        # 1/sqrt(d) as the float32 value the kernel receives.
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """A decode step: the n stream queries of token T-1 against a per-stream
    cache holding tokens 0..T-1 (T_max >= T slots per stream)."""
    name: str
    n: int
    T: int
    T_max: int
    batch: int
    hq: int
    hkv: int
    d: int
    mode: str
    window: int = 0
    seed: int = 0

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))


# Seeds are 1000 + the workload's index in the list of five workloads
# (tiny, intra 16k, window 16k, 32k, decode).
TINY_INTRA = Workload("tiny_intra", 4, 64, 1, 4, 4, 64, "intra", seed=1000, dtype="fp32")
TINY_CROSS = Workload("tiny_cross_full", 4, 64, 1, 4, 4, 64, "cross_full", seed=1000, dtype="fp32")
INTRA_16K = Workload("intra_16k", 4, 4096, 2, 32, 8, 128, "intra", seed=1001)
WINDOW_16K = Workload("cross_window_16k", 4, 4096, 2, 32, 8, 128, "cross_window", window=4096, seed=1002)
CROSS_32K = Workload("cross_full_32k", 4, 8192, 1, 32, 8, 128, "cross_full", seed=1003)
INTRA_32K = Workload("intra_32k", 4, 8192, 1, 32, 8, 128, "intra", seed=1003)

PREFILL_WORKLOADS = (TINY_INTRA, TINY_CROSS, INTRA_16K, WINDOW_16K, CROSS_32K, INTRA_32K)


def decode_workload(batch: int, mode: str, T: int = 8192, T_max: int | None = None,
                    window: int = 0) -> DecodeWorkload:
    """The decode workload: 8192 tokens x 4 streams, 32/8 heads, d=128."""
    return DecodeWorkload(f"decode_{mode}_b{batch}", 4, T, T if T_max is None else T_max,
                          batch, 32, 8, 128, mode, window=window, seed=1004)


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, gen: torch.Generator) -> torch.Tensor:
    """float32 N(0,1) on the generator's device."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round float32 to bfloat16 (torch's CPU cast rounds to nearest even)."""
    return x.to(torch.bfloat16)


def stream_qkv(n: int, L: int, batch: int, hq: int, hkv: int, d: int, seed: int,
               dtype: str = "bf16", device="cpu"):
    """Per-stream Q, K, V as produced by the n stream embeddings: layout
    [n][batch][L][heads][d], drawn Q then K then V."""
    g = _gen(seed, device)
    q = normal((n, batch, L, hq, d), g)
    k = normal((n, batch, L, hkv, d), g)
    v = normal((n, batch, L, hkv, d), g)
    if dtype == "bf16":
        q, k, v = to_bf16(q), to_bf16(k), to_bf16(v)
    return q, k, v


def expanded_qkv(S: int, batch: int, hq: int, hkv: int, d: int, seed: int, device="cpu"):
    """Q, K, V already in the expanded layout [batch][S][heads][d] (bf16),
    drawn Q then K then V. Used where the interleave is not under test."""
    g = _gen(seed, device)
    q = to_bf16(normal((batch, S, hq, d), g))
    k = to_bf16(normal((batch, S, hkv, d), g))
    v = to_bf16(normal((batch, S, hkv, d), g))
    return q, k, v


def workload_qkv(w: Workload, device="cpu"):
    """Expanded-layout bf16 Q, K, V for a prefill workload."""
    return expanded_qkv(w.S, w.batch, w.hq, w.hkv, w.d, w.seed, device)


def decode_inputs(w: DecodeWorkload, device="cpu"):
    """q_new [batch][n][hq][d] and the per-stream caches [batch][n][T_max][hkv][d]
    (bf16), drawn q_new, then K cache, then V cache. Slots t >= T hold random
    values too; a correct decode never reads them."""
    g = _gen(w.seed, device)
    q = to_bf16(normal((w.batch, w.n, w.hq, w.d), g))
    kc = to_bf16(normal((w.batch, w.n, w.T_max, w.hkv, w.d), g))
    vc = to_bf16(normal((w.batch, w.n, w.T_max, w.hkv, w.d), g))
    return q, kc, vc


def uniform_keys(shape, value: float = 0.0) -> torch.Tensor:
    """Constant keys: every score in a row is equal, so the softmax is uniform
    over whatever keys the mask admits (used to probe masks exactly)."""
    return torch.full(shape, value, dtype=torch.bfloat16)


@dataclasses.dataclass(frozen=True)
class PagedDecodeWorkload:
    """Decode of a batch of sequences of different lengths (lens[b] tokens in
    sequence b's per-stream caches) whose caches are spread over pages of
    `page` tokens."""
    name: str
    n: int
    lens: tuple
    page: int
    hq: int
    hkv: int
    d: int
    mode: str
    window: int = 0
    seed: int = 0
    spare_pages: int = 3

    @property
    def batch(self) -> int:
        return len(self.lens)

    @property
    def max_pages(self) -> int:
        return max(1, max(-(-t // self.page) for t in self.lens))

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))


def paged_decode_inputs(w: PagedDecodeWorkload, device="cpu"):
    """q_new [batch][n][hq][d], page pools k_pages, v_pages
    [num_pages][page][hkv][d] (bf16), block_table int32 [batch][n][max_pages]
    and seq_lens int32 [batch]. Each (sequence, stream) gets its own pages
    for its tokens, at places drawn by a random permutation of the pool;
    table entries past a sequence's last page are -1 (never read). Drawn in
    that order: q_new, K pages, V pages, the permutation."""
    g = _gen(w.seed, device)
    used = [-(-t // w.page) for t in w.lens]
    need = sum(u * w.n for u in used)
    num_pages = need + w.spare_pages
    q = to_bf16(normal((w.batch, w.n, w.hq, w.d), g))
    kp = to_bf16(normal((num_pages, w.page, w.hkv, w.d), g))
    vp = to_bf16(normal((num_pages, w.page, w.hkv, w.d), g))
    perm = torch.randperm(num_pages, generator=g, device=device).to(torch.int32)
    table = torch.full((w.batch, w.n, w.max_pages), -1, dtype=torch.int32, device=device)
    i = 0
    for b, u in enumerate(used):
        for k in range(w.n):
            table[b, k, :u] = perm[i:i + u]
            i += u
    lens = torch.tensor(w.lens, dtype=torch.int32, device=device)
    return q, kp, vp, table, lens
