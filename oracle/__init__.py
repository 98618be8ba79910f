"""CPU oracle for stream-factorized attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct statement of what the GPU
path computes, in float64 NumPy. It exists to check the HIP library. Only the
test suite (``tests/``), the smoke check in ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run it. The product package
``hidden_decoding_stream_amd`` never imports it, and the oracle imports nothing
from the product (it shares no kernels, headers, helpers or tables with it).

Sources. The method is described on these pages; citations name the page and
the section (or numbered step) on it:

* [HD-tahou] "微信WeLM提出Hidden Decoding：大模型推理新范式",
  www.tahou.com/article/212669152970878981. Sections: 隐式序列缩放的技术细节
  (three numbered steps), 规模化落地的工程优化 (stream-factorized attention and
  KV-mirror), 实验效果与成本分析 (cost and decode regimes), 中间流的作用验证
  (ablations and probes).
* [HD-aiflow] aiflownews.com/?p=965, sections "Latent computation scaling and
  Hidden Decoding" and "Tencent's ecosystem first scaling strategy" (GQA).

Every function is pinned by tests in ``tests/test_oracle.py`` against things
other than itself (brute force, library routines, closed forms, the pages'
printed ratios); no function here is "parity unpinned".
"""
from .sfa import (  # noqa: F401
    MODES,
    interleave,
    deinterleave,
    mask,
    attend,
    attn_fwd,
    decode,
    pair_count,
)
