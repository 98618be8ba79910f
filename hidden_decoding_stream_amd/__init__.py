"""Stream-factorized attention (Hidden Decoding) for AMD Instinct MI355X.

The compute lives in libsfattn.so (HIP kernels for gfx950, C ABI in
include/sfattn.h); this package is its thin Python binding. Build the library
with ``python -m hidden_decoding_stream_amd.build``.
"""
from .sfattn import (  # noqa: F401
    MODES,
    SFError,
    lib,
    sf_abi_version,
    sf_attn_bwd,
    sf_attn_decode,
    sf_attn_decode_noalloc,
    sf_attn_decode_paged,
    sf_attn_decode_paged_workspace_bytes,
    sf_attn_decode_workspace_bytes,
    sf_attn_fwd,
    sf_attn_fwd_last_stream,
    sf_expand_embed,
    sf_interleave,
    sf_interleave_multi,
    sf_last_error,
    sf_rope,
)
