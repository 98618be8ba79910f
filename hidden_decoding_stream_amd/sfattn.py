"""Python binding of libsfattn (ctypes): argument marshalling only.

Every function here has the name of the C entry point it calls (declared in
include/sfattn.h). They take torch tensors that already live on the GPU, pass
their device pointers and torch's current HIP stream, and raise SFError when
the library returns a non-OK status. All computation happens in the library's
HIP kernels; there is no fallback path. If libsfattn.so has not been built,
the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import pathlib

import torch

_PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = pathlib.Path(os.environ.get("SFATTN_LIB", str(_PKG / "libsfattn.so")))

SF_OK, SF_ERR_INVALID, SF_ERR_UNSUPPORTED, SF_ERR_DEVICE = 0, 1, 2, 3
MODES = {"intra": 0, "cross_full": 1, "cross_window": 2}

_lib_handle = None


class SFError(RuntimeError):
    """A non-OK status from libsfattn, with the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libsfattn status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libsfattn.so (once) and declare the C signatures."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m hidden_decoding_stream_amd.build`")
    L = ctypes.CDLL(str(LIB_PATH))
    c = ctypes
    L.sf_abi_version.restype = c.c_int32
    L.sf_abi_version.argtypes = []
    L.sf_last_error.restype = c.c_char_p
    L.sf_last_error.argtypes = []
    L.sf_interleave.restype = c.c_int
    L.sf_interleave.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_int64, c.c_int64, c.c_int64,
                                c.c_int32, c.c_void_p]
    L.sf_interleave_multi.restype = c.c_int
    L.sf_interleave_multi.argtypes = [c.POINTER(c.c_void_p), c.POINTER(c.c_void_p), c.POINTER(c.c_int64),
                                      c.c_int32, c.c_int32, c.c_int64, c.c_int64, c.c_int32, c.c_void_p]
    L.sf_attn_fwd.restype = c.c_int
    L.sf_attn_fwd.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                              c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_int32, c.c_int32,
                              c.c_int32, c.c_int64, c.c_float, c.c_void_p]
    L.sf_expand_embed.restype = c.c_int
    L.sf_expand_embed.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64, c.c_int32, c.c_int64, c.c_int64,
                                  c.c_int64, c.c_void_p]
    L.sf_rope.restype = c.c_int
    L.sf_rope.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int32, c.c_int32, c.c_float, c.c_int64, c.c_void_p]
    L.sf_attn_fwd_last_stream.restype = c.c_int
    L.sf_attn_fwd_last_stream.argtypes = L.sf_attn_fwd.argtypes
    L.sf_attn_bwd_workspace_bytes.restype = c.c_size_t
    L.sf_attn_bwd_workspace_bytes.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_int32, c.c_int32,
                                              c.c_int32, c.c_int64]
    L.sf_attn_bwd.restype = c.c_int
    L.sf_attn_bwd.argtypes = [c.c_void_p] * 9 + [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_int32, c.c_int32,
                                                 c.c_int32, c.c_int64, c.c_float, c.c_void_p, c.c_size_t, c.c_void_p]
    L.sf_attn_decode_workspace_bytes.restype = c.c_size_t
    L.sf_attn_decode_workspace_bytes.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_int32,
                                                 c.c_int32, c.c_int32, c.c_int64, c.c_int32]
    L.sf_attn_decode.restype = c.c_int
    L.sf_attn_decode.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                 c.c_int64, c.c_int32, c.c_int64, c.c_int64, c.c_int32, c.c_int32,
                                 c.c_int32, c.c_int32, c.c_int64, c.c_float, c.c_int32,
                                 c.c_void_p, c.c_size_t, c.c_void_p]
    L.sf_attn_decode_noalloc.restype = c.c_int
    L.sf_attn_decode_noalloc.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                         c.c_int64, c.c_int32, c.c_int64, c.c_int64, c.c_int32, c.c_int32,
                                         c.c_int32, c.c_int32, c.c_int64, c.c_float, c.c_int32, c.c_void_p]
    L.sf_attn_decode_paged_workspace_bytes.restype = c.c_size_t
    L.sf_attn_decode_paged_workspace_bytes.argtypes = L.sf_attn_decode_workspace_bytes.argtypes
    L.sf_attn_decode_paged.restype = c.c_int
    L.sf_attn_decode_paged.argtypes = [c.c_void_p] * 6 + [c.c_int64, c.c_int32, c.c_int64, c.c_int64, c.c_int32,
                                                          c.c_int64, c.c_int32, c.c_int32, c.c_int32, c.c_int32,
                                                          c.c_int64, c.c_float, c.c_int32, c.c_void_p, c.c_size_t,
                                                          c.c_void_p]
    _lib_handle = L
    return L


def _check(status: int) -> None:
    if status != SF_OK:
        raise SFError(status, lib().sf_last_error().decode(errors="replace"))


def _mode(mode) -> int:
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"unknown mode {mode!r}")
        return MODES[mode]
    return int(mode)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _expect(t: torch.Tensor, name: str, shape, device: torch.device) -> None:
    """A caller-supplied tensor must have exactly the shape the call writes or
    reads, on the same device as the call's inputs: the library sees only raw
    pointers, so a short tensor would be read or written out of bounds."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def sf_abi_version() -> int:
    return int(lib().sf_abi_version())


def sf_last_error() -> str:
    return lib().sf_last_error().decode(errors="replace")


def _interleave_shape(src: torch.Tensor, n: int, inverse: bool):
    """(B, L, output shape, row bytes) of an interleave of src."""
    if not inverse:
        if src.dim() < 3 or src.shape[0] != n:
            raise ValueError("forward interleave expects src of shape [n][B][L][...]")
        _, B, L = src.shape[:3]
        out_shape = (B, n * L) + tuple(src.shape[3:])
    else:
        if src.dim() < 2 or src.shape[1] % n:
            raise ValueError("inverse interleave expects src of shape [B][n*L][...]")
        B, S = src.shape[:2]
        L = S // n
        out_shape = (n, B, L) + tuple(src.shape[2:])
    row_bytes = src.element_size() * int(math.prod(out_shape[3:] if inverse else src.shape[3:]))
    return B, L, out_shape, row_bytes


def _interleave_out(src: torch.Tensor, out_shape, out: torch.Tensor | None) -> torch.Tensor:
    if out is None:
        return torch.empty(out_shape, dtype=src.dtype, device=src.device)
    if out.dtype != src.dtype:
        raise ValueError(f"out must be {src.dtype}")
    _expect(out, "out", out_shape, src.device)
    return out


def sf_interleave(src: torch.Tensor, n: int, inverse: bool = False, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Forward: src [n][B][L][...] -> [B][n*L][...]; inverse: [B][n*L][...] -> [n][B][L][...].
    Any dtype; a bit-exact copy."""
    B, L, out_shape, row_bytes = _interleave_shape(src, n, inverse)
    out = _interleave_out(src, out_shape, out)
    _check(lib().sf_interleave(_dev(src, "src"), _dev(out, "out"), n, L, B, row_bytes, int(inverse),
                               _stream(stream)))
    return out


def sf_interleave_multi(srcs, n: int, inverse: bool = False, outs=None, stream=None) -> list:
    """sf_interleave of 1 to 4 tensors with the same n, B and L (rows may
    differ in size and dtype) in one launch; returns the outputs in order."""
    srcs = list(srcs)
    if not 1 <= len(srcs) <= 4:
        raise ValueError("sf_interleave_multi takes 1 to 4 tensors")
    outs = [None] * len(srcs) if outs is None else list(outs)
    if len(outs) != len(srcs):
        raise ValueError("outs must match srcs")
    shapes = [_interleave_shape(x, n, inverse) for x in srcs]
    if len({(B, L) for B, L, _, _ in shapes}) != 1:
        raise ValueError("all tensors must share batch and L")
    B, L = shapes[0][:2]
    outs = [_interleave_out(x, sh[2], o) for x, sh, o in zip(srcs, shapes, outs)]
    cnt = len(srcs)
    src_p = (ctypes.c_void_p * cnt)(*[_dev(x, "src") for x in srcs])
    dst_p = (ctypes.c_void_p * cnt)(*[_dev(o, "out") for o in outs])
    rows = (ctypes.c_int64 * cnt)(*[sh[3] for sh in shapes])
    _check(lib().sf_interleave_multi(src_p, dst_p, rows, cnt, n, L, B, int(inverse), _stream(stream)))
    return outs


def sf_expand_embed(ids: torch.Tensor, tables: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Gather and interleave: ids int32 [B][L], tables [n][vocab][...] (any
    dtype) -> out [B][n*L][...] with out[b][i*n+k] = tables[k][ids[b][i]]
    (zeros for an id outside the vocabulary)."""
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise ValueError("ids must be an int32 [B][L] tensor")
    B, L = ids.shape
    n, vocab = tables.shape[:2]
    row = tables[0, 0].numel() * tables.element_size()
    if out is None:
        out = torch.empty((B, n * L) + tuple(tables.shape[2:]), dtype=tables.dtype, device=tables.device)
    if ids.device != tables.device:
        raise ValueError("ids and tables must be on the same device")
    if out.dtype != tables.dtype:
        raise ValueError(f"out must be {tables.dtype}")
    _expect(out, "out", (B, n * L) + tuple(tables.shape[2:]), tables.device)
    _check(lib().sf_expand_embed(_dev(ids, "ids"), _dev(tables, "tables"), _dev(out, "out"), B, n, L, vocab, row,
                                 _stream(stream)))
    return out


def sf_rope(x: torch.Tensor, base: float = 10000.0, pos0: int = 0, stream=None) -> torch.Tensor:
    """Rotary encoding in place at continuous positions pos0 + s: x bf16
    [B][S][heads][d]. Returns x."""
    B, S, H, d = x.shape
    _check(lib().sf_rope(_dev(x, "x", torch.bfloat16), B, S, H, d, float(base), int(pos0), _stream(stream)))
    return x


def sf_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode, n: int, window: int = 0,
                scale: float | None = None, out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = None,
                stream=None):
    """Prefill attention. q [B][n*L][hq][d], k/v [B][n*L][hkv][d], bf16.
    Returns out, or (out, lse) when lse is True or a float32 [B][hq][n*L] tensor."""
    B, S, hq, d = q.shape
    hkv = k.shape[2]
    if S % n:
        raise ValueError("sequence length must be a multiple of n")
    if k.shape != (B, S, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B][S][hkv][d] matching q")
    _expect(k, "k", (B, S, hkv, d), q.device)
    _expect(v, "v", (B, S, hkv, d), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = torch.empty((B, hq, S), dtype=torch.float32, device=q.device)
    if want_lse:
        _expect(lse, "lse", (B, hq, S), q.device)
    lse_ptr = _dev(lse, "lse", torch.float32) if want_lse else None
    bf = torch.bfloat16
    _check(lib().sf_attn_fwd(_dev(q, "q", bf), _dev(k, "k", bf), _dev(v, "v", bf), _dev(out, "out", bf),
                             lse_ptr, B, n, S // n, hq, hkv, d, _mode(mode), int(window), float(scale),
                             _stream(stream)))
    return (out, lse) if want_lse else out


def sf_attn_fwd_last_stream(q_last: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode, n: int,
                            window: int = 0, scale: float | None = None, out: torch.Tensor | None = None,
                            lse: torch.Tensor | bool | None = None, stream=None):
    """Attention of the last stream's queries only. q_last [B][L][hq][d] (row i
    = stream n-1 of token i), k/v [B][n*L][hkv][d], bf16. Returns out
    [B][L][hq][d], or (out, lse) when lse is True or a float32 [B][hq][L] tensor."""
    B, L, hq, d = q_last.shape
    hkv = k.shape[2]
    if k.shape != (B, n * L, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B][n*L][hkv][d] matching q_last")
    _expect(k, "k", (B, n * L, hkv, d), q_last.device)
    _expect(v, "v", (B, n * L, hkv, d), q_last.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q_last)
    _expect(out, "out", q_last.shape, q_last.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = torch.empty((B, hq, L), dtype=torch.float32, device=q_last.device)
    if want_lse:
        _expect(lse, "lse", (B, hq, L), q_last.device)
    lse_ptr = _dev(lse, "lse", torch.float32) if want_lse else None
    bf = torch.bfloat16
    _check(lib().sf_attn_fwd_last_stream(_dev(q_last, "q_last", bf), _dev(k, "k", bf), _dev(v, "v", bf),
                                         _dev(out, "out", bf), lse_ptr, B, n, L, hq, hkv, d, _mode(mode),
                                         int(window), float(scale), _stream(stream)))
    return (out, lse) if want_lse else out


def sf_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
                lse: torch.Tensor, mode, n: int, window: int = 0, scale: float | None = None,
                out=None, workspace: torch.Tensor | None = None, stream=None):
    """Gradients (dq, dk, dv) of sf_attn_fwd for the loss sum(dout * o).
    q, o, dout [B][n*L][hq][d]; k, v [B][n*L][hkv][d]; bf16; lse float32
    [B][hq][n*L] as returned by sf_attn_fwd(..., lse=True)."""
    B, S, hq, d = q.shape
    hkv = k.shape[2]
    if S % n:
        raise ValueError("sequence length must be a multiple of n")
    dev = q.device
    for t, name in ((k, "k"), (v, "v")):
        _expect(t, name, (B, S, hkv, d), dev)
    for t, name in ((o, "o"), (dout, "dout")):
        _expect(t, name, (B, S, hq, d), dev)
    _expect(lse, "lse", (B, hq, S), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    _expect(dq, "dq", (B, S, hq, d), dev)
    _expect(dk, "dk", (B, S, hkv, d), dev)
    _expect(dv, "dv", (B, S, hkv, d), dev)
    need = int(lib().sf_attn_bwd_workspace_bytes(B, n, S // n, hq, hkv, d, _mode(mode), int(window)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev:
        raise ValueError(f"workspace must be on {dev}")
    bf = torch.bfloat16
    _check(lib().sf_attn_bwd(_dev(q, "q", bf), _dev(k, "k", bf), _dev(v, "v", bf), _dev(o, "o", bf),
                             _dev(dout, "dout", bf), _dev(lse, "lse", torch.float32), _dev(dq, "dq", bf),
                             _dev(dk, "dk", bf), _dev(dv, "dv", bf), B, n, S // n, hq, hkv, d, _mode(mode),
                             int(window), float(scale), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def sf_attn_decode_workspace_bytes(batch: int, n: int, T: int, hq: int, hkv: int, d: int, mode,
                                   window: int = 0, num_splits: int = 0) -> int:
    return int(lib().sf_attn_decode_workspace_bytes(batch, n, T, hq, hkv, d, _mode(mode), int(window),
                                                    int(num_splits)))


def sf_attn_decode(q_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, T: int, mode,
                   window: int = 0, scale: float | None = None, num_splits: int = 0,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Decode the n stream queries of token T-1. q_new [B][n][hq][d];
    caches [B][n][T_max][hkv][d]; bf16. The workspace is allocated with torch
    when not given."""
    B, n, hq, d = q_new.shape
    T_max, hkv = k_cache.shape[2], k_cache.shape[3]
    if k_cache.shape != (B, n, T_max, hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B][n][T_max][hkv][d] matching q_new")
    dev = q_new.device
    _expect(k_cache, "k_cache", (B, n, T_max, hkv, d), dev)
    _expect(v_cache, "v_cache", (B, n, T_max, hkv, d), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q_new)
    _expect(out, "out", q_new.shape, dev)
    need = sf_attn_decode_workspace_bytes(B, n, T, hq, hkv, d, mode, window, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev:
        raise ValueError(f"workspace must be on {dev}")
    bf = torch.bfloat16
    _check(lib().sf_attn_decode(_dev(q_new, "q_new", bf), _dev(k_cache, "k_cache", bf),
                                _dev(v_cache, "v_cache", bf), _dev(out, "out", bf), B, n, int(T), T_max,
                                hq, hkv, d, _mode(mode), int(window), float(scale), int(num_splits),
                                _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream)))
    return out


def sf_attn_decode_noalloc(q_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, T: int, mode,
                           window: int = 0, scale: float | None = None, num_splits: int = 0,
                           out: torch.Tensor | None = None, stream=None):
    """sf_attn_decode with the library's fixed per-GPU scratch instead of a
    workspace: it allocates nothing when `out` is given. Calls that overlap in
    time on one GPU race on that scratch."""
    B, n, hq, d = q_new.shape
    T_max, hkv = k_cache.shape[2], k_cache.shape[3]
    if k_cache.shape != (B, n, T_max, hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B][n][T_max][hkv][d] matching q_new")
    dev = q_new.device
    _expect(k_cache, "k_cache", (B, n, T_max, hkv, d), dev)
    _expect(v_cache, "v_cache", (B, n, T_max, hkv, d), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q_new)
    _expect(out, "out", q_new.shape, dev)
    bf = torch.bfloat16
    _check(lib().sf_attn_decode_noalloc(_dev(q_new, "q_new", bf), _dev(k_cache, "k_cache", bf),
                                        _dev(v_cache, "v_cache", bf), _dev(out, "out", bf), B, n, int(T), T_max,
                                        hq, hkv, d, _mode(mode), int(window), float(scale), int(num_splits),
                                        _stream(stream)))
    return out


def sf_attn_decode_paged_workspace_bytes(batch: int, n: int, max_T: int, hq: int, hkv: int, d: int, mode,
                                         window: int = 0, num_splits: int = 0) -> int:
    return int(lib().sf_attn_decode_paged_workspace_bytes(batch, n, int(max_T), hq, hkv, d, _mode(mode),
                                                          int(window), int(num_splits)))


def sf_attn_decode_paged(q_new: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, mode, max_T: int | None = None,
                         window: int = 0, scale: float | None = None, num_splits: int = 0,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Decode each sequence's n stream queries of its newest token against a
    paged per-stream cache. q_new [B][n][hq][d]; page pools
    [num_pages][page][hkv][d] bf16; block_table int32 [B][n][max_pages];
    seq_lens int32 [B] on the device. max_T bounds seq_lens (default: what
    the block table can hold). The workspace is allocated with torch when not
    given."""
    B, n, hq, d = q_new.shape
    num_pages, page, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if k_pages.shape != (num_pages, page, hkv, d) or v_pages.shape != k_pages.shape:
        raise ValueError("page pools must be [num_pages][page][hkv][d] matching q_new")
    if block_table.dim() != 3 or block_table.shape[:2] != (B, n):
        raise ValueError("block_table must be [B][n][max_pages]")
    if seq_lens.shape != (B,):
        raise ValueError("seq_lens must be [B]")
    max_pages = block_table.shape[2]
    dev = q_new.device
    for t, name in ((k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                    (seq_lens, "seq_lens")):
        if t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
    if max_T is None:
        max_T = max_pages * page
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q_new)
    _expect(out, "out", q_new.shape, dev)
    need = sf_attn_decode_paged_workspace_bytes(B, n, max_T, hq, hkv, d, mode, window, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev:
        raise ValueError(f"workspace must be on {dev}")
    bf, i32 = torch.bfloat16, torch.int32
    _check(lib().sf_attn_decode_paged(
        _dev(q_new, "q_new", bf), _dev(k_pages, "k_pages", bf), _dev(v_pages, "v_pages", bf),
        _dev(block_table, "block_table", i32), _dev(seq_lens, "seq_lens", i32), _dev(out, "out", bf),
        B, n, int(max_T), num_pages, page, max_pages, hq, hkv, d, _mode(mode), int(window), float(scale),
        int(num_splits), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out
