"""libsfattn loads, exports what include/sfattn.h declares, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import pathlib
import re

import pytest

import hidden_decoding_stream_amd as sfa
from hidden_decoding_stream_amd import sfattn as B

HEADER = pathlib.Path(__file__).resolve().parent.parent / "include" / "sfattn.h"

# conftest.py builds the library when it is missing; if it is still absent the
# boundary tests fail here rather than turning into skips.
assert B.LIB_PATH.exists(), f"{B.LIB_PATH} is missing and could not be built"
L = sfa.lib()
# fake, 16-byte aligned, never dereferenced device addresses
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x40000000)
P3 = ctypes.c_void_p(0x80000000)
P4 = ctypes.c_void_p(0xC0000000)


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sf_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"sf_interleave", "sf_interleave_multi", "sf_expand_embed", "sf_rope", "sf_attn_fwd", "sf_attn_fwd_last_stream",
            "sf_attn_bwd", "sf_attn_bwd_workspace_bytes", "sf_attn_decode", "sf_attn_decode_workspace_bytes",
            "sf_attn_decode_paged", "sf_attn_decode_paged_workspace_bytes",
            "sf_abi_version", "sf_last_error"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_abi_version():
    assert sfa.sf_abi_version() == 1


def fwd(q=P, k=P2, v=P3, o=P4, lse=None, batch=1, n=4, Lt=64, hq=4, hkv=4, d=64, mode=1, window=0,
        scale=0.125, last=False):
    f = L.sf_attn_fwd_last_stream if last else L.sf_attn_fwd
    return f(q, k, v, o, lse, batch, n, Lt, hq, hkv, d, mode, window, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), B.SF_ERR_INVALID),
    (dict(batch=-1), B.SF_ERR_INVALID),
    (dict(Lt=-3), B.SF_ERR_INVALID),
    (dict(hq=0), B.SF_ERR_INVALID),
    (dict(hq=6, hkv=4), B.SF_ERR_INVALID),
    (dict(mode=7), B.SF_ERR_INVALID),
    (dict(mode=2, window=0), B.SF_ERR_INVALID),
    (dict(scale=float("nan")), B.SF_ERR_INVALID),
    (dict(scale=float("inf")), B.SF_ERR_INVALID),
    (dict(scale=-1.0), B.SF_ERR_UNSUPPORTED),
    (dict(d=96), B.SF_ERR_UNSUPPORTED),
    (dict(d=256), B.SF_ERR_UNSUPPORTED),
    (dict(q=None), B.SF_ERR_INVALID),
    (dict(o=None), B.SF_ERR_INVALID),
    (dict(q=ctypes.c_void_p(0x10008)), B.SF_ERR_UNSUPPORTED),
    (dict(lse=ctypes.c_void_p(0x20002)), B.SF_ERR_UNSUPPORTED),
    (dict(o=P), B.SF_ERR_INVALID),                       # o aliases q
    (dict(batch=1 << 20, Lt=1 << 20), B.SF_ERR_UNSUPPORTED),  # beyond 2^30 elements
    (dict(batch=1 << 40, Lt=1 << 40), B.SF_ERR_INVALID),      # int64 overflow
    (dict(n=1 << 10, Lt=1 << 14), B.SF_ERR_UNSUPPORTED),      # k beyond 2^30 elements
])
@pytest.mark.parametrize("last", [False, True], ids=["fwd", "last_stream"])
def test_fwd_rejects(kw, status, last):
    assert fwd(**kw, last=last) == status
    assert sfa.sf_last_error() != ""


@pytest.mark.parametrize("kw", [dict(batch=0), dict(Lt=0), dict(batch=0, q=None, k=None, v=None, o=None)])
@pytest.mark.parametrize("last", [False, True], ids=["fwd", "last_stream"])
def test_fwd_empty_is_noop(kw, last):
    assert fwd(**kw, last=last) == B.SF_OK
    assert sfa.sf_last_error() == ""


def ilv(src=P, dst=P2, n=4, Lt=16, batch=2, row=64, inverse=0):
    return L.sf_interleave(src, dst, n, Lt, batch, row, inverse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), B.SF_ERR_INVALID),
    (dict(Lt=-1), B.SF_ERR_INVALID),
    (dict(row=0), B.SF_ERR_INVALID),
    (dict(inverse=2), B.SF_ERR_INVALID),
    (dict(src=None), B.SF_ERR_INVALID),
    (dict(dst=ctypes.c_void_p(0x10000 + 64)), B.SF_ERR_INVALID),   # overlap
    (dict(row=1 << 40, Lt=1 << 30), B.SF_ERR_INVALID),            # overflow
    (dict(row=1 << 30, Lt=1 << 4, n=64, batch=64, dst=ctypes.c_void_p(1 << 50)), B.SF_ERR_UNSUPPORTED),
])
def test_interleave_rejects(kw, status):
    assert ilv(**kw) == status


def test_interleave_empty_is_noop():
    assert ilv(Lt=0, src=None, dst=None) == B.SF_OK
    assert ilv(batch=0) == B.SF_OK


def ilvm(srcs=(0x10000, 0x40000000, 0x80000000), dsts=(0x100000000, 0x140000000, 0x180000000),
         rows=(256, 64, 64), count=None, n=4, Lt=16, batch=2, inverse=0, arrays=True):
    c = len(srcs) if count is None else count
    k = max(1, len(srcs))
    sp = (ctypes.c_void_p * k)(*srcs) if arrays else None
    dp = (ctypes.c_void_p * k)(*dsts) if arrays else None
    rp = (ctypes.c_int64 * k)(*rows) if arrays else None
    return L.sf_interleave_multi(sp, dp, rp, c, n, Lt, batch, inverse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(count=0), B.SF_ERR_INVALID),
    (dict(srcs=(1 << 16,) * 5, dsts=tuple((i + 1) << 32 for i in range(5)), rows=(64,) * 5),
     B.SF_ERR_UNSUPPORTED),                                               # more than 4 tensors
    (dict(arrays=False), B.SF_ERR_INVALID),
    (dict(n=0), B.SF_ERR_INVALID),
    (dict(Lt=-1), B.SF_ERR_INVALID),
    (dict(inverse=2), B.SF_ERR_INVALID),
    (dict(rows=(256, 0, 64)), B.SF_ERR_INVALID),
    (dict(srcs=(0x10000, 0, 0x80000000)), B.SF_ERR_INVALID),
    (dict(dsts=(0x100000000, 0x40000000 + 64, 0x180000000)), B.SF_ERR_INVALID),   # dst 1 inside src 1
    (dict(dsts=(0x100000000, 0x80000000 + 64, 0x180000000)), B.SF_ERR_INVALID),   # dst 1 inside src 2
    (dict(dsts=(0x100000000, 0x100000000 + 64, 0x180000000)), B.SF_ERR_INVALID),  # two dsts overlap
    (dict(rows=(256, 1 << 40, 64), Lt=1 << 30), B.SF_ERR_INVALID),                # overflow
    (dict(rows=(256, 1 << 30, 64), Lt=1 << 4, n=64, batch=64,
          dsts=(1 << 50, 1 << 51, 1 << 52)), B.SF_ERR_UNSUPPORTED),                # 2^32 vectors
])
def test_interleave_multi_rejects(kw, status):
    assert ilvm(**kw) == status
    assert sfa.sf_last_error() != ""


def test_interleave_multi_empty_is_noop():
    assert ilvm(Lt=0, srcs=(0, 0, 0), dsts=(0, 0, 0)) == B.SF_OK
    assert ilvm(batch=0) == B.SF_OK


def dec(q=P, kc=P2, vc=P3, o=P4, batch=1, n=4, T=16, Tmax=16, hq=32, hkv=8, d=128, mode=1, window=0,
        scale=0.088, splits=0, ws=ctypes.c_void_p(0x100000000), wsb=1 << 30):
    return L.sf_attn_decode(q, kc, vc, o, batch, n, T, Tmax, hq, hkv, d, mode, window, scale, splits,
                            ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), B.SF_ERR_INVALID),
    (dict(T=17), B.SF_ERR_INVALID),                  # T > T_max
    (dict(batch=-1), B.SF_ERR_INVALID),
    (dict(splits=-1), B.SF_ERR_INVALID),
    (dict(n=17), B.SF_ERR_UNSUPPORTED),               # n*G = 68 > 64 rows under cross
    (dict(hq=128, hkv=1, mode=0), B.SF_ERR_UNSUPPORTED),  # G = 128 > 64 under intra
    (dict(d=80), B.SF_ERR_UNSUPPORTED),
    (dict(mode=2, window=0), B.SF_ERR_INVALID),
    (dict(ws=None, splits=2, T=200, Tmax=200), B.SF_ERR_INVALID),   # two splits need a workspace
    (dict(wsb=16, splits=2, T=200, Tmax=200), B.SF_ERR_INVALID),    # workspace too small
    (dict(q=None), B.SF_ERR_INVALID),
    (dict(kc=ctypes.c_void_p(0x40000004)), B.SF_ERR_UNSUPPORTED),
])
def test_decode_rejects(kw, status):
    assert dec(**kw) == status


def test_decode_empty_batch_is_noop():
    assert dec(batch=0) == B.SF_OK


def dec_noalloc(q=P, kc=P2, vc=P3, o=P4, batch=1, n=4, T=16, Tmax=16, hq=32, hkv=8, d=128, mode=1, window=0,
                scale=0.088, splits=0):
    return L.sf_attn_decode_noalloc(q, kc, vc, o, batch, n, T, Tmax, hq, hkv, d, mode, window, scale, splits, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), B.SF_ERR_INVALID),
    (dict(T=17), B.SF_ERR_INVALID),
    (dict(splits=-1), B.SF_ERR_INVALID),
    (dict(n=17), B.SF_ERR_UNSUPPORTED),
    (dict(q=None), B.SF_ERR_INVALID),
    (dict(o=P), B.SF_ERR_INVALID),                     # output overlaps q
    # 1024 splits of 4 x 8192 positions at batch 4: 68 MB of partials, beyond the 16 MiB scratch
    (dict(batch=4, T=8192, Tmax=8192, splits=1024), B.SF_ERR_UNSUPPORTED),
])
def test_decode_noalloc_rejects(kw, status):
    assert dec_noalloc(**kw) == status


def test_decode_noalloc_names_the_scratch_limit():
    assert dec_noalloc(batch=4, T=8192, Tmax=8192, splits=1024) == B.SF_ERR_UNSUPPORTED
    assert "scratch" in sfa.sf_last_error()
    assert dec_noalloc(batch=0) == B.SF_OK


def test_workspace_query():
    ws = sfa.sf_attn_decode_workspace_bytes(1, 4, 8192, 32, 8, 128, "cross_full")
    assert ws > 0 and ws % 256 == 0
    # one split writes the output directly: no workspace
    assert sfa.sf_attn_decode_workspace_bytes(1, 4, 8192, 32, 8, 128, "cross_full", num_splits=1) == 0
    # s splits: rows * s * (d + 2) floats, each part rounded to 256 bytes
    rows, s = 1 * 4 * 32, 3
    three = sfa.sf_attn_decode_workspace_bytes(1, 4, 8192, 32, 8, 128, "cross_full", num_splits=s)
    assert three == -(-rows * s * 128 * 4 // 256) * 256 + -(-rows * s * 2 * 4 // 256) * 256
    assert sfa.sf_attn_decode_workspace_bytes(0, 4, 8192, 32, 8, 128, "intra") == 0
    assert sfa.sf_attn_decode_workspace_bytes(1, 4, 0, 32, 8, 128, "intra") == 0
    assert sfa.sf_attn_decode_workspace_bytes(1, 4, 16, 32, 8, 96, "intra") == 0


def test_decode_accepts_more_rows_per_kv_head():
    """n*G up to 64 rows per kv head (e.g. n = 8 streams with G = 8): only
    the argument checks run, on a null-sized workspace query."""
    assert sfa.sf_attn_decode_workspace_bytes(1, 8, 1024, 64, 8, 128, "cross_full") > 0
    assert dec(batch=0, n=8, hq=64) == B.SF_OK
    assert dec(batch=0, n=16, hq=32) == B.SF_OK
    assert dec(batch=0, hq=64, hkv=1, mode=0) == B.SF_OK


def pdec(q=P, kp=P2, vp=P3, table=ctypes.c_void_p(0x20000000), lens=ctypes.c_void_p(0x30000000), o=P4,
         batch=2, n=4, max_T=100, num_pages=64, page=32, max_pages=4, hq=32, hkv=8, d=128, mode=1, window=0,
         scale=0.088, splits=0, ws=ctypes.c_void_p(0x100000000), wsb=1 << 30):
    return L.sf_attn_decode_paged(q, kp, vp, table, lens, o, batch, n, max_T, num_pages, page, max_pages, hq,
                                  hkv, d, mode, window, scale, splits, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(max_T=0), B.SF_ERR_INVALID),
    (dict(batch=-1), B.SF_ERR_INVALID),
    (dict(num_pages=0), B.SF_ERR_INVALID),
    (dict(page=0), B.SF_ERR_INVALID),
    (dict(page=48), B.SF_ERR_UNSUPPORTED),            # not a multiple of 32 tokens
    (dict(max_pages=3), B.SF_ERR_INVALID),            # 3 pages of 32 cannot hold 100 tokens
    (dict(splits=-1), B.SF_ERR_INVALID),
    (dict(n=17), B.SF_ERR_UNSUPPORTED),               # 68 rows per kv head
    (dict(d=96), B.SF_ERR_UNSUPPORTED),
    (dict(mode=2, window=0), B.SF_ERR_INVALID),
    (dict(page=1 << 20, max_pages=1), B.SF_ERR_UNSUPPORTED),   # a page of 2^31 bytes
    (dict(max_T=1 << 30, max_pages=1 << 25), B.SF_ERR_UNSUPPORTED),   # n * max_T >= 2^31
    (dict(table=None), B.SF_ERR_INVALID),
    (dict(lens=None), B.SF_ERR_INVALID),
    (dict(lens=ctypes.c_void_p(0x30000002)), B.SF_ERR_INVALID),
    (dict(kp=ctypes.c_void_p(0x40000008)), B.SF_ERR_UNSUPPORTED),
    (dict(o=ctypes.c_void_p(0x20000000)), B.SF_ERR_INVALID),   # output overlaps the block table
    (dict(ws=None, splits=2), B.SF_ERR_INVALID),
    (dict(wsb=16, splits=2), B.SF_ERR_INVALID),
])
def test_decode_paged_rejects(kw, status):
    assert pdec(**kw) == status


def test_decode_paged_empty_batch_and_workspace_query():
    assert pdec(batch=0) == B.SF_OK
    # one split: no workspace; two: rows * 2 * (d + 2) floats
    assert sfa.sf_attn_decode_paged_workspace_bytes(2, 4, 100, 32, 8, 128, "cross_full", num_splits=1) == 0
    rows = 2 * 4 * 32
    assert (sfa.sf_attn_decode_paged_workspace_bytes(2, 4, 100, 32, 8, 128, "cross_full", num_splits=2)
            == -(-rows * 2 * 128 * 4 // 256) * 256 + -(-rows * 2 * 2 * 4 // 256) * 256)
    assert sfa.sf_attn_decode_paged_workspace_bytes(2, 4, 0, 32, 8, 128, "intra") == 0
    # a window bounds the keys a sequence can see, whatever max_T is
    w = sfa.sf_attn_decode_paged_workspace_bytes(1, 4, 1 << 20, 32, 8, 128, "cross_window", window=4096)
    assert 0 < w <= sfa.sf_attn_decode_workspace_bytes(1, 4, 1 << 20, 32, 8, 128, "cross_full")


def emb(ids=P, tables=P2, out=P3, batch=2, n=4, Lt=16, vocab=100, row=64):
    return L.sf_expand_embed(ids, tables, out, batch, n, Lt, vocab, row, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), B.SF_ERR_INVALID),
    (dict(Lt=-1), B.SF_ERR_INVALID),
    (dict(vocab=0), B.SF_ERR_INVALID),
    (dict(row=0), B.SF_ERR_INVALID),
    (dict(ids=None), B.SF_ERR_INVALID),
    (dict(out=ctypes.c_void_p(0x40000000 + 64)), B.SF_ERR_INVALID),     # out overlaps tables
    (dict(ids=ctypes.c_void_p(0x10002)), B.SF_ERR_UNSUPPORTED),         # ids misaligned
    (dict(row=1 << 40, Lt=1 << 30), B.SF_ERR_INVALID),                 # int64 overflow
    (dict(row=1 << 30, Lt=1 << 10, n=64, out=ctypes.c_void_p(1 << 50)), B.SF_ERR_UNSUPPORTED),
])
def test_expand_embed_rejects(kw, status):
    assert emb(**kw) == status
    assert sfa.sf_last_error() != ""


def test_expand_embed_empty_is_noop():
    assert emb(batch=0) == B.SF_OK
    assert emb(Lt=0, ids=None, tables=None, out=None) == B.SF_OK


def rope(x=P, batch=1, S=16, heads=4, d=128, base=10000.0, pos0=0):
    return L.sf_rope(x, batch, S, heads, d, base, pos0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), B.SF_ERR_INVALID),
    (dict(heads=0), B.SF_ERR_INVALID),
    (dict(d=7), B.SF_ERR_INVALID),
    (dict(base=1.0), B.SF_ERR_INVALID),
    (dict(base=float("nan")), B.SF_ERR_INVALID),
    (dict(pos0=-1), B.SF_ERR_INVALID),
    (dict(d=12), B.SF_ERR_UNSUPPORTED),
    (dict(d=512), B.SF_ERR_UNSUPPORTED),
    (dict(x=None), B.SF_ERR_INVALID),
    (dict(x=ctypes.c_void_p(0x10004)), B.SF_ERR_UNSUPPORTED),
])
def test_rope_rejects(kw, status):
    assert rope(**kw) == status
    assert sfa.sf_last_error() != ""


PB = [ctypes.c_void_p(a << 32) for a in range(1, 11)]   # ten disjoint fake device buffers


def bwd(ptrs=None, batch=1, n=4, Lt=16, hq=4, hkv=2, d=64, mode=1, window=0, scale=0.125, wsb=1 << 20, **over):
    p = list(PB if ptrs is None else ptrs)
    names = ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"]
    for key, val in over.items():
        p[names.index(key)] = val
    return L.sf_attn_bwd(*p[:9], batch, n, Lt, hq, hkv, d, mode, window, scale, p[9], wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), B.SF_ERR_INVALID),
    (dict(n=0), B.SF_ERR_INVALID),
    (dict(hq=6, hkv=4), B.SF_ERR_INVALID),
    (dict(mode=2, window=0), B.SF_ERR_INVALID),
    (dict(d=96), B.SF_ERR_UNSUPPORTED),
    (dict(dq=None), B.SF_ERR_INVALID),
    (dict(lse=None), B.SF_ERR_INVALID),
    (dict(ws=None), B.SF_ERR_INVALID),
    (dict(wsb=16), B.SF_ERR_INVALID),                               # workspace too small
    (dict(dk=PB[0]), B.SF_ERR_INVALID),                             # dk aliases q
    (dict(dv=PB[6]), B.SF_ERR_INVALID),                             # dv aliases dq
    (dict(q=ctypes.c_void_p((1 << 32) + 8)), B.SF_ERR_UNSUPPORTED),  # misaligned
    (dict(batch=1 << 20, Lt=1 << 20), B.SF_ERR_UNSUPPORTED),        # beyond 2^30 elements
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status
    assert sfa.sf_last_error() != ""


def test_bwd_workspace_query():
    # lse*log2(e) and D per (batch, position, query head), 8 bytes each, rounded to 256
    assert sfa.lib().sf_attn_bwd_workspace_bytes(2, 4, 100, 8, 2, 128, 1, 0) == -(-2 * 400 * 8 * 8 // 256) * 256
    assert sfa.lib().sf_attn_bwd_workspace_bytes(0, 4, 100, 8, 2, 128, 1, 0) == 0
    assert bwd(batch=0) == B.SF_OK


def test_every_default_decode_plan_fits_the_noalloc_scratch():
    # The plan puts at most one group per CU (256 groups) of at most 64 query
    # rows, each row's partial (d + 2) floats: at most about 8.5 MB, within
    # the 16 MiB array sf_attn_decode_noalloc holds. Unit counts that do not
    # divide 256 are the edge (255 units at two splits each would need 17 MB).
    limit = int(re.search(r"#define SF_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", HEADER.read_text()).group(1)) << 20
    worst = 0
    for mode in ("intra", "cross_full", "cross_window"):
        for n, hkv, G in ((1, 1, 64), (4, 8, 4), (16, 1, 4), (8, 2, 8), (3, 5, 3), (4, 7, 16), (2, 3, 1)):
            if mode != "intra" and n * G > 64:
                continue
            for batch in (1, 2, 3, 7, 31, 63, 127, 255, 257):
                for T in (1, 100, 1000, 8192):
                    for d in (64, 128):
                        ws = sfa.sf_attn_decode_workspace_bytes(batch, n, T, hkv * G, hkv, d, mode,
                                                                window=4096 if mode == "cross_window" else 0)
                        worst = max(worst, ws)
    assert 0 < worst <= 256 * 64 * (128 + 2) * 4 + 512 <= limit
