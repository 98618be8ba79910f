"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function takes an oracle module (normally ``oracle.sfa``) and
raises AssertionError when the oracle disagrees with an independent statement
of the method: a brute force written in (token, stream) terms, a library
routine (torch's scaled_dot_product_attention in float64), a closed form, or a
figure the pages print. ``tests/test_oracle.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on oracle copies with planted
mistakes and requires every mistake to be caught.
"""
from __future__ import annotations

import math
import pathlib

import numpy as np
import torch

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16ish(rng, shape):
    """Random values that are exactly representable in bfloat16."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# (token, stream) brute force, independent of the p = i*n+k formula
# ---------------------------------------------------------------------------

def allowed_ts(mode, n, tp, kp, tq, kq, window=None):
    """May query (token tp, stream kp) attend to key (token tq, stream kq)?
    Stated in token/stream terms, 0-indexed."""
    if mode == "intra":
        return kq == kp and tq <= tp
    earlier = tq < tp or (tq == tp and kq <= kp)
    if mode == "cross_full":
        return earlier
    dist = (tp - tq) * n + (kp - kq)  # how many expanded positions back
    return earlier and dist < window


def pin_interleave_golden(orc):
    """Positions from the page's 1-indexed formula, evaluated by hand."""
    rows = [list(map(int, ln.split())) for ln in (GOLDEN / "interleave_positions.txt").read_text().splitlines()
            if ln.strip() and not ln.startswith("#")]
    for n in sorted({r[0] for r in rows}):
        sub = [r for r in rows if r[0] == n]
        L = max(r[1] for r in sub)
        # tag each (token, stream) with a unique id and find where it lands
        src = np.zeros((n, 1, L), dtype=np.int64)
        for i in range(L):
            for k in range(n):
                src[k, 0, i] = 1000 * (i + 1) + (k + 1)
        out = orc.interleave(src)[0]
        for _, i1, k1, pos1 in sub:
            assert out[pos1 - 1] == 1000 * i1 + k1, (n, i1, k1, pos1)


def pin_interleave_bruteforce(orc):
    rng = _rng(1)
    for n, B, L, R in [(1, 1, 5, 3), (3, 2, 5, 7), (4, 2, 6, 4)]:
        src = rng.integers(-1000, 1000, size=(n, B, L, R))
        out = orc.interleave(src)
        assert out.shape == (B, n * L, R)
        for b in range(B):
            for i in range(L):
                for k in range(n):
                    assert np.array_equal(out[b, i * n + k], src[k, b, i])
        back = orc.deinterleave(out, n)
        assert np.array_equal(back, src)


def pin_mask_bruteforce(orc):
    for n in (1, 2, 3, 4):
        for L in (1, 2, 5, 9):
            S = n * L
            for mode, windows in (("intra", [None]), ("cross_full", [None]),
                                  ("cross_window", sorted({1, 2, n, n + 1, 3 * n - 1, S, S + 3}))):
                for W in windows:
                    M = orc.mask(mode, n, L, W)
                    assert M.shape == (S, S)
                    for tp in range(L):
                        for kp in range(n):
                            for tq in range(L):
                                for kq in range(n):
                                    want = allowed_ts(mode, n, tp, kp, tq, kq, W)
                                    assert bool(M[tp * n + kp, tq * n + kq]) == want, (mode, n, L, W, tp, kp, tq, kq)


def closed_form_pairs(mode, n, L, W=None):
    """Allowed pairs per head. intra: n streams of causal length L;
    cross_full: causal length S; cross_window: rows p < W see p+1 keys, the
    rest W keys."""
    S = n * L
    if mode == "intra":
        return n * L * (L + 1) // 2
    if mode == "cross_full" or W >= S:
        return S * (S + 1) // 2
    return W * (W + 1) // 2 + (S - W) * W


def pin_pair_counts(orc):
    for n in (1, 2, 4):
        for L in (1, 3, 16, 33):
            S = n * L
            for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 1),
                            ("cross_window", 5), ("cross_window", S // 2 + 1), ("cross_window", S + 7)):
                assert orc.pair_count(mode, n, L, W) == closed_form_pairs(mode, n, L, W), (mode, n, L, W)


def pin_cost_ratios(orc):
    """The page's 16x (dense at n=4) and ~n x (factorised) figures."""
    rows = {}
    for ln in (GOLDEN / "cost_ratios.txt").read_text().splitlines():
        if ln.strip() and not ln.startswith("#"):
            name, n, r = ln.split()
            rows[name] = (int(n), float(r))
    n, dense = rows["dense_over_base"]
    L = 256
    base = orc.pair_count("cross_full", 1, L)
    full = orc.pair_count("cross_full", n, L)
    assert abs(full / base - dense) / dense < 0.01, full / base
    n2, fact = rows["factorized_over_base"]
    intra = orc.pair_count("intra", n2, L)
    assert intra / base == fact


def _sdpa_causal(q, k, v, scale):
    """Textbook causal attention via torch in float64. q,k,v: [S][H][D]."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def pin_cross_full_is_causal(orc):
    rng = _rng(2)
    n, L, B, H, D = 4, 6, 2, 3, 8
    S = n * L
    q, k, v = (_bf16ish(rng, (B, S, H, D)) for _ in range(3))
    scale = 0.37
    o = orc.attn_fwd(q, k, v, "cross_full", n, scale=scale)
    for b in range(B):
        ref = _sdpa_causal(q[b], k[b], v[b], scale)
        assert np.allclose(o[b], ref, atol=1e-12, rtol=1e-12)


def pin_intra_is_per_stream_causal(orc):
    rng = _rng(3)
    n, L, B, H, D = 3, 7, 2, 2, 8
    S = n * L
    q, k, v = (_bf16ish(rng, (B, S, H, D)) for _ in range(3))
    scale = 0.5
    o = orc.attn_fwd(q, k, v, "intra", n, scale=scale)
    for b in range(B):
        for s in range(n):
            # stream s = positions s, n+s, 2n+s, ... (written with explicit indices)
            idx = [i * n + s for i in range(L)]
            ref = _sdpa_causal(q[b, idx], k[b, idx], v[b, idx], scale)
            assert np.allclose(o[b, idx], ref, atol=1e-12, rtol=1e-12)


def pin_n1_all_modes_causal(orc):
    rng = _rng(4)
    L, H, D = 9, 2, 4
    q, k, v = (_bf16ish(rng, (1, L, H, D)) for _ in range(3))
    ref = _sdpa_causal(q[0], k[0], v[0], 0.5)
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", L)):
        o = orc.attn_fwd(q, k, v, mode, 1, window=W, scale=0.5)
        assert np.allclose(o[0], ref, atol=1e-12, rtol=1e-12), mode


def pin_window_limits(orc):
    rng = _rng(5)
    n, L, H, D = 4, 5, 2, 8
    S = n * L
    q, k, v = (_bf16ish(rng, (1, S, H, D)) for _ in range(3))
    full = orc.attn_fwd(q, k, v, "cross_full", n, scale=0.3)
    for W in (S, S + 1, 10 * S):
        assert np.allclose(orc.attn_fwd(q, k, v, "cross_window", n, window=W, scale=0.3), full, atol=1e-12)
    # a one-position window is the query itself: O = V exactly
    assert np.array_equal(orc.attn_fwd(q, k, v, "cross_window", n, window=1, scale=0.3), v)


def pin_uniform_keys_closed_form(orc):
    """Constant keys give a uniform softmax over the allowed keys: O is the
    mean of the allowed values and lse = ln(#allowed) + scale*q.k0. With
    values equal to 1 on key j only, O * #allowed is the 0/1 mask row."""
    n, L, D = 3, 6, 4
    S = n * L
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 4), ("cross_window", 7)):
        q = np.ones((1, S, 1, D))
        k = np.zeros((1, S, 1, D))
        for j in range(S):
            v = np.zeros((1, S, 1, D))
            v[0, j, 0, :] = 1.0
            o, lse = orc.attn_fwd(q, k, v, mode, n, window=W, scale=1.0, with_lse=True)
            for p in range(S):
                tp, kp = divmod(p, n)
                cnt = sum(allowed_ts(mode, n, tp, kp, tq, kq, W) for tq in range(L) for kq in range(n))
                tj, kj = divmod(j, n)
                want = (1.0 / cnt) if allowed_ts(mode, n, tp, kp, tj, kj, W) else 0.0
                assert abs(o[0, p, 0, 0] - want) < 1e-14, (mode, W, p, j)
                assert abs(lse[0, 0, p] - math.log(cnt)) < 1e-12


def pin_gqa_is_repeated_mha(orc):
    rng = _rng(6)
    n, L, B, Hq, Hkv, D = 2, 5, 1, 6, 2, 4
    S = n * L
    q = _bf16ish(rng, (B, S, Hq, D))
    k = _bf16ish(rng, (B, S, Hkv, D))
    v = _bf16ish(rng, (B, S, Hkv, D))
    G = Hq // Hkv
    # consecutive query heads share a key/value head
    k_rep = np.stack([k[:, :, h // G] for h in range(Hq)], axis=2)
    v_rep = np.stack([v[:, :, h // G] for h in range(Hq)], axis=2)
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 3)):
        a = orc.attn_fwd(q, k, v, mode, n, window=W, scale=0.4)
        b = orc.attn_fwd(q, k_rep, v_rep, mode, n, window=W, scale=0.4)
        assert np.allclose(a, b, atol=1e-13), mode


def _py_attention(q, k, v, scale, ok):
    """Pure-Python attention, one head: q,k,v lists of D-vectors; ok(p, j)."""
    out, lses = [], []
    for p, qp in enumerate(q):
        s = {j: scale * sum(a * b for a, b in zip(qp, kj)) for j, kj in enumerate(k) if ok(p, j)}
        mx = max(s.values())
        w = {j: math.exp(x - mx) for j, x in s.items()}
        tot = sum(w.values())
        out.append([sum(w[j] * v[j][d] for j in w) / tot for d in range(len(v[0]))])
        lses.append(mx + math.log(tot))
    return out, lses


def pin_pure_python_bruteforce(orc):
    rng = _rng(7)
    for n, L, W in ((2, 4, 3), (4, 4, 6), (3, 5, 2)):
        S = n * L
        D = 3
        q, k, v = (_bf16ish(rng, (1, S, 1, D)) for _ in range(3))
        for mode in ("intra", "cross_full", "cross_window"):
            ok = lambda p, j: allowed_ts(mode, n, p // n, p % n, j // n, j % n, W)  # noqa: E731
            ref, ref_lse = _py_attention(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), 0.7, ok)
            o, lse = orc.attn_fwd(q, k, v, mode, n, window=W, scale=0.7, with_lse=True)
            assert np.allclose(o[0, :, 0], np.array(ref), atol=1e-12, rtol=0), mode
            assert np.allclose(lse[0, 0], np.array(ref_lse), atol=1e-12, rtol=0), mode


def pin_stream_permutation_equivariance(orc):
    """Intra attention treats streams independently: permuting the streams of
    the inputs permutes the streams of the output."""
    rng = _rng(8)
    n, L, H, D = 4, 5, 2, 4
    S = n * L
    q, k, v = (_bf16ish(rng, (1, S, H, D)) for _ in range(3))
    perm = [2, 0, 3, 1]
    idx = np.array([i * n + perm[s] for i in range(L) for s in range(n)])
    o = orc.attn_fwd(q, k, v, "intra", n, scale=0.5)
    o_perm = orc.attn_fwd(q[:, idx], k[:, idx], v[:, idx], "intra", n, scale=0.5)
    assert np.allclose(o_perm, o[:, idx], atol=1e-13)


def pin_decode_bruteforce(orc):
    """Decode straight from the per-stream cache, written with (token, stream)
    predicates and no interleave; also equal to the last n prefill rows."""
    rng = _rng(9)
    B, n, T, Tmax, Hq, Hkv, D = 2, 3, 4, 6, 4, 2, 3
    G = Hq // Hkv
    q = _bf16ish(rng, (B, n, Hq, D))
    kc = _bf16ish(rng, (B, n, Tmax, Hkv, D))
    vc = _bf16ish(rng, (B, n, Tmax, Hkv, D))
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 5)):
        o = orc.decode(q, kc, vc, T, mode, window=W, scale=0.6)
        for b in range(B):
            for h in range(Hq):
                kh = h // G
                keys = [(t, s) for t in range(T) for s in range(n)]
                for kp in range(n):
                    sel = [(t, s) for (t, s) in keys if allowed_ts(mode, n, T - 1, kp, t, s, W)]
                    sc = [0.6 * float(np.dot(q[b, kp, h], kc[b, s, t, kh])) for t, s in sel]
                    mx = max(sc)
                    w = [math.exp(x - mx) for x in sc]
                    want = sum(wi * vc[b, s, t, kh] for wi, (t, s) in zip(w, sel)) / sum(w)
                    assert np.allclose(o[b, kp, h], want, atol=1e-12), (mode, b, h, kp)
        # decode == the last n rows of prefill over the T tokens
        K = np.stack([np.stack([kc[b, s, t] for t in range(T) for s in range(n)]) for b in range(B)])
        V = np.stack([np.stack([vc[b, s, t] for t in range(T) for s in range(n)]) for b in range(B)])
        Q = np.zeros((B, n * T, Hq, D))
        Q[:, (T - 1) * n:] = q
        full = orc.attn_fwd(Q, K, V, mode, n, window=W, scale=0.6)
        assert np.allclose(full[:, (T - 1) * n:], o, atol=1e-12), mode


def pin_rows_subset(orc):
    """Computing selected rows gives the same values as the full output."""
    rng = _rng(10)
    n, L, H, D = 4, 8, 2, 4
    S = n * L
    q, k, v = (_bf16ish(rng, (1, S, H, D)) for _ in range(3))
    rows = np.array([0, 3, 7, 8, 17, S - 1])
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 9)):
        full = orc.attn_fwd(q, k, v, mode, n, window=W, scale=0.5, block=5)
        sub = orc.attn_fwd(q, k, v, mode, n, window=W, scale=0.5, rows=rows)
        assert np.allclose(full[:, rows], sub, atol=1e-14, rtol=0)


def pin_last_stream(orc):
    """Last-stream queries (stream n-1 of each token) against torch SDPA and a
    pure-Python brute force, both stated in (token, stream) terms: under
    cross_full the query of token i sees every stream of tokens 0..i; under
    intra it is causal attention over stream n-1 alone; under cross_window the
    (token, stream) window predicate."""
    rng = _rng(11)
    n, L, B, Hq, Hkv, D = 3, 5, 2, 4, 2, 4
    G = Hq // Hkv
    ql = _bf16ish(rng, (B, L, Hq, D))
    # K/V listed as (token, stream) pairs in token-major order
    ts = [(t, s) for t in range(L) for s in range(n)]
    k, v = (_bf16ish(rng, (B, len(ts), Hkv, D)) for _ in range(2))
    scale = 0.45
    o = orc.attn_fwd_last_stream(ql, k, v, "cross_full", n, scale=scale)
    for b in range(B):
        for h in range(Hq):
            allow = torch.tensor([[tk <= i for (tk, _) in ts] for i in range(L)])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(ql[b, :, h])[None], torch.from_numpy(k[b, :, h // G])[None],
                torch.from_numpy(v[b, :, h // G])[None], attn_mask=allow[None], scale=scale)[0].numpy()
            assert np.allclose(o[b, :, h], ref, atol=1e-12), ("cross_full", b, h)
    o = orc.attn_fwd_last_stream(ql, k, v, "intra", n, scale=scale)
    last = [j for j, (_, sk) in enumerate(ts) if sk == n - 1]
    for b in range(B):
        ref = _sdpa_causal(ql[b, :, ::G], k[b, last], v[b, last], scale)    # heads h = 0, G, 2G, ...
        assert np.allclose(o[b, :, ::G], ref, atol=1e-12), ("intra", b)
    W = 4
    o = orc.attn_fwd_last_stream(ql, k, v, "cross_window", n, window=W, scale=scale)
    for h in range(Hq):
        ok = lambda i, j: allowed_ts("cross_window", n, i, n - 1, ts[j][0], ts[j][1], W)  # noqa: E731
        ref, _ = _py_attention(ql[0, :, h].tolist(), k[0, :, h // G].tolist(), v[0, :, h // G].tolist(), scale, ok)
        assert np.allclose(o[0, :, h], np.array(ref), atol=1e-12), ("cross_window", h)


def pin_expand_embed(orc):
    """Each output row against the page's 1-indexed placement, evaluated with
    explicit loops; ids outside the vocabulary give zero rows."""
    rng = _rng(12)
    n, B, L, vocab, R = 3, 2, 5, 7, 4
    tables = rng.integers(-1000, 1000, size=(n, vocab, R))
    ids = rng.integers(0, vocab, size=(B, L))
    ids[1, 2] = vocab          # out of range
    ids[0, 4] = -1             # out of range
    out = orc.expand_embed(ids, tables)
    assert out.shape == (B, n * L, R)
    for b in range(B):
        for i1 in range(1, L + 1):             # 1-indexed token
            for k1 in range(1, n + 1):         # 1-indexed stream
                pos = (i1 - 1) * n + k1 - 1    # the page's (i-1)n+k, made 0-indexed
                tok = ids[b, i1 - 1]
                want = tables[k1 - 1, tok] if 0 <= tok < vocab else np.zeros(R, dtype=tables.dtype)
                assert np.array_equal(out[b, pos], want), (b, i1, k1)


def pin_rope(orc):
    """Rotate-half rotary encoding against its complex-number statement
    (z_j = x_j + i x_{j+d/2} times e^{i p theta_j}), the identity at position
    0, norm preservation, and the relative-position property: shifting every
    position by the same amount leaves all q.k products unchanged."""
    rng = _rng(13)
    B, S, H, d, base = 2, 9, 3, 8, 500.0
    x = rng.standard_normal((B, S, H, d))
    y = orc.rope(x, base, pos0=5)
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    theta = np.array([base ** (-(2 * j) / d) for j in range(half)])
    for s_ in range(S):
        w = z[:, s_] * np.exp(1j * (5 + s_) * theta)
        assert np.allclose(y[:, s_, :, :half], w.real, atol=1e-12)
        assert np.allclose(y[:, s_, :, half:], w.imag, atol=1e-12)
    assert np.allclose(orc.rope(x[:, :1], base, pos0=0), x[:, :1], atol=0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    q, k = x, rng.standard_normal((B, S, H, d))
    dots = np.einsum("bshd,bthd->bhst", orc.rope(q, base, 0), orc.rope(k, base, 0))
    dots_shift = np.einsum("bshd,bthd->bhst", orc.rope(q, base, 37), orc.rope(k, base, 37))
    assert np.allclose(dots, dots_shift, atol=1e-10)


def pin_backward(orc):
    """Gradients against central finite differences of the scalar loss
    sum(dout * o) (all three masks, GQA), against torch autograd through
    causal SDPA (cross_full), and GQA against MHA with repeated K/V whose
    key/value gradients are summed over each group."""
    rng = _rng(14)
    n, L, B, Hq, Hkv, D = 2, 3, 1, 4, 2, 3
    S = n * L
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    do = rng.standard_normal((B, S, Hq, D))
    scale, eps = 0.6, 1e-6
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 3)):
        dq, dk, dv = orc.attn_bwd(q, k, v, do, mode, n, window=W, scale=scale)
        loss = lambda q_, k_, v_: float(np.sum(do * orc.attn_fwd(q_, k_, v_, mode, n, window=W, scale=scale)))  # noqa: E731
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert np.allclose(g, num, atol=1e-6), (mode, name)
    # torch autograd through causal SDPA, one head group at a time
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q[0], k[0], v[0]))
    G = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.transpose(0, 1), kt.repeat_interleave(G, dim=1).transpose(0, 1),
        vt.repeat_interleave(G, dim=1).transpose(0, 1), is_causal=True, scale=scale).transpose(0, 1)
    (o * torch.tensor(do[0])).sum().backward()
    dq, dk, dv = orc.attn_bwd(q, k, v, do, "cross_full", n, scale=scale)
    assert np.allclose(dq[0], qt.grad.numpy(), atol=1e-12)
    assert np.allclose(dk[0], kt.grad.numpy(), atol=1e-12)
    assert np.allclose(dv[0], vt.grad.numpy(), atol=1e-12)
    # selected query rows and key rows equal the same rows of the full gradients
    rows, keys = np.array([0, 3, S - 1]), np.array([1, 4, S - 2])
    for mode, W in (("intra", None), ("cross_full", None), ("cross_window", 3)):
        full = orc.attn_bwd(q, k, v, do, mode, n, window=W, scale=scale)
        sub = orc.attn_bwd(q, k, v, do, mode, n, window=W, scale=scale, rows=rows, key_rows=keys, block=2)
        assert np.allclose(sub[0], full[0][:, rows], atol=1e-13), mode
        assert np.allclose(sub[1], full[1][:, keys], atol=1e-13), mode
        assert np.allclose(sub[2], full[2][:, keys], atol=1e-13), mode
    # GQA: repeated K/V as MHA, gradients summed over each group
    k_rep, v_rep = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    for mode, W in (("intra", None), ("cross_window", 4)):
        a = orc.attn_bwd(q, k, v, do, mode, n, window=W, scale=scale)
        m = orc.attn_bwd(q, k_rep, v_rep, do, mode, n, window=W, scale=scale)
        assert np.allclose(a[0], m[0], atol=1e-12)
        assert np.allclose(a[1], m[1].reshape(B, S, Hkv, G, D).sum(axis=3), atol=1e-12)
        assert np.allclose(a[2], m[2].reshape(B, S, Hkv, G, D).sum(axis=3), atol=1e-12)


def pin_decode_paged(orc):
    """Paged decode with per-sequence lengths: a (token, stream) brute force
    that walks the block table by explicit loops, the last n prefill rows of
    each sequence at its own length, and invariance under a permutation of the
    physical pages. Includes n = 8 with n*G = 32 rows per kv head."""
    rng = _rng(21)
    for n, Hq, Hkv, P, lens, W in ((3, 4, 2, 2, (5, 1, 3), 4), (8, 8, 2, 3, (2, 4), 11)):
        B = len(lens)
        D = 3
        G = Hq // Hkv
        maxp = max((t + P - 1) // P for t in lens) + 1
        npages = B * n * maxp + 2
        kp = _bf16ish(rng, (npages, P, Hkv, D))
        vp = _bf16ish(rng, (npages, P, Hkv, D))
        table = rng.permutation(npages)[:B * n * maxp].reshape(B, n, maxp)
        q = _bf16ish(rng, (B, n, Hq, D))
        for mode in ("intra", "cross_full", "cross_window"):
            o = orc.decode_paged(q, kp, vp, table, np.array(lens), mode, window=W, scale=0.6)
            for b in range(B):
                T = lens[b]

                def key(arr, t, s, kh):
                    page = int(table[b][s][t // P])
                    return arr[page][t - (t // P) * P][kh]
                for h in range(Hq):
                    kh = h // G
                    for kq in range(n):
                        sel = [(t, s) for t in range(T) for s in range(n)
                               if allowed_ts(mode, n, T - 1, kq, t, s, W)]
                        sc = [0.6 * float(np.dot(q[b, kq, h], key(kp, t, s, kh))) for t, s in sel]
                        mx = max(sc)
                        w = [math.exp(x - mx) for x in sc]
                        want = sum(wi * key(vp, t, s, kh) for wi, (t, s) in zip(w, sel)) / sum(w)
                        assert np.allclose(o[b, kq, h], want, atol=1e-12), (mode, b, h, kq)
                # the last n rows of prefill over this sequence's T tokens
                K = np.stack([key(kp, t, s, slice(None)) for t in range(T) for s in range(n)])[None]
                V = np.stack([key(vp, t, s, slice(None)) for t in range(T) for s in range(n)])[None]
                Q = np.zeros((1, n * T, Hq, D))
                Q[0, (T - 1) * n:] = q[b]
                full = orc.attn_fwd(Q, K, V, mode, n, window=W, scale=0.6)
                assert np.allclose(full[0, (T - 1) * n:], o[b], atol=1e-12), (mode, b)
            # moving the pages and rewriting the table changes nothing
            perm = rng.permutation(npages)
            kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
            kp2[perm], vp2[perm] = kp, vp
            o2 = orc.decode_paged(q, kp2, vp2, perm[table], np.array(lens), mode, window=W, scale=0.6)
            assert np.array_equal(o, o2), mode


ALL_PINS = [
    pin_interleave_golden,
    pin_interleave_bruteforce,
    pin_mask_bruteforce,
    pin_pair_counts,
    pin_cost_ratios,
    pin_cross_full_is_causal,
    pin_intra_is_per_stream_causal,
    pin_n1_all_modes_causal,
    pin_window_limits,
    pin_uniform_keys_closed_form,
    pin_gqa_is_repeated_mha,
    pin_pure_python_bruteforce,
    pin_stream_permutation_equivariance,
    pin_decode_bruteforce,
    pin_decode_paged,
    pin_last_stream,
    pin_expand_embed,
    pin_rope,
    pin_backward,
    pin_rows_subset,
]
