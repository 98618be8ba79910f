"""Stream-factorized attention, written as its plain definition (float64).

TEST INFRASTRUCTURE ONLY: see the package docstring for who may import this.

Notation (0-indexed): n streams, L tokens, S = n*L expanded positions.
Token i, stream k sits at expanded position p = i*n + k. The page writes the
same map 1-indexed as (i-1)n + k ([HD-tahou] 隐式序列缩放的技术细节, step 1);
subtracting 1 from a 1-indexed position gives this 0-indexed form. Hence
stream(p) = p mod n and token(p) = p div n.
"""
from __future__ import annotations

import numpy as np

MODES = ("intra", "cross_full", "cross_window")


# ---------------------------------------------------------------------------
# Stream expansion
# ---------------------------------------------------------------------------

def interleave(src: np.ndarray) -> np.ndarray:
    """Place stream k of token i at expanded position i*n + k.

    [HD-tahou] 隐式序列缩放的技术细节, step 1: given the n per-stream embeddings,
    the k-th stream representation of the i-th token goes to position
    (i-1)n+k (1-indexed), giving a sequence of length nL.

    src: [n][B][L][...] (one slab per stream). Returns [B][n*L][...].
    """
    src = np.asarray(src)
    n, B, L = src.shape[:3]
    out = np.empty((B, n * L) + src.shape[3:], dtype=src.dtype)
    for k in range(n):
        # positions k, n+k, 2n+k, ... are token 0, 1, 2, ... of stream k
        out[:, k::n] = src[k]
    return out


def deinterleave(x: np.ndarray, n: int) -> np.ndarray:
    """Inverse of :func:`interleave`: [B][n*L][...] -> [n][B][L][...].

    Used to split an expanded sequence back into per-stream slabs, e.g. to
    fill the per-stream KV cache ([HD-aiflow] "Latent computation scaling and
    Hidden Decoding": the KV cache of the internal streams is kept as context).
    """
    x = np.asarray(x)
    S = x.shape[1]
    if S % n:
        raise ValueError("expanded length must be a multiple of n")
    return np.stack([x[:, k::n] for k in range(n)])


def expand_embed(ids: np.ndarray, tables: np.ndarray) -> np.ndarray:
    """The expanded sequence's input rows, straight from the n embedding tables.

    [HD-tahou] 隐式序列缩放的技术细节, step 1: with n copies of the vocabulary
    embedding, stream k's representation of token i is row ids[i] of table k,
    and it is placed at expanded position (i-1)n+k (1-indexed).

    ids: [B][L] integers; tables: [n][vocab][...]. Returns [B][n*L][...].
    An id outside [0, vocab) gives a row of zeros (the kernel's documented
    behaviour; the pages do not consider invalid ids).
    """
    ids = np.asarray(ids)
    tables = np.asarray(tables)
    n, vocab = tables.shape[:2]
    B, L = ids.shape
    per_stream = np.zeros((n, B, L) + tables.shape[2:], dtype=tables.dtype)
    valid = (ids >= 0) & (ids < vocab)
    for k in range(n):
        per_stream[k][valid] = tables[k][ids[valid]]
    return interleave(per_stream)


def rope(x: np.ndarray, base: float, pos0: int = 0) -> np.ndarray:
    """Rotary position encoding at continuous expanded positions (float64).

    [HD-tahou] 隐式序列缩放的技术细节, step 2: the expanded sequence runs under
    a continuous position encoding, so row s of the expanded sequence has
    position pos0 + s: the streams of a token take consecutive positions. The
    page does not name the encoding; the rotary encoding in its rotate-half
    form is taken: for j < d/2, with theta_j = base^(-2j/d) and angle
    a = position * theta_j,
        y[j]       = x[j] cos a - x[j + d/2] sin a
        y[j + d/2] = x[j + d/2] cos a + x[j] sin a.

    x: [B][S][H][d]. Returns float64 [B][S][H][d].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    pos = pos0 + np.arange(x.shape[1], dtype=np.float64)
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = pos[:, None] * theta[None, :]                    # [S][d/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# Masks
# ---------------------------------------------------------------------------

def mask(mode: str, n: int, L: int, window: int | None = None, rows=None) -> np.ndarray:
    """Which keys each query may attend to, as an explicit boolean matrix.

    Returns M[len(rows)][S] with M[r, q] True iff query position p = rows[r]
    may attend to key position q. ``rows`` defaults to all S positions.

    * cross_full: standard causal attention over the expanded sequence,
      q <= p ([HD-tahou] 隐式序列缩放的技术细节, step 2, and the cross-stream
      layer of 规模化落地的工程优化 in its full-attention form).
    * cross_window: the same, kept within a sliding window of ``window``
      expanded positions counting the query itself: 0 <= p - q < window
      (规模化落地的工程优化: cross-stream layers keep the base layer's form,
      sliding window or full).
    * intra: only earlier positions of the same stream, the query itself
      included: q <= p and q mod n == p mod n (规模化落地的工程优化, the
      intra-stream layer).
    """
    if mode not in MODES:
        raise ValueError(f"unknown mode {mode!r}")
    S = n * L
    p = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    q = np.arange(S, dtype=np.int64)
    P = p[:, None]
    Q = q[None, :]
    allowed = Q <= P
    if mode == "intra":
        allowed &= (Q % n) == (P % n)
    elif mode == "cross_window":
        if window is None or window < 1:
            raise ValueError("cross_window needs window >= 1")
        allowed &= (P - Q) < window
    return allowed


def pair_count(mode: str, n: int, L: int, window: int | None = None, block: int = 2048) -> int:
    """Number of allowed (query, key) pairs of one head: the popcount of
    :func:`mask`, counted in row blocks. Useful attention work is proportional
    to it ([HD-tahou] 规模化落地的工程优化: dense attention grows with the
    square of the sequence length, 16x at n=4; the factorised form adds about
    n times)."""
    S = n * L
    total = 0
    for r0 in range(0, S, block):
        total += int(mask(mode, n, L, window, np.arange(r0, min(S, r0 + block))).sum())
    return total


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray, scale: float):
    """Masked softmax attention for one head, the textbook definition.

    q: [R][D] queries, k and v: [S][D] keys and values, allowed: [R][S].
    Returns (o [R][D], lse [R]) with
        o[r]   = sum_j w[r,j] v[j] / sum_j w[r,j],   w[r,j] = exp(s[r,j] - max_j s[r,j])
        lse[r] = ln sum_{j allowed} exp(s[r,j]),     s = scale * q k^T,
    where disallowed scores are -inf. Every row must admit at least one key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = float(scale) * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row admits no key")
    w = np.exp(s - m)
    den = w.sum(axis=1, keepdims=True)
    o = (w @ v) / den
    lse = m[:, 0] + np.log(den[:, 0])
    return o, lse


def attn_fwd(q, k, v, mode: str, n: int, window: int | None = None, scale: float | None = None,
             rows=None, block: int = 512, with_lse: bool = False):
    """Stream-factorized attention over the expanded sequence.

    q: [B][S][Hq][D], k and v: [B][S][Hkv][D] (any real dtype; computed in
    float64). Grouped-query attention ([HD-aiflow] "Tencent's ecosystem first
    scaling strategy"): query head h reads key/value head h // (Hq/Hkv).
    ``rows`` restricts the output to those query positions (all by default).

    Returns o [B][len(rows)][Hq][D] (and lse [B][Hq][len(rows)] if asked).
    The mask rows are built explicitly, ``block`` query rows at a time, and the
    full dense score rows are computed, masked pairs included: nothing is
    skipped.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if S % n or Hq % Hkv:
        raise ValueError("S must be a multiple of n and Hq of Hkv")
    G = Hq // Hkv
    L = S // n
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((B, len(rows), Hq, D))
    lse = np.empty((B, Hq, len(rows)))
    for r0 in range(0, len(rows), block):
        rr = rows[r0:r0 + block]
        allowed = mask(mode, n, L, window, rr)
        for b in range(B):
            for h in range(Hq):
                kh = h // G
                ob, lb = attend(q[b, rr, h], k[b, :, kh], v[b, :, kh], allowed, scale)
                o[b, r0:r0 + len(rr), h] = ob
                lse[b, h, r0:r0 + len(rr)] = lb
    return (o, lse) if with_lse else o


def attn_fwd_last_stream(q_last, k, v, mode: str, n: int, window: int | None = None,
                         scale: float | None = None, with_lse: bool = False):
    """Attention for the queries of the last stream only.

    [HD-tahou] 规模化落地的工程优化 (KV mirror: only the final stream passes
    through the mirrored layers) and 中间流的作用验证 (the final stream reads
    the intermediate streams): for token i the query is stream n-1, at
    expanded position i*n + n-1, and it attends under the same masks as every
    other position. So the result is rows i*n + n-1 of :func:`attn_fwd`.

    q_last: [B][L][Hq][D] (row i = stream n-1 of token i); k, v:
    [B][n*L][Hkv][D]. Returns o [B][L][Hq][D] (and lse [B][Hq][L]).
    """
    q_last = np.asarray(q_last, dtype=np.float64)
    B, L, Hq, D = q_last.shape
    q = np.zeros((B, n * L, Hq, D))
    rows = np.arange(L) * n + (n - 1)
    q[:, rows] = q_last
    return attn_fwd(q, k, v, mode, n, window=window, scale=scale, rows=rows, with_lse=with_lse)


def _probs_and_dscores(qh, kh, vh, do, allowed, scale):
    """One head's P (masked softmax rows of scale * Q K^T, zero where masked)
    and dS = P * (dP - rowsum(dP * P)) with dP = dO V^T."""
    s = float(scale) * (qh @ kh.T)
    s = np.where(allowed, s, -np.inf)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    pr = w / w.sum(axis=1, keepdims=True)
    dp = do @ vh.T
    ds = pr * (dp - (dp * pr).sum(axis=1, keepdims=True))
    return pr, ds


def attn_bwd(q, k, v, dout, mode: str, n: int, window: int | None = None, scale: float | None = None,
             block: int = 512, rows=None, key_rows=None):
    """Gradients of :func:`attn_fwd` for the loss sum(dout * o), in float64.

    The pages report training step times for the method ([HD-tahou]
    实验效果与成本分析); training needs the backward of each attention layer.
    With P the masked softmax of S = scale * Q K^T (rows over admitted keys),
    O = P V and the upstream gradient dO:
        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dP * P)),
        dQ = scale dS K,   dK = scale dS^T Q,
    and under grouped-query attention a key/value head's gradients are the
    sums over the query heads that read it.

    q, dout: [B][S][Hq][D]; k, v: [B][S][Hkv][D]. Returns (dq, dk, dv).
    With ``rows`` and ``key_rows`` (position arrays) only dq at those query
    rows and dk, dv at those key rows are returned; the query rows that see
    one of the keys are found from the mask and computed in full.
    """
    if rows is not None or key_rows is not None:
        return _attn_bwd_subset(q, k, v, dout, mode, n, window, scale, block,
                                np.arange(0) if rows is None else np.asarray(rows, dtype=np.int64),
                                np.arange(0) if key_rows is None else np.asarray(key_rows, dtype=np.int64))
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    L = S // n
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, S, block):
        rr = np.arange(r0, min(S, r0 + block))
        allowed = mask(mode, n, L, window, rr)
        for b in range(B):
            for h in range(Hq):
                kh = h // G
                do = dout[b, rr, h]
                pr, ds = _probs_and_dscores(q[b, rr, h], k[b, :, kh], v[b, :, kh], do, allowed, scale)
                dv[b, :, kh] += pr.T @ do
                dq[b, rr, h] = float(scale) * (ds @ k[b, :, kh])
                dk[b, :, kh] += float(scale) * (ds.T @ q[b, rr, h])
    return dq, dk, dv


def _attn_bwd_subset(q, k, v, dout, mode, n, window, scale, block, rows, key_rows):
    """dq at ``rows`` and dk, dv at ``key_rows`` (same formulas as attn_bwd)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    L = S // n
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    # query rows whose softmax touches one of the keys
    seeing = np.zeros(S, dtype=bool)
    for r0 in range(0, S, block):
        rr = np.arange(r0, min(S, r0 + block))
        if len(key_rows):
            seeing[rr] = mask(mode, n, L, window, rr)[:, key_rows].any(axis=1)
    need = np.union1d(rows, np.nonzero(seeing)[0])
    dq = np.zeros((B, len(rows), Hq, D))
    dk = np.zeros((B, len(key_rows), Hkv, D))
    dv = np.zeros((B, len(key_rows), Hkv, D))
    row_at = {int(r): i for i, r in enumerate(rows)}
    for r0 in range(0, len(need), block):
        rr = need[r0:r0 + block]
        allowed = mask(mode, n, L, window, rr)
        for b in range(B):
            for h in range(Hq):
                kh = h // G
                do = dout[b, rr, h]
                pr, ds = _probs_and_dscores(q[b, rr, h], k[b, :, kh], v[b, :, kh], do, allowed, scale)
                for i, r in enumerate(rr):
                    if int(r) in row_at:
                        dq[b, row_at[int(r)], h] = float(scale) * (ds[i] @ k[b, :, kh])
                if len(key_rows):
                    dv[b, :, kh] += pr[:, key_rows].T @ do
                    dk[b, :, kh] += float(scale) * (ds[:, key_rows].T @ q[b, rr, h])
    return dq, dk, dv


def decode(q_new, k_cache, v_cache, T: int, mode: str, window: int | None = None,
           scale: float | None = None):
    """One decode step: the n stream queries of token T-1 in one pass.

    [HD-tahou] 实验效果与成本分析: the n streams of a new token are processed
    in parallel in one forward pass. The per-stream KV cache ([HD-aiflow]
    "Latent computation scaling and Hidden Decoding"; independent per-stream
    state, [HD-tahou] 中间流的作用验证) holds tokens 0..T-1, token T-1's own
    n rows included.

    q_new: [B][n][Hq][D]; k_cache, v_cache: [B][n][T_max][Hkv][D].
    Returns o [B][n][Hq][D]: row k is the output at expanded position
    (T-1)*n + k, i.e. the last n rows of :func:`attn_fwd` over the T tokens.
    """
    q_new = np.asarray(q_new, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)[:, :, :T]
    vc = np.asarray(v_cache, dtype=np.float64)[:, :, :T]
    B, n, Hq, D = q_new.shape
    Hkv = kc.shape[3]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    # Rebuild the expanded key/value sequence: position t*n + k holds stream k of token t.
    K = interleave(np.moveaxis(kc, 1, 0))  # [B][nT][Hkv][D]
    V = interleave(np.moveaxis(vc, 1, 0))
    rows = (T - 1) * n + np.arange(n)
    allowed = mask(mode, n, T, window, rows)
    o = np.empty((B, n, Hq, D))
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            o[b, :, h], _ = attend(q_new[b, :, h], K[b, :, kh], V[b, :, kh], allowed, scale)
    return o


def gather_pages(pages, block_table, T: int):
    """The logical per-stream cache of one sequence from a paged pool.

    pages: [num_pages][P][Hkv][D]; block_table: [n][max_pages] (ints).
    Token t of stream k lives in row t mod P of page block_table[k][t div P].
    Returns [n][T][Hkv][D].
    """
    pages = np.asarray(pages)
    P = pages.shape[1]
    bt = np.asarray(block_table)
    n = bt.shape[0]
    t = np.arange(T)
    return np.stack([pages[bt[k, t // P], t % P] for k in range(n)])


def decode_paged(q_new, k_pages, v_pages, block_table, seq_lens, mode: str,
                 window: int | None = None, scale: float | None = None):
    """Decode of a batch of sequences of different lengths against a paged
    per-stream cache.

    Each sequence b runs :func:`decode` at its own length T_b = seq_lens[b]
    (its n stream queries of token T_b - 1, [HD-tahou] 实验效果与成本分析)
    against its per-stream caches ([HD-aiflow] "Latent computation scaling and
    Hidden Decoding"), which here are spread over fixed-size pages: stream k's
    token t is row t mod P of page block_table[b][k][t div P].

    q_new: [B][n][Hq][D]; k_pages, v_pages: [num_pages][P][Hkv][D];
    block_table: [B][n][max_pages]; seq_lens: [B], each >= 1.
    Returns o [B][n][Hq][D].
    """
    q_new = np.asarray(q_new, dtype=np.float64)
    B = q_new.shape[0]
    out = np.empty_like(q_new)
    for b in range(B):
        T = int(seq_lens[b])
        if T < 1:
            raise ValueError("every sequence holds at least its newest token")
        kc = gather_pages(np.asarray(k_pages, dtype=np.float64), block_table[b], T)
        vc = gather_pages(np.asarray(v_pages, dtype=np.float64), block_table[b], T)
        out[b] = decode(q_new[b:b + 1], kc[None], vc[None], T, mode, window=window, scale=scale)[0]
    return out
