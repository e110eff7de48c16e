"""Plain float64 attention: the definition, its gradient, and the blocked model.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every array here is a
numpy float64 array; callers convert bf16/fp32 inputs with ``np.float64`` on
the exact values the GPU sees.

Conventions fixed by the pages:
  * O = softmax(scale * Q K^T) V, each row of weights summing to one
    ("What attention computes", first page).
  * softmax is the max-shifted form e^(x-m) / sum e^(x-m)
    ("What stops us: softmax needs the whole row", first page).
  * The per-row statistic L is the natural-log logsumexp of the *scaled*
    scores, L = m + ln(l) ("Build it", first page).
  * Causal masking is upper-left: key j is hidden from query i when j > i,
    the convention of F.scaled_dot_product_attention(is_causal=True)
    ("Build it", note "Two things this deliberately doesn't do").
  * No keys at all gives O = 0 and L = -inf, by the stated policy
    ("Check it", empty key sequence).
"""

import math

import numpy as np

_NEG_INF = -np.inf


def _as2d(x, name):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError(f"{name} must be rank 2 (one head), got shape {x.shape}")
    return x


def _scores(q_rows, row_index, k, scale, causal):
    """scale * q_rows @ k.T with the upper-left causal mask applied.

    ``row_index`` holds the absolute query position of each row in q_rows, so
    that a chunk or a sample of rows is masked exactly as in the full matrix.
    """
    s = (q_rows @ k.T) * scale
    if causal:
        key_pos = np.arange(k.shape[0])[None, :]
        s = np.where(key_pos > row_index[:, None], _NEG_INF, s)
    return s


def _softmax_rows(s):
    """Max-shifted softmax of each row, plus the row max and row sum.

    Returns (P, m, l) with P = e^(s - m) / l.  A row that is entirely -inf
    (only possible with no visible key) gets P = 0, m = -inf, l = 0.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def attention_forward(q, k, v, scale, causal=False, rows=None, chunk=512):
    """Exact attention for one head, materialising full score rows.

    q: (Tq, d), k: (Tk, d), v: (Tk, dv).  Returns (O, L): O of shape
    (n_rows, dv) and L = logsumexp of the scaled (masked) scores, natural log.
    ``rows`` selects which query positions to evaluate (all by default); the
    mask uses their absolute positions.  Rows are processed ``chunk`` at a time
    so that a long sequence never needs the whole square at once -- each chunk
    still holds complete rows, so nothing about the arithmetic is blocked.
    """
    q = _as2d(q, "Q")
    k = _as2d(k, "K")
    v = _as2d(v, "V")
    if q.shape[1] != k.shape[1]:
        raise ValueError("Q and K widths differ")
    if k.shape[0] != v.shape[0]:
        raise ValueError("K and V lengths differ")
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    n = idx.shape[0]
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), _NEG_INF, dtype=np.float64)
    if k.shape[0] == 0 or n == 0:
        return o, lse
    for c0 in range(0, n, chunk):
        ri = idx[c0:c0 + chunk]
        s = _scores(q[ri], ri, k, scale, causal)
        p, m, l = _softmax_rows(s)
        o[c0:c0 + chunk] = p @ v
        with np.errstate(divide="ignore"):
            lse[c0:c0 + chunk] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), _NEG_INF)
    return o, lse


def attention_backward(q, k, v, do, scale, causal=False, chunk=512):
    """Gradients of sum(dO * O) for O = attention_forward(q, k, v).

    The pages say only that the backward rebuilds the probability tiles from
    Q, K and the saved statistics; they give no equations.  This is the chain
    rule applied to the definition, with P recomputed from the definition
    (not from a saved L):
        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
    Masked pairs have P = 0 and hence dS = 0.  Returns (dQ, dK, dV, D).
    """
    q = _as2d(q, "Q")
    k = _as2d(k, "K")
    v = _as2d(v, "V")
    do = _as2d(do, "dO")
    tq = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros((tq,), dtype=np.float64)
    if k.shape[0] == 0 or tq == 0:
        return dq, dk, dv, dvec
    for c0 in range(0, tq, chunk):
        ri = np.arange(c0, min(tq, c0 + chunk))
        s = _scores(q[ri], ri, k, scale, causal)
        p, _, _ = _softmax_rows(s)
        g = do[ri]
        dv += p.T @ g
        dp = g @ v.T
        drow = (p * dp).sum(axis=1)
        ds = p * (dp - drow[:, None])
        dq[ri] = scale * (ds @ k)
        dk += scale * (ds.T @ q[ri])
        dvec[ri] = drow
    return dq, dk, dv, dvec


def attention_forward_bhnd(q, k, v, scale, causal=False, rows=None):
    """attention_forward applied to every (batch, head) of [B, H, N, d] arrays.

    ``rows`` may be None (all rows), an index array shared by every head, or a
    callable (b, h) -> index array.  Returns O [B, H, n, dv] and L [B, H, n].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H = q.shape[0], q.shape[1]
    outs, lses = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(H):
            r = rows(b, h) if callable(rows) else rows
            o, l = attention_forward(q[b, h], k[b, h], v[b, h], scale, causal, rows=r)
            ob.append(o)
            lb.append(l)
        outs.append(np.stack(ob))
        lses.append(np.stack(lb))
    return np.stack(outs), np.stack(lses)


def attention_backward_bhnd(q, k, v, do, scale, causal=False):
    """attention_backward applied to every (batch, head) of [B, H, N, d] arrays."""
    q = np.asarray(q, dtype=np.float64)
    B, H = q.shape[0], q.shape[1]
    res = [[attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
            for h in range(H)] for b in range(B)]
    return tuple(np.stack([np.stack([res[b][h][t] for h in range(H)]) for b in range(B)])
                 for t in range(4))


def online_normalizer_trace(blocks):
    """Running (max, sum, rescale factor) after each block of a score row.

    The online normalizer of "The identity: you can fix what you already
    wrote" (first page) and "Tiles need a shared softmax normalization"
    (second page): when a block raises the maximum from m to m_new, the sum
    kept so far is multiplied by e^(m - m_new) before the block's own terms
    are added.  The factor is forced to 0 while the running max is still
    -inf (nothing accumulated yet), and a block that is entirely -inf is
    skipped.  Returns a list of (m, l, factor) tuples, one per block that
    contributed.
    """
    m, l = _NEG_INF, 0.0
    trace = []
    for blk in blocks:
        blk = np.asarray(blk, dtype=np.float64)
        if blk.size == 0:
            continue
        bmax = float(blk.max())
        if bmax == _NEG_INF:
            continue
        m_new = max(m, bmax)
        factor = 0.0 if m == _NEG_INF else math.exp(m - m_new)
        l = l * factor + float(np.exp(blk - m_new).sum())
        m = m_new
        trace.append((m, l, factor))
    return trace


def streaming_logsumexp(x, block=7):
    """log(sum(exp(x))) in one pass over blocks of ``block`` values.

    Uses online_normalizer_trace; an input with no finite value returns -inf
    rather than log(0) ("The identity", first page).
    """
    x = np.asarray(x, dtype=np.float64).ravel()
    trace = online_normalizer_trace(x[i:i + block] for i in range(0, x.size, block))
    if not trace or trace[-1][1] == 0.0:
        return _NEG_INF
    m, l, _ = trace[-1]
    return m + math.log(l)


def tiled_forward(q, k, v, scale, causal=False, block_q=32, block_k=32):
    """The blocked recurrence of "From softmax to attention" (first page).

    For each block of query rows, three running quantities start at
    m = -inf, l = 0 and an unnormalised output of zeros.  Each key/value block
    visited (in increasing key order) gives a score tile S; with
    m_new = max(m, rowmax S) and factor a = e^(m - m_new) (0 while m is -inf),
    the update is l <- a*l + rowsum(e^(S - m_new)), O <- a*O + e^(S - m_new) V,
    m <- m_new.  The division by l happens once, after the last block, and
    L = m + ln(l).  With the causal mask, a key block that starts after the
    last query of the query block is never visited, nor is any later one.

    Returns (O, L, tiles) where ``tiles`` counts the score tiles computed.
    The largest query-by-key array built is one block_q x block_k tile.
    """
    q = _as2d(q, "Q")
    k = _as2d(k, "K")
    v = _as2d(v, "V")
    if block_q < 1 or block_k < 1:
        raise ValueError("block sizes must be positive")
    tq, tk, dv = q.shape[0], k.shape[0], v.shape[1]
    o = np.zeros((tq, dv), dtype=np.float64)
    lse = np.full((tq,), _NEG_INF, dtype=np.float64)
    tiles = 0
    if tk == 0:
        return o, lse, tiles
    for q0 in range(0, tq, block_q):
        qi = np.arange(q0, min(tq, q0 + block_q))
        run_m = np.full((qi.size,), _NEG_INF)
        run_l = np.zeros((qi.size,))
        acc = np.zeros((qi.size, dv))
        for k0 in range(0, tk, block_k):
            if causal and k0 > qi[-1]:
                break
            kj = slice(k0, min(tk, k0 + block_k))
            s = (q[qi] @ k[kj].T) * scale
            if causal:
                key_pos = np.arange(kj.start, kj.stop)[None, :]
                s = np.where(key_pos > qi[:, None], _NEG_INF, s)
            tiles += 1
            m_new = np.maximum(run_m, s.max(axis=1))
            # rows whose max is still -inf have seen no visible key yet: shift by 0
            shift = np.where(np.isneginf(m_new), 0.0, m_new)
            factor = np.where(np.isneginf(run_m), 0.0, np.exp(run_m - shift))
            e = np.exp(s - shift[:, None])
            run_l = factor * run_l + e.sum(axis=1)
            acc = factor[:, None] * acc + e @ v[kj]
            run_m = m_new
        o[qi] = acc / run_l[:, None]
        lse[qi] = run_m + np.log(run_l)
    return o, lse, tiles
