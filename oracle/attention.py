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


def _merge(state_a, state_b):
    """Combine two partial softmax states over disjoint key sets.

    A state (m, l, o) summarises a set of scores x_j (with values v_j) of one
    row: m = max x_j, l = sum_j e^(x_j - m), o = sum_j e^(x_j - m) v_j.  The
    identity of "The identity: you can fix what you already wrote" (first
    page), used across tiles in "Tiles need a shared softmax normalization"
    (second page): with m = max(m_a, m_b), the union has
    l = e^(m_a - m) l_a + e^(m_b - m) l_b and likewise for o.  A set with no
    finite score has m = -inf, l = 0, o = 0 and weight 0; works elementwise
    on arrays of rows (o may be None when only (m, l) is tracked).
    """
    ma, la, oa = state_a
    mb, lb, ob = state_b
    m = np.maximum(ma, mb)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isneginf(ma), 0.0, np.exp(ma - np.where(np.isneginf(m), 0.0, m)))
        wb = np.where(np.isneginf(mb), 0.0, np.exp(mb - np.where(np.isneginf(m), 0.0, m)))
    l = wa * la + wb * lb
    o = None if oa is None else np.asarray(wa)[..., None] * oa + np.asarray(wb)[..., None] * ob
    return m, l, o


def _block_state(x, vals=None):
    """Partial state (m, l, o) of each row of a score block x (rows x keys)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1) if x.shape[-1] else np.full(x.shape[:-1], _NEG_INF)
    shift = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(x - shift[..., None])  # -inf scores give exactly 0
    l = e.sum(axis=-1)
    return m, l, (None if vals is None else e @ vals)


def online_normalizer_trace(blocks):
    """Running (max, sum, factor) of one score row consumed block by block.

    After each block that holds a finite score, the running state is merged
    with the block's own state; ``factor`` is the multiplier the merge applies
    to the sum kept so far, e^(m_old - m_new) (0 before anything was kept) --
    the rescale of "The identity" (first page).  Blocks with no finite score
    leave the state unchanged and produce no entry.  Returns a list of
    (m, l, factor).
    """
    state = (_NEG_INF, 0.0, None)
    trace = []
    for blk in blocks:
        b = _block_state(np.asarray(blk, dtype=np.float64).ravel()[None, :])
        if np.isneginf(b[0][0]):
            continue
        m_old = state[0]
        m, l, _ = _merge(state, (b[0][0], b[1][0], None))
        factor = 0.0 if m_old == _NEG_INF else math.exp(m_old - m)
        state = (float(m), float(l), None)
        trace.append((state[0], state[1], factor))
    return trace


def logsumexp_by_blocks(x, block_size=16):
    """ln(sum_j e^(x_j)) of a 1-D array, reading it block_size values at a time.

    Each block's (max, sum) is merged into the running one (see _merge); an
    input with no finite value gives -inf rather than the log of 0 ("The
    identity", first page).
    """
    x = np.asarray(x, dtype=np.float64).ravel()
    state = (_NEG_INF, 0.0, None)
    for a in range(0, x.size, block_size):
        b = _block_state(x[a:a + block_size][None, :])
        state = _merge(state, (b[0][0], b[1][0], None))
    m, l = float(state[0]), float(state[1])
    return _NEG_INF if l == 0.0 else m + math.log(l)


def tiled_forward(q, k, v, scale, causal=False, block_q=16, block_k=16):
    """The blocked form of attention of "From softmax to attention" (first page).

    Queries are cut into blocks of block_q rows and keys into blocks of
    block_k.  Every (query block, key block) score tile yields one partial
    state per row, merged into the row's running state by the identity of
    _merge, in increasing key order; the division by l happens once, at the
    end, and L = m + ln l.  With the causal mask ("Causal masking", first
    page) a key block whose first key comes after the block's last query is
    never formed -- every score in it would be -inf.  Returns (O, L, tiles);
    the largest query-by-key array built is one tile.
    """
    q = _as2d(q, "Q")
    k = _as2d(k, "K")
    v = _as2d(v, "V")
    if block_q <= 0 or block_k <= 0:
        raise ValueError("tile sides must be at least 1")
    tq, tk, dv = q.shape[0], k.shape[0], v.shape[1]
    out = np.zeros((tq, dv), dtype=np.float64)
    lse = np.full((tq,), _NEG_INF, dtype=np.float64)
    tiles = 0
    for r0 in range(0, tq, block_q):
        rows = np.arange(r0, min(tq, r0 + block_q))
        starts = [c0 for c0 in range(0, tk, block_k) if not (causal and c0 > rows[-1])]
        state = (np.full(rows.size, _NEG_INF), np.zeros(rows.size), np.zeros((rows.size, dv)))
        for c0 in starts:
            cols = np.arange(c0, min(tk, c0 + block_k))
            x = _scores(q[rows], rows, k[cols], scale, False)
            if causal:
                x = np.where(cols[None, :] > rows[:, None], _NEG_INF, x)
            state = _merge(state, _block_state(x, v[cols]))
            tiles += 1
        m, l, o = state
        seen = l > 0
        out[rows] = np.where(seen[:, None], o / np.where(seen, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            lse[rows] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), _NEG_INF)
    return out, lse, tiles
