"""Attention dropout whose mask the backward regenerates instead of storing.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module, and it shares no code with the HIP library.

Source: "Why FlashAttention Can Avoid a Square Attention Array Without Making
Attention Linear" (leviathansystems.co), section "Backward can recreate tiles
instead of retaining the square": under dropout, only the generator state is
kept from the forward, and the backward regenerates the identical mask from it,
so no N x N mask is ever stored.  The pages name no
generator, no mask layout and no rescaling rule; the choices below are this
implementation's reading and are stated once here.

Generator.  Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror
and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): a 128-bit
counter and a 64-bit key go through ten rounds; each round multiplies counter
words 0 and 2 by the two Philox multipliers, keeps both halves of the 64-bit
products, and mixes the high halves with the other two words and the key; the
key is advanced by the two Weyl constants between rounds.  It is pinned by the
published known-answer vectors (tests/golden/philox_kat.json).

Mask.  For head (b, h) of H heads, query row i and key j (0-based, within the
head), with seed s (64 bit) and offset o (32 bit):
    words  = Philox4x32-10(counter = (j div 4, i div 4, b*H + h, o),
                           key     = (s mod 2^32, s div 2^32))
    byte   = bits 8 (j mod 4) .. 8 (j mod 4) + 7 of words[i mod 4]
    t      = min(255, floor(256 p + 1/2))          (p = dropout probability)
    keep   = byte >= t
One generator call covers a 4 x 4 block of (query, key) pairs.  The keep
probability is (256 - t) / 256 and kept weights are multiplied by
256 / (256 - t), so the expected output equals the output without dropout.

Forward.  P = softmax(scale Q K^T) (masked as usual), O = (P * keep * r) V with
r = 256 / (256 - t); L is the logsumexp of the scores, untouched by dropout.
Backward (chain rule on that definition, our derivation):
    dV = (P * keep * r)^T dO,   dP = (dO V^T) * keep * r,
    D_i = sum_j P_ij dP_ij = dO_i . O_i,   dS = P * (dP - D),
    dQ = scale dS K,   dK = scale dS^T Q.
"""

import math

import numpy as np

from .attention import _as2d, _scores, _softmax_rows

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counters, key):
    """Philox4x32 with ten rounds.

    counters: integer array of shape (..., 4) (each word < 2^32); key: a pair
    of 32-bit integers.  Returns a uint32 array of the same shape.
    """
    c = np.asarray(counters, dtype=np.uint64) & _MASK32
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = np.uint64(key[0] & 0xFFFFFFFF), np.uint64(key[1] & 0xFFFFFFFF)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = x0 * m0  # < 2^64: exact in uint64
        p1 = x2 * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def keep_threshold(p):
    """Byte threshold t for dropout probability p (0 <= p < 1)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(math.floor(256.0 * p + 0.5)))


def keep_scale(t):
    """Factor applied to kept weights: 256 / (256 - t)."""
    return 256.0 / (256 - t)


def dropout_bytes(rows, tk, bh, seed, offset):
    """The generator byte of every (row, key) pair: shape (len(rows), tk)."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0 or tk == 0:
        return np.zeros((rows.size, tk), dtype=np.uint8)
    jb = np.arange((tk + 3) // 4, dtype=np.int64)
    ib = np.unique(rows // 4)
    ctr = np.zeros((ib.size, jb.size, 4), dtype=np.uint64)
    ctr[..., 0] = jb[None, :]
    ctr[..., 1] = ib[:, None]
    ctr[..., 2] = bh
    ctr[..., 3] = offset
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))  # (ib, jb, 4)
    pos = np.searchsorted(ib, rows // 4)
    w = words[pos][:, :, :]  # (n_rows, jb, 4)
    w = np.take_along_axis(w, (rows % 4)[:, None, None].repeat(jb.size, axis=1), axis=2)[..., 0]  # (n, jb)
    by = np.stack([(w >> (8 * e)) & 0xFF for e in range(4)], axis=-1).reshape(rows.size, -1)
    return by[:, :tk].astype(np.uint8)


def dropout_keep(rows, tk, bh, seed, offset, t):
    """Boolean keep mask of shape (len(rows), tk)."""
    return dropout_bytes(rows, tk, bh, seed, offset) >= t


def attention_forward_dropout(q, k, v, scale, causal, keep, t, rows=None):
    """Forward with dropout on the normalised weights.

    keep: boolean (n_rows, Tk) mask of the evaluated rows; t: the byte
    threshold it was made with.  Returns (O, L); L ignores dropout.
    """
    q = _as2d(q, "Q")
    k = _as2d(k, "K")
    v = _as2d(v, "V")
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((idx.size, v.shape[1]))
    lse = np.full((idx.size,), -np.inf)
    if k.shape[0] == 0 or idx.size == 0:
        return o, lse
    s = _scores(q[idx], idx, k, scale, causal)
    p, m, l = _softmax_rows(s)
    o = (p * keep * keep_scale(t)) @ v
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_backward_dropout(q, k, v, do, scale, causal, keep, t):
    """Gradients of sum(dO * O) for O = attention_forward_dropout(...).

    keep covers every query row.  Returns (dQ, dK, dV, D).
    """
    q = _as2d(q, "Q")
    k = _as2d(k, "K")
    v = _as2d(v, "V")
    do = _as2d(do, "dO")
    tq = q.shape[0]
    if k.shape[0] == 0 or tq == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros((tq,))
    ri = np.arange(tq)
    s = _scores(q, ri, k, scale, causal)
    p, _, _ = _softmax_rows(s)
    r = keep_scale(t)
    pd = p * keep * r
    dv = pd.T @ do
    dp = (do @ v.T) * keep * r
    drow = (p * dp).sum(axis=1)
    ds = p * (dp - drow[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv, drow


def dropout_forward_bhnd(q, k, v, scale, causal, p_drop, seed, offset, rows=None):
    """attention_forward_dropout over every head of [B, H, N, d] arrays."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H = q.shape[:2]
    t = keep_threshold(p_drop)
    idx = np.arange(q.shape[2]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, H, idx.size, v.shape[3]))
    lse = np.zeros((B, H, idx.size))
    for b in range(B):
        for h in range(H):
            keep = dropout_keep(idx, k.shape[2], b * H + h, seed, offset, t)
            o[b, h], lse[b, h] = attention_forward_dropout(q[b, h], k[b, h], v[b, h], scale, causal, keep, t, rows=idx)
    return o, lse


def dropout_backward_bhnd(q, k, v, do, scale, causal, p_drop, seed, offset):
    """attention_backward_dropout over every head of [B, H, N, d] arrays."""
    q = np.asarray(q, dtype=np.float64)
    B, H, n = q.shape[:3]
    t = keep_threshold(p_drop)
    out = [np.zeros_like(q), np.zeros(np.shape(k)), np.zeros(np.shape(v)), np.zeros((B, H, n))]
    for b in range(B):
        for h in range(H):
            keep = dropout_keep(np.arange(n), np.shape(k)[2], b * H + h, seed, offset, t)
            res = attention_backward_dropout(q[b, h], np.asarray(k[b, h], np.float64), np.asarray(v[b, h], np.float64),
                                             np.asarray(do[b, h], np.float64), scale, causal, keep, t)
            for x, y in zip(out, res):
                x[b, h] = y
    return tuple(out)
