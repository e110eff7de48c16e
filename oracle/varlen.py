"""Variable-length packed attention: sequences of different lengths share one
token axis, and each attends only within itself.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module, and it shares no code with the HIP library.

Source: "FlashAttention: The Matrix You Never Have to Write Down"
(maitreyasuin.github.io), the tips on PyTorch calls under "What it doesn't
solve": when every sequence of a batch is padded to the longest, a fused
kernel still spends work on the padded positions, so for batches of mixed
lengths the page recommends packing the sequences (or a kernel that takes
variable lengths).  The page fixes no layout; this implementation's reading:

  * Q, K, V are [H, total, d] (head-major): sequence b occupies rows
    cu[b] .. cu[b+1]-1 of every head, with cu non-decreasing, cu[0] = 0 and
    cu[B] = total; O is [H, total, dv], L is [H, total].
  * Row i of sequence b attends to the keys of sequence b only; causal
    masking is upper-left within the sequence (key j hidden iff j > i).
  * A sequence of length 0 contributes no rows.
"""

import numpy as np

from .attention import attention_backward, attention_forward


def _segments(cu):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu must start at 0 and be non-decreasing")
    return [(int(cu[b]), int(cu[b + 1])) for b in range(cu.size - 1)]


def varlen_forward(q, k, v, cu, scale, causal=False):
    """Per sequence and head, the plain attention of attention_forward."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    H, total = q.shape[0], q.shape[1]
    o = np.zeros((H, total, v.shape[2]))
    lse = np.zeros((H, total))
    for s0, s1 in _segments(cu):
        for h in range(H):
            o[h, s0:s1], lse[h, s0:s1] = attention_forward(q[h, s0:s1], k[h, s0:s1], v[h, s0:s1], scale, causal)
    return o, lse


def varlen_backward(q, k, v, do, cu, scale, causal=False):
    """Per sequence and head, attention_backward.  Returns (dQ, dK, dV, D)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    H, total = q.shape[0], q.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dvec = np.zeros((H, total))
    for s0, s1 in _segments(cu):
        for h in range(H):
            r = attention_backward(q[h, s0:s1], k[h, s0:s1], v[h, s0:s1], do[h, s0:s1], scale, causal)
            dq[h, s0:s1], dk[h, s0:s1], dv[h, s0:s1], dvec[h, s0:s1] = r
    return dq, dk, dv, dvec


def segment_mask(cu, causal):
    """Boolean [total, total] visibility of the packed axis: same sequence,
    and (causal) key position <= query position."""
    total = int(np.asarray(cu)[-1])
    seg = np.zeros((total,), dtype=np.int64)
    for b, (s0, s1) in enumerate(_segments(cu)):
        seg[s0:s1] = b
    vis = seg[:, None] == seg[None, :]
    if causal:
        pos = np.arange(total)
        vis &= pos[None, :] <= pos[:, None]
    return vis
