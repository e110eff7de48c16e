"""Pins of the variable-length oracle (oracle/varlen.py).

The per-sequence loop is checked against a different formulation of the same
definition: one softmax over the whole packed token axis with an explicit
visibility mask (same sequence, and key <= query when causal), for the
outputs, and torch float64 autograd of that masked formulation for the
gradients.  Sequences of length 0 and a single sequence are covered.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import varlen as VL

CUS = [[0, 5, 5, 17, 18, 40], [0, 64], [0, 0, 3], [0, 1, 2, 3]]


def _draw(cu, H=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    total = cu[-1]
    return [rng.standard_normal((H, total, d)) for _ in range(4)]


def _masked_torch(q, k, v, cu, scale, causal):
    vis = torch.from_numpy(VL.segment_mask(cu, causal))
    s = torch.einsum("htd,hsd->hts", q, k) * scale
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return p @ v, torch.logsumexp(s, dim=-1)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cu", CUS)
def test_per_sequence_equals_packed_masked_softmax(cu, causal):
    q, k, v, do = _draw(cu)
    o, l = VL.varlen_forward(q, k, v, cu, 0.3, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ot, lt = _masked_torch(tq, tk, tv, cu, 0.3, causal)
    assert np.allclose(o, ot.detach().numpy(), atol=1e-13)
    assert np.allclose(l, lt.detach().numpy(), atol=1e-13)
    (ot * torch.from_numpy(do)).sum().backward()
    dq, dk, dv, dvec = VL.varlen_backward(q, k, v, do, cu, 0.3, causal)
    for x, g in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(x, g.grad.numpy(), atol=1e-12)
    assert np.allclose(dvec, (do * o).sum(axis=-1), atol=1e-12)


def test_single_sequence_is_plain_attention():
    q, k, v, _ = _draw([0, 50], H=1)
    o, l = VL.varlen_forward(q, k, v, [0, 50], 0.5, True)
    o0, l0 = A.attention_forward(q[0], k[0], v[0], 0.5, True)
    assert np.array_equal(o[0], o0) and np.array_equal(l[0], l0)


def test_segment_mask_is_block_diagonal():
    m = VL.segment_mask([0, 2, 2, 5], False)
    expect = np.zeros((5, 5), dtype=bool)
    expect[:2, :2] = True
    expect[2:, 2:] = True
    assert np.array_equal(m, expect)
    mc = VL.segment_mask([0, 2, 2, 5], True)
    assert np.array_equal(mc, expect & np.tri(5, dtype=bool))


def test_invalid_offsets_rejected():
    for bad in ([1, 4], [0, 4, 3], []):
        with pytest.raises(ValueError):
            VL.varlen_forward(np.zeros((1, 4, 2)), np.zeros((1, 4, 2)), np.zeros((1, 4, 2)), bad, 1.0)
