"""Pins of the dropout oracle (oracle/dropout.py) to things other than itself.

The pages ("Why FlashAttention Can Avoid a Square Attention Array ...",
"Backward can recreate tiles instead of retaining the square") only say that
the generator state, not the mask, is kept for the backward; the generator,
mask layout and rescaling are this implementation's reading, documented in the
oracle.  Pins: the generator's published known-answer vectors, the mask layout
written out element by element, the keep rate, the zero-probability case, the
expectation of the output, finite differences of the backward, and the D
identity.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import dropout as Dr

HERE = os.path.dirname(__file__)


def test_philox_known_answers():
    kat = json.load(open(os.path.join(HERE, "golden", "philox_kat.json")))
    for vec in kat["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], dtype=np.uint64)
        key = tuple(int(x, 16) for x in vec["key"])
        out = Dr.philox4x32_10(ctr, key)
        assert [f"{int(x):08x}" for x in out] == vec["output"]


def test_mask_layout_element_by_element():
    """byte(i, j) is byte j%4 of word i%4 of the call with counter
    (j//4, i//4, bh, offset); checked one element at a time on a ragged head."""
    tq, tk, bh, seed, off = 11, 13, 5, 0x123456789ABCDEF0, 7
    got = Dr.dropout_bytes(np.arange(tq), tk, bh, seed, off)
    for i in range(tq):
        for j in range(tk):
            w = Dr.philox4x32_10(np.array([j // 4, i // 4, bh, off], dtype=np.uint64),
                                 (seed & 0xFFFFFFFF, seed >> 32))
            assert got[i, j] == (int(w[i % 4]) >> (8 * (j % 4))) & 0xFF
    # a subset of rows gives the same bytes as the full evaluation
    rows = np.array([10, 3, 4, 0])
    assert np.array_equal(Dr.dropout_bytes(rows, tk, bh, seed, off), got[rows])


def test_threshold_and_scale():
    assert Dr.keep_threshold(0.0) == 0 and Dr.keep_scale(0) == 1.0
    assert Dr.keep_threshold(0.25) == 64 and Dr.keep_scale(64) == 256 / 192
    assert Dr.keep_threshold(0.1) == 26  # 25.6 rounds to 26
    assert Dr.keep_threshold(0.999) == 255  # at least one byte value is kept
    for bad in (-0.1, 1.0, 2.0):
        with pytest.raises(ValueError):
            Dr.keep_threshold(bad)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_keep_rate(p):
    """The kept fraction of a 512 x 512 head is (256 - t) / 256 within 5 sigma."""
    t = Dr.keep_threshold(p)
    keep = Dr.dropout_keep(np.arange(512), 512, 3, 2024, 0, t)
    q = (256 - t) / 256
    n = keep.size
    assert abs(keep.mean() - q) < 5 * math.sqrt(q * (1 - q) / n)


def test_masks_depend_on_every_counter_input():
    base = Dr.dropout_bytes(np.arange(64), 64, 1, 99, 0)
    for args in ((64, 2, 99, 0), (64, 1, 100, 0), (64, 1, 99, 1)):
        other = Dr.dropout_bytes(np.arange(64), *args)
        assert (other != base).mean() > 0.9
    assert np.array_equal(base, Dr.dropout_bytes(np.arange(64), 64, 1, 99, 0))


def test_zero_probability_is_plain_attention():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((37, 16)) for _ in range(3))
    for causal in (False, True):
        keep = Dr.dropout_keep(np.arange(37), 37, 0, 5, 0, 0)
        o, l = Dr.attention_forward_dropout(q, k, v, 0.25, causal, keep, 0)
        o0, l0 = A.attention_forward(q, k, v, 0.25, causal)
        assert np.array_equal(o, o0) and np.array_equal(l, l0)


def test_expected_output_is_the_undropped_output():
    """Averaged over seeds, the dropped output approaches the plain one; a
    missing or wrong rescale of the kept weights shifts the mean by ~10%."""
    rng = np.random.default_rng(2)
    tq, tk, d = 8, 64, 4
    q, k = rng.standard_normal((tq, d)), rng.standard_normal((tk, d))
    v = 1.0 + 0.1 * rng.standard_normal((tk, d))
    p = 0.1
    t = Dr.keep_threshold(p)
    o0, _ = A.attention_forward(q, k, v, 0.5, False)
    acc = np.zeros_like(o0)
    n_seed = 400
    for s in range(n_seed):
        keep = Dr.dropout_keep(np.arange(tq), tk, 0, s, 0, t)
        acc += Dr.attention_forward_dropout(q, k, v, 0.5, False, keep, t)[0]
    mean = acc / n_seed
    # per-seed std of an output element is below 0.1 here; 6 sigma of the mean
    assert np.abs(mean - o0).max() < 6 * 0.1 / math.sqrt(n_seed)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    rng = np.random.default_rng(3)
    n, d, scale, p = 6, 3, 0.7, 0.3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    t = Dr.keep_threshold(p)
    keep = Dr.dropout_keep(np.arange(n), n, 2, 11, 4, t)
    assert 0 < keep.sum() < keep.size

    def loss(q_, k_, v_):
        return float((Dr.attention_forward_dropout(q_, k_, v_, scale, causal, keep, t)[0] * do).sum())

    dq, dk, dv, dvec = Dr.attention_backward_dropout(q, k, v, do, scale, causal, keep, t)
    h = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - g).max() < 1e-7
    # D is the row sum of dO * O with the dropped output
    o, _ = Dr.attention_forward_dropout(q, k, v, scale, causal, keep, t)
    assert np.allclose(dvec, (do * o).sum(axis=1), atol=1e-13)


def test_bhnd_wrappers_use_the_head_index():
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((2, 3, 9, 4)) for _ in range(4))
    o, l = Dr.dropout_forward_bhnd(q, k, v, 0.5, True, 0.2, 77, 3)
    t = Dr.keep_threshold(0.2)
    for b in range(2):
        for h in range(3):
            keep = Dr.dropout_keep(np.arange(9), 9, b * 3 + h, 77, 3, t)
            ref = Dr.attention_forward_dropout(q[b, h], k[b, h], v[b, h], 0.5, True, keep, t)
            assert np.array_equal(o[b, h], ref[0]) and np.array_equal(l[b, h], ref[1])
    g = Dr.dropout_backward_bhnd(q, k, v, do, 0.5, True, 0.2, 77, 3)
    keep = Dr.dropout_keep(np.arange(9), 9, 1 * 3 + 2, 77, 3, t)
    ref = Dr.attention_backward_dropout(q[1, 2], k[1, 2], v[1, 2], do[1, 2], 0.5, True, keep, t)
    for x, y in zip(g, ref):
        assert np.array_equal(x[1, 2], y)
