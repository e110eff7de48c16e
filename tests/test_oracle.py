"""Pins for the CPU float64 oracle, independent of the oracle's own formulas.

Each test checks the oracle against something it cannot get from itself:
values the pages print for a worked example (tests/golden/pages_examples.json),
closed forms, brute-force per-row loops written with ``math``, a library
routine (torch's float64 softmax, SDPA and autograd), finite differences, or
an invariant of the mathematics.  All run on the CPU.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))
LN2 = math.log(2.0)


# --------------------------------------------------------------------- worked examples
def test_two_block_example_gives_twenty_thirds():
    g = GOLDEN["two_block"]
    q = np.array(g["q"])
    k = np.array([[0.0], [0.0], [LN2], [LN2]])  # scores = q.k with q = 1, scale 1
    v = np.array(g["v"])[:, None]
    o, lse = oracle.attention_forward(q, k, v, g["scale"])
    assert abs(o[0, 0] - 20.0 / 3.0) <= 1e-14
    assert round(float(o[0, 0]), 3) == g["expected_output_printed"]
    assert abs(o[0, 0] - g["wrong_equal_average"]) > 1.0
    assert abs(lse[0] - math.log(6.0)) <= 1e-15
    ot, lt, tiles = oracle.tiled_forward(q, k, v, g["scale"], block_q=1, block_k=g["block_k"])
    assert tiles == 2
    assert abs(ot[0, 0] - 20.0 / 3.0) <= 1e-14 and abs(lt[0] - math.log(6.0)) <= 1e-15
    # the per-block statistics the page walks through
    tr = oracle.online_normalizer_trace([[0.0, 0.0], [LN2, LN2]])
    assert tr[0][0] == 0.0 and tr[0][1] == g["block1"]["sum"]
    assert abs(tr[1][2] - g["rescale_of_block1"]) <= 1e-16
    assert abs(tr[1][1] - 3.0) <= 1e-15  # 2*(1/2) + 2


def test_four_number_online_example():
    g = GOLDEN["four_numbers"]
    tr = oracle.online_normalizer_trace(g["blocks"])
    (m1, l1, _), (m2, l2, a2) = tr
    assert m1 == g["after_block1_max"]
    assert f"{l1:.4f}" == g["after_block1_sum_4dp"]
    assert f"{a2:.2e}" == g["rescale_2e"]
    assert m2 == 10.0
    assert f"{l2:.6f}" == g["final_sum_6dp"]
    dense = sum(math.exp(x - 10.0) for blk in g["blocks"] for x in blk)
    assert f"{dense:.6f}" == g["dense_sum_6dp"]
    assert abs(l2 - dense) <= 1e-15
    assert abs(oracle.logsumexp_by_blocks([1.0, 2.0, 10.0, 0.0], block_size=2) - (10.0 + math.log(dense))) <= 1e-15


def test_late_max_in_final_key_tile():
    g = GOLDEN["late_max"]
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    exact = 4.0 - 6.0 / (3.0 + math.exp(20.0))
    o, _ = oracle.attention_forward(q, k, v, 1.0)
    ot, _, _ = oracle.tiled_forward(q, k, v, 1.0, block_q=g["block_q"], block_k=g["block_k"])
    assert abs(o[0, 0] - exact) <= 1e-15
    assert abs(ot[0, 0] - exact) <= 1e-15
    assert f"{ot[0, 0]:.7f}" == g["printed_7dp"]


def test_blockwise_logsumexp_guards_and_seeded_example():
    g = GOLDEN["streaming_lse"]
    assert oracle.logsumexp_by_blocks(np.full(4, -np.inf)) == -np.inf
    assert oracle.logsumexp_by_blocks(np.array([])) == -np.inf
    # a block of pure -inf in the middle is skipped, not turned into NaN
    x = np.array([-np.inf, -np.inf, 1.0, 2.0, -np.inf, -np.inf, 0.5])
    want = math.log(math.exp(1.0) + math.exp(2.0) + math.exp(0.5))
    assert abs(oracle.logsumexp_by_blocks(x, block_size=2) - want) <= 1e-14
    torch.manual_seed(g["torch_manual_seed"])
    xs = (torch.randn(g["count"]) * g["multiplier"]).double().numpy()
    got = oracle.logsumexp_by_blocks(xs, block_size=g["block"])
    assert f"{got:.8f}" == g["streaming_printed_8dp"]
    assert abs(got - float(g["dense_fp32_printed_8dp"])) < g["page_tolerance"]
    for blk in (1, 3, 64, 1000, 4096):
        assert abs(oracle.logsumexp_by_blocks(xs, block_size=blk) - got) <= 1e-12


# --------------------------------------------------------------------- closed forms and brute force
def test_rows_of_weights_sum_to_one():
    """With V = I the output is the weight matrix itself."""
    rng = np.random.default_rng(11)
    for causal in (False, True):
        q, k = rng.normal(size=(40, 7)), rng.normal(size=(40, 7)) * 3
        p, _ = oracle.attention_forward(q, k, np.eye(40), 0.7, causal)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-14
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


def test_uniform_scores_average_visible_values():
    rng = np.random.default_rng(12)
    n, dv = 33, 5
    v = rng.normal(size=(n, dv))
    q = np.zeros((n, 4))
    k = rng.normal(size=(n, 4))
    o, lse = oracle.attention_forward(q, k, v, 0.5, causal=False)
    assert np.max(np.abs(o - v.mean(axis=0))) <= 1e-14
    assert np.max(np.abs(lse - math.log(n))) <= 1e-14
    o, lse = oracle.attention_forward(q, k, v, 0.5, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(o - prefix)) <= 1e-14
    assert np.max(np.abs(lse - np.log(np.arange(1, n + 1)))) <= 1e-14


def _brute_row(qrow, i, k, v, scale, causal):
    """softmax(scale q.k) v for one query, with plain Python loops."""
    scores = []
    for j in range(len(k)):
        if causal and j > i:
            continue
        scores.append((j, scale * sum(a * b for a, b in zip(qrow, k[j]))))
    m = max(s for _, s in scores)
    w = [(j, math.exp(s - m)) for j, s in scores]
    tot = sum(x for _, x in w)
    out = [sum(x * v[j][c] for j, x in w) / tot for c in range(len(v[0]))]
    return out, m + math.log(tot)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_brute_force_loops(causal):
    rng = np.random.default_rng(13)
    q, k, v = rng.normal(size=(9, 4)), rng.normal(size=(9, 4)) * 2, rng.normal(size=(9, 3))
    o, lse = oracle.attention_forward(q, k, v, 0.9, causal, chunk=4)
    for i in range(9):
        ob, lb = _brute_row(q[i].tolist(), i, k.tolist(), v.tolist(), 0.9, causal)
        assert np.max(np.abs(o[i] - ob)) <= 1e-13
        assert abs(lse[i] - lb) <= 1e-13


def test_forward_matches_torch_float64_softmax_and_sdpa():
    rng = np.random.default_rng(14)
    for tq, tk, d, dv in [(50, 50, 16, 16), (37, 53, 8, 11), (64, 64, 64, 64)]:
        for causal in ([False, True] if tq == tk else [False]):
            q, k, v = rng.normal(size=(tq, d)), rng.normal(size=(tk, d)), rng.normal(size=(tk, dv))
            scale = 1 / math.sqrt(d)
            o, lse = oracle.attention_forward(q, k, v, scale, causal)
            tq_, tk_, tv_ = (torch.from_numpy(x) for x in (q, k, v))
            ref = F.scaled_dot_product_attention(tq_[None, None], tk_[None, None], tv_[None, None],
                                                 is_causal=causal, scale=scale)[0, 0].numpy()
            s = (tq_ @ tk_.T) * scale
            if causal:
                s = s.masked_fill(torch.triu(torch.ones(tq, tk, dtype=torch.bool), 1), -torch.inf)
            assert np.max(np.abs(o - ref)) <= 1e-12
            assert np.max(np.abs(lse - torch.logsumexp(s, -1).numpy())) <= 1e-12


def test_non_square_causal_is_upper_left():
    g = GOLDEN["non_square_causal"]
    rng = np.random.default_rng(15)
    for tq, tk in g["shapes_tq_tk"]:
        q, k, v = rng.normal(size=(tq, g["d"])), rng.normal(size=(tk, g["d"])), rng.normal(size=(tk, g["dv"]))
        scale = 1 / math.sqrt(g["d"])
        o, _ = oracle.attention_forward(q, k, v, scale, causal=True)
        ot, _, _ = oracle.tiled_forward(q, k, v, scale, True, g["block_q"], g["block_k"])
        ref = F.scaled_dot_product_attention(*(torch.from_numpy(x)[None, None] for x in (q, k, v)),
                                             is_causal=True)[0, 0].numpy()
        assert np.max(np.abs(o - ref)) <= 1e-12
        assert np.max(np.abs(ot - ref)) <= 1e-12


def test_empty_key_sequence_policy():
    o, lse = oracle.attention_forward(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 5)), 0.5)
    assert o.shape == (3, 5) and np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse, tiles = oracle.tiled_forward(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 5)), 0.5)
    assert tiles == 0 and np.all(o == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------- the blocked model
def test_tiled_equals_one_shot_on_ragged_blocks():
    g = GOLDEN["tiled_vs_dense_sweep"]
    rng = np.random.default_rng(16)
    # upper-left causal masking is defined for any (Tq, Tk), so every shape
    # runs both ways, with every tile shape of the fixture
    cases = [(shape, causal, blocks) for shape in g["shapes_tq_tk_d_dv"] for causal in (False, True)
             for blocks in g["blocks_q_k"]]
    worst = 0.0
    for (tq, tk, d, dv), causal, (bq, bk) in cases:
        q, k, v = rng.normal(size=(tq, d)), rng.normal(size=(tk, d)), rng.normal(size=(tk, dv))
        scale = 1 / math.sqrt(d)
        o, l, _ = oracle.tiled_forward(q, k, v, scale, causal, bq, bk)
        oe, le = oracle.attention_forward(q, k, v, scale, causal)
        worst = max(worst, np.max(np.abs(o - oe)), np.max(np.abs(l - le)))
    assert worst <= 1e-12


def test_causal_tile_counts_match_the_page():
    for case in GOLDEN["causal_tile_counts"]["cases"]:
        T, blk = case["T"], case["block"]
        q = np.zeros((T, 1))
        _, _, tiles = oracle.tiled_forward(q, q, q, 1.0, True, blk, blk)
        _, _, total = oracle.tiled_forward(q, q, q, 1.0, False, blk, blk)
        assert tiles == case["computed"] and total == case["total"]
        assert round(100 * (1 - tiles / total)) == case["skipped_pct"]


def test_permutation_invariance_non_causal():
    g = GOLDEN["permutation"]
    rng = np.random.default_rng(3)
    q, k, v = rng.normal(size=(g["tq"], g["d"])), rng.normal(size=(g["tk"], g["d"])), rng.normal(size=(g["tk"], g["dv"]))
    perm = rng.permutation(g["tk"])
    o1, l1, _ = oracle.tiled_forward(q, k, v, 0.2, False, g["block_q"], g["block_k"])
    o2, l2, _ = oracle.tiled_forward(q, k[perm], v[perm], 0.2, False, g["block_q"], g["block_k"])
    assert np.max(np.abs(o1 - o2)) <= 1e-13 and np.max(np.abs(l1 - l2)) <= 1e-13
    o3, _ = oracle.attention_forward(q, k[perm], v[perm], 0.2)
    assert np.max(np.abs(o1 - o3)) <= 1e-13


def test_forward_rows_and_batched_wrapper_agree_with_full():
    rng = np.random.default_rng(17)
    q, k, v = (rng.normal(size=(2, 3, 70, 8)) for _ in range(3))
    ob, lb = oracle.attention_forward_bhnd(q, k, v, 0.3, causal=True)
    rows = np.array([0, 5, 33, 69])
    os_, ls_ = oracle.attention_forward_bhnd(q, k, v, 0.3, causal=True, rows=rows)
    for b in range(2):
        for h in range(3):
            o, l = oracle.attention_forward(q[b, h], k[b, h], v[b, h], 0.3, True)
            assert np.array_equal(ob[b, h], o) and np.array_equal(lb[b, h], l)
            assert np.max(np.abs(os_[b, h] - o[rows])) <= 1e-15
            assert np.max(np.abs(ls_[b, h] - l[rows])) <= 1e-15


# --------------------------------------------------------------------- backward
def _objective(q, k, v, do, scale, causal):
    o, _ = oracle.attention_forward(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_finite_differences(causal):
    rng = np.random.default_rng(18)
    n, d = 5, 3
    q, k, v, do = (rng.normal(size=(n, d)) for _ in range(4))
    scale, h = 0.8, 1e-6
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _objective(**{**args, name: xp}, do=do, scale=scale, causal=causal)
            fm = _objective(**{**args, name: xm}, do=do, scale=scale, causal=causal)
            fd[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(fd - grad)) <= 1e-7, name


@pytest.mark.parametrize("tq,tk,dv", [(3, 6, 3), (6, 3, 2), (1, 4, 3), (5, 1, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_non_square_matches_central_finite_differences(tq, tk, dv, causal):
    """Tq != Tk (upper-left causal mask) and dv != d, against finite
    differences of the forward: pins the gradients of the general shapes
    (keys past the last query row get zero gradients under the mask)."""
    rng = np.random.default_rng(100 + 10 * tq + tk)
    d = 3
    q, k = rng.normal(size=(tq, d)), rng.normal(size=(tk, d))
    v, do = rng.normal(size=(tk, dv)), rng.normal(size=(tq, dv))
    scale, h = 0.7, 1e-6
    dq, dk, dv_, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    assert dq.shape == q.shape and dk.shape == k.shape and dv_.shape == v.shape
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv_)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _objective(**{**args, name: xp}, do=do, scale=scale, causal=causal)
            fm = _objective(**{**args, name: xm}, do=do, scale=scale, causal=causal)
            fd[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(fd - grad)) <= 1e-7, name
    if causal and tk > tq:
        assert np.all(dk[tq:] == 0) and np.all(dv_[tq:] == 0)


def test_backward_matches_torch_float64_autograd():
    rng = np.random.default_rng(19)
    for causal in (False, True):
        n, d = 45, 16
        arrs = [rng.normal(size=(n, d)) for _ in range(4)]
        dq, dk, dv, _ = oracle.attention_backward(*arrs, 0.25, causal, chunk=16)
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in arrs[:3])
        s = (tq @ tk.T) * 0.25
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), -torch.inf)
        (torch.softmax(s, -1) @ tv).backward(torch.tensor(arrs[3]))
        for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(a - b.numpy())) <= 1e-12


def test_backward_invariants():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i; D_i = dO_i . O_i."""
    rng = np.random.default_rng(20)
    for causal in (False, True):
        q, k, v, do = (rng.normal(size=(64, 8)) for _ in range(4))
        dq, dk, dv, dvec = oracle.attention_backward(q, k, v, do, 0.35, causal, chunk=20)
        o, _ = oracle.attention_forward(q, k, v, 0.35, causal)
        assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12
        assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-12
        assert np.max(np.abs(dvec - (do * o).sum(axis=1))) <= 1e-12


def test_backward_batched_wrapper():
    rng = np.random.default_rng(21)
    q, k, v, do = (rng.normal(size=(1, 2, 30, 8)) for _ in range(4))
    res = oracle.attention_backward_bhnd(q, k, v, do, 0.3, True)
    for h in range(2):
        single = oracle.attention_backward(q[0, h], k[0, h], v[0, h], do[0, h], 0.3, True)
        for a, b in zip(res, single):
            assert np.array_equal(a[0, h], b)
