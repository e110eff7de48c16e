"""GPU parity of attention dropout (fa_fwd_dropout / fa_bwd_dropout) against
the float64 dropout oracle.  The mask is regenerated from (seed, offset) by
the forward and by both backward kernels ("Backward can recreate tiles instead
of retaining the square", second page), so the gradients only match when all
three kernels rebuild the same mask the oracle draws.  Tolerances as in
test_gpu_parity: O max-abs 1e-2 / relative L2 5e-3, gradients 1e-2 / 2e-2
(the max-abs gate scaled by the keep factor 1/(1-p), see gmax),
L 1e-3.
"""

import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_16_amd as fa
from exact_io_aware_16_amd import inputs as I
from oracle import attention as A
from oracle import dropout as Dr

pytestmark = pytest.mark.gpu

O_MAX, O_REL = 1e-2, 5e-3
G_MAX, G_REL = 1e-2, 2e-2
L_MAX = 1e-3


def gmax(p):
    """Max-abs gate of the gradients under dropout.  Kept weights are
    multiplied by r = 256 / (256 - t) (t / 256 the applied probability), and
    so are O, dV and the dropout terms of dS: the absolute error of the
    bf16-rounded weights scales with r while the relative error does not.
    The absolute gate is therefore G_MAX * r (relative L2 stays G_REL); r = 1
    without dropout."""
    t = min(255, int(math.floor(256 * p + 0.5)))
    return G_MAX * 256 / (256 - t)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def errs(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0, 0.0
    nref = np.linalg.norm(ref)
    return float(np.abs(x - ref).max()), float(np.linalg.norm(x - ref) / nref) if nref > 0 else 0.0


def inputs(B, H, N, d, seed, with_do=True):
    w = I.Workload(f"drop_{B}_{H}_{N}_{d}", seed, B, H, N, d, False, "bf16")
    return I.make_inputs(w, with_do=with_do)


def gpu(t, *names):
    return [t[n].cuda() for n in names]


CASES = [(1, 2, 64, 64), (1, 2, 200, 128), (1, 2, 1000, 64), (2, 3, 517, 128)]


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", CASES)
def test_dropout_forward_and_backward(B, H, N, d, causal, p):
    seed, offset = 0x9E3779B97F4A7C15 ^ (N * 131 + d), 3
    t = inputs(B, H, N, d, 900 + N + d)
    scale = 1 / math.sqrt(d)
    say(f"dropout B={B} H={H} N={N} d={d} causal={causal} p={p}")
    q, k, v, do = gpu(t, "q", "k", "v", "do")
    o, l, p_applied = fa.forward_dropout(q, k, v, p, seed, offset, causal=causal)
    assert p_applied == round(256 * p) / 256
    dq, dk, dv = fa.backward_dropout(q, k, v, o, l, do, p, seed, offset, causal=causal)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (I.to_f64(t[n]) for n in ("q", "k", "v", "do"))
    oref, lref = Dr.dropout_forward_bhnd(q64, k64, v64, scale, causal, p, seed, offset)
    me, re_ = errs(o.cpu().numpy(), oref)
    le, _ = errs(l.cpu().numpy(), lref)
    say(f"  O max-abs {me:.3e} rel-L2 {re_:.3e}  L max-abs {le:.3e}")
    assert me <= O_MAX and re_ <= O_REL and le <= L_MAX
    gref = Dr.dropout_backward_bhnd(q64, k64, v64, do64, scale, causal, p, seed, offset)
    for name, x, ref in (("dQ", dq, gref[0]), ("dK", dk, gref[1]), ("dV", dv, gref[2])):
        ge, gr = errs(x.cpu().numpy(), ref)
        say(f"  {name} max-abs {ge:.3e} rel-L2 {gr:.3e}")
        assert ge <= gmax(p) and gr <= G_REL, name


def test_dropout_in_the_large_grid_launch():
    # >= 2 workgroups per CU: the 4-wave forward rather than the split one;
    # 64 heads, the oracle checks a sample of them
    B, H, N, d, p, seed = 4, 16, 1024, 128, 0.2, 12345
    t = inputs(B, H, N, d, 951)
    q, k, v, do = gpu(t, "q", "k", "v", "do")
    say("dropout large grid B=4 H=16 N=1024 d=128 causal")
    o, l, _ = fa.forward_dropout(q, k, v, p, seed, 0, causal=True)
    dq, dk, dv = fa.backward_dropout(q, k, v, o, l, do, p, seed, 0, causal=True)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    t_ = Dr.keep_threshold(p)
    for b, h in ((0, 0), (1, 7), (3, 15)):
        q64, k64, v64, do64 = (I.to_f64(t[n])[b, h] for n in ("q", "k", "v", "do"))
        keep = Dr.dropout_keep(np.arange(N), N, b * H + h, seed, 0, t_)
        oref, lref = Dr.attention_forward_dropout(q64, k64, v64, scale, True, keep, t_)
        me, re_ = errs(o[b, h].cpu().numpy(), oref)
        le, _ = errs(l[b, h].cpu().numpy(), lref)
        assert me <= O_MAX and re_ <= O_REL and le <= L_MAX, (b, h)
        gref = Dr.attention_backward_dropout(q64, k64, v64, do64, scale, True, keep, t_)
        for name, x, ref in (("dQ", dq, gref[0]), ("dK", dk, gref[1]), ("dV", dv, gref[2])):
            ge, gr = errs(x[b, h].cpu().numpy(), ref)
            assert ge <= gmax(p) and gr <= G_REL, (name, b, h)
        say(f"  head ({b},{h}) O max-abs {me:.3e}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_dropout_forward_rising_scores(d, causal):
    """Every query all ones and keys rising by about 400 base-2 units along
    the sequence: against a reference from the first key tile the weights
    leave float32, and the forward restarts against the exact row max.  The
    regenerated mask of the restart is the same, so O and L match the
    dropout oracle."""
    B, H, N, p, seed = 1, 2, 1200, 0.2, 4242
    c = (1 / math.sqrt(d)) * math.log2(math.e)
    g = torch.Generator("cpu").manual_seed(970 + d)
    ramp = torch.linspace(0.0, 400.0 / (c * d), N)[None, None, :, None]
    q = torch.ones((B, H, N, d)).to(torch.bfloat16)
    k = (ramp + 0.05 * torch.randn((B, H, N, d), generator=g)).to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    say(f"dropout rising scores d={d} causal={causal}")
    o, l, _ = fa.forward_dropout(q.cuda(), k.cuda(), v.cuda(), p, seed, 0, causal=causal)
    torch.cuda.synchronize()
    q64, k64, v64 = (x.to(torch.float64).numpy() for x in (q, k, v))
    oref, lref = Dr.dropout_forward_bhnd(q64, k64, v64, 1 / math.sqrt(d), causal, p, seed, 0)
    me, re_ = errs(o.cpu().numpy(), oref)
    le, _ = errs(l.cpu().numpy(), lref)
    say(f"  O max-abs {me:.3e} rel-L2 {re_:.3e}  L max-abs {le:.3e}")
    assert me <= O_MAX and re_ <= O_REL and le <= L_MAX


def test_dropout_forward_rising_scores_large_grid():
    """The same restart in the 4-wave launch (512 workgroups, two per CU):
    d = 64, 64 heads with keys rising by about 400 base-2 units; a sample of
    heads against the dropout oracle."""
    B, H, N, d, p, seed = 1, 64, 1024, 64, 0.3, 4343
    c = (1 / math.sqrt(d)) * math.log2(math.e)
    g = torch.Generator("cpu").manual_seed(975)
    ramp = torch.linspace(0.0, 400.0 / (c * d), N)[None, None, :, None]
    q = torch.ones((B, H, N, d)).to(torch.bfloat16)
    k = (ramp + 0.05 * torch.randn((B, H, N, d), generator=g)).to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    say("dropout rising scores, large grid, d=64 causal")
    o, l, _ = fa.forward_dropout(q.cuda(), k.cuda(), v.cuda(), p, seed, 0, causal=True)
    torch.cuda.synchronize()
    t_ = Dr.keep_threshold(p)
    for h in (0, 21, 63):
        q64, k64, v64 = (x[0, h].to(torch.float64).numpy() for x in (q, k, v))
        keep = Dr.dropout_keep(np.arange(N), N, h, seed, 0, t_)
        oref, lref = Dr.attention_forward_dropout(q64, k64, v64, 1 / math.sqrt(d), True, keep, t_)
        me, re_ = errs(o[0, h].cpu().numpy(), oref)
        le, _ = errs(l[0, h].cpu().numpy(), lref)
        say(f"  head {h}: O max-abs {me:.3e} rel-L2 {re_:.3e}  L max-abs {le:.3e}")
        assert me <= O_MAX and re_ <= O_REL and le <= L_MAX, h


def test_dropout_zero_probability_is_the_plain_path():
    t = inputs(1, 2, 300, 128, 961)
    q, k, v, do = gpu(t, "q", "k", "v", "do")
    o0, l0 = fa.forward(q, k, v, causal=True)
    o1, l1, p0 = fa.forward_dropout(q, k, v, 0.0, 77, causal=True)
    assert p0 == 0.0
    g0 = fa.backward(q, k, v, o0, l0, do, causal=True)
    g1 = fa.backward_dropout(q, k, v, o1, l1, do, 0.0, 77, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_dropout_mask_follows_seed_and_offset():
    t = inputs(1, 1, 256, 64, 962)
    q, k, v = gpu(t, "q", "k", "v")
    a = fa.forward_dropout(q, k, v, 0.3, 5, 0)[0]
    b = fa.forward_dropout(q, k, v, 0.3, 5, 0)[0]
    c = fa.forward_dropout(q, k, v, 0.3, 6, 0)[0]
    e = fa.forward_dropout(q, k, v, 0.3, 5, 1)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, e)
