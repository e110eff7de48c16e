"""fa_bwd_noalloc, the backward entry point that allocates nothing, against
the existing fa_bwd (caller workspace) on the same inputs: two calls in a
row, the second on a smaller problem, each compared element by element with
fa_bwd's gradients (the same kernels run, so they must agree bitwise, and so
within the gradient tolerance of test_gpu_parity).  Also the host-side
rejection of problems larger than the built-in scratch."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_16_amd as fa
from exact_io_aware_16_amd import inputs as I

pytestmark = pytest.mark.gpu

G_MAX, G_REL = 1e-2, 2e-2
FA_ERR_SCRATCH = 8


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(q, k, v, o, l, do, causal, scale):
    B, H, N, d = q.shape
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = fa.library().fa_bwd_noalloc(p(q), p(k), p(v), p(o), p(l), p(do), p(dq), p(dk), p(dv), B, H, N, d,
                                     ctypes.c_float(scale), int(causal),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.status_string(st)
    return dq, dk, dv


def test_noalloc_backward_equals_workspace_backward_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call on the larger problem, second on a smaller one: the second
    # reads only rows its own preprocess wrote in the shared scratch
    for B, H, N, d, causal, seed in ((2, 16, 1000, 128, True, 71), (1, 3, 300, 64, False, 72)):
        say(f"noalloc backward B{B} H{H} N{N} d{d} causal={causal}")
        w = I.Workload(f"noalloc_{B}_{H}_{N}_{d}", seed, B, H, N, d, causal, "bf16", backward=True)
        t = I.make_inputs(w)
        q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
        o, l = fa.forward(q, k, v, causal=causal)
        ref = fa.backward(q, k, v, o, l, do, causal=causal)
        got = _noalloc(q, k, v, o, l, do, causal, w.scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            a64, b64 = a.double().cpu().numpy(), b.double().cpu().numpy()
            me = float(np.max(np.abs(a64 - b64)))
            rel = float(np.linalg.norm(a64 - b64) / max(np.linalg.norm(b64), 1e-300))
            say(f"  {name}: max-abs {me:.3e} rel-L2 {rel:.3e} against fa_bwd")
            assert me <= G_MAX and rel <= G_REL, name
            assert torch.equal(a, b), name


def test_noalloc_rejects_problems_beyond_its_scratch():
    lib = fa.library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails first
    st = lib.fa_bwd_noalloc(*([fake] * 9), 1, 2, (1 << 20) + 1, 64, ctypes.c_float(0.125), 0, None)
    assert st == FA_ERR_SCRATCH
    assert "scratch" in fa.status_string(st)
