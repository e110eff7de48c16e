"""Seeded synthetic inputs for attention, shared by tests, bench and smoke.

This module holds no attention arithmetic: it only draws seeded normal
values, rounds them to the storage dtype and picks sampled row indices.  The
HIP path and the CPU oracle both receive exactly these values.

Recipe: each tensor is drawn in float32 from ``torch.Generator('cpu')``
seeded with ``1000 * case + {q: 1, k: 2, v: 3, dO: 4}``, multiplied by its
standard deviation, then rounded to bfloat16 with round-to-nearest-even
(``Tensor.to(torch.bfloat16)``) unless the workload is float32.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

_TENSOR_SEED = {"q": 1, "k": 2, "v": 3, "do": 4}


@dataclass(frozen=True)
class Workload:
    """One attention problem: [B, H, N, d] tensors and how they are drawn."""

    name: str
    case: int            # seed base: seeds are 1000 * case + tensor id
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str           # "bf16" or "f32" storage of Q, K, V (and dO)
    qk_std: float = 1.0  # standard deviation of Q and K
    v_std: float = 1.0   # standard deviation of V (and dO)
    backward: bool = False
    sample_rows: int = 0  # >0: parity on this many seeded rows per head
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def fwd_flop(self) -> float:
        """4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


# The five workloads the hot path is measured and checked on.
TINY_F32 = Workload("fwd_f32_b1h1n512d64", 1, 1, 1, 512, 64, False, "f32",
                    note="tiny exact check, float32 inputs, forward only")
FWD_4K_D128 = Workload("fwd_bf16_b1h8n4096d128", 2, 1, 8, 4096, 128, False, "bf16",
                       note="forward, non-causal")
CAUSAL_8K_D64_WIDE = Workload("fwd_bf16_causal_b4h16n8192d64_qk3", 3, 4, 16, 8192, 64, True,
                              "bf16", qk_std=3.0,
                              note="forward, causal, Q and K ~ N(0, 3^2): the running max moves often")
CAUSAL_32K_D128 = Workload("fwd_bf16_causal_b1h8n32768d128", 4, 1, 8, 32768, 128, True, "bf16",
                           sample_rows=256, note="long-context causal forward")
# the forward workload at twice the sequence length: per-head HBM bytes of
# the two should differ by about 2x (K and V re-reads absorbed on chip), not 4x
FWD_8K_D128 = Workload("fwd_bf16_b1h8n8192d128", 2, 1, 8, 8192, 128, False, "bf16",
                       note="forward, non-causal, twice the sequence length of the forward workload")
FWDBWD_4K_D128 = Workload("fwdbwd_bf16_causal_b2h16n4096d128", 5, 2, 16, 4096, 128, True, "bf16",
                          backward=True, note="forward + recompute backward, causal")

WORKLOADS = [TINY_F32, FWD_4K_D128, CAUSAL_8K_D64_WIDE, CAUSAL_32K_D128, FWDBWD_4K_D128]


def draw(shape, seed, std=1.0, dtype="bf16"):
    """Seeded N(0, std^2) values of ``shape`` stored as ``dtype`` (CPU tensor)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * float(std)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, with_do=None):
    """Q, K, V (and dO when the workload has a backward) as CPU tensors."""
    shape = (w.B, w.H, w.N, w.d)
    out = {
        "q": draw(shape, 1000 * w.case + _TENSOR_SEED["q"], w.qk_std, w.dtype),
        "k": draw(shape, 1000 * w.case + _TENSOR_SEED["k"], w.qk_std, w.dtype),
        "v": draw(shape, 1000 * w.case + _TENSOR_SEED["v"], w.v_std, w.dtype),
    }
    if w.backward if with_do is None else with_do:
        out["do"] = draw(shape, 1000 * w.case + _TENSOR_SEED["do"], w.v_std, w.dtype)
    return out


def make_general(B, H, Nq, Nk, d, dv, seed, std=1.0, with_do=False):
    """Seeded bf16 Q [B,H,Nq,d], K [B,H,Nk,d], V [B,H,Nk,dv] (CPU tensors) for
    the general forward contract, and dO [B,H,Nq,dv] when with_do; seeds
    1000*seed + {q:1, k:2, v:3, do:4}."""
    base = 1000 * int(seed)
    t = {"q": draw((B, H, Nq, d), base + _TENSOR_SEED["q"], std),
         "k": draw((B, H, Nk, d), base + _TENSOR_SEED["k"], std),
         "v": draw((B, H, Nk, dv), base + _TENSOR_SEED["v"])}
    if with_do:
        t["do"] = draw((B, H, Nq, dv), base + _TENSOR_SEED["do"])
    return t


# Decoding: one query row per head against a long key sequence (split-KV).
DECODE_32K = {"name": "decode_bf16_b1h32nq1nk32768d128", "B": 1, "H": 32, "Nq": 1, "Nk": 32768, "d": 128,
              "dv": 128, "seed": 6}


def sample_rows(N, count, seed):
    """Rows 0 and N-1 plus ``count - 2`` distinct other rows, sorted."""
    if count >= N:
        return np.arange(N, dtype=np.int64)
    rng = np.random.default_rng(int(seed))
    middle = rng.choice(np.arange(1, N - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], middle]).astype(np.int64))


def to_f64(t):
    """Exact float64 copy of a CPU/GPU tensor's stored values, as numpy."""
    return t.detach().to("cpu", torch.float64).numpy()
