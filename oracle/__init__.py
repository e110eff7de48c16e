"""CPU float64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; both are fed the same seeded inputs by the test harness.

Sources (the three pages on FlashAttention):
  * "FlashAttention: The Matrix You Never Have to Write Down"
    (maitreyasuin.github.io) -- sections "What attention computes",
    "What stops us", "The identity", "From softmax to attention", "Build it",
    "Check it", "Causal masking".
  * "Why FlashAttention Can Avoid a Square Attention Array Without Making
    Attention Linear" (leviathansystems.co) -- sections "Tiles need a shared
    softmax normalization", "A two-block example", "Backward can recreate
    tiles".

Functions and what pins each one (tests/test_oracle.py):
  attention_forward   plain materialised definition.  Pinned by the two-block
                      example (20/3), the late-max example, uniform-score
                      closed form, brute-force per-row loops, torch SDPA.
  attention_backward  chain rule on the definition (the pages give no
                      gradient equations; this is the textbook derivation).
                      Pinned by central finite differences, by torch
                      autograd of a float64 softmax, and by the row-sum
                      invariants of dK and dV.
  tiled_forward       the pages' blocked form: per-tile partial states merged
                      by the logsumexp identity, used to show that the online
                      rescale reaches the one-shot result.  Pinned by the
                      two-block example, the late max, the causal tile counts
                      (36/64, 528/1024) and equality with attention_forward
                      on ragged block sizes.
  logsumexp_by_blocks the one-pass (max, sum) reduction with its guards;
  online_normalizer_trace  its per-block trace.  Pinned by the four-number
                      example and the seeded 1000-value example printed on
                      the first page.
  dropout (module)    dropout whose mask the backward regenerates from the
                      generator state ("Backward can recreate tiles", second
                      page): Philox4x32-10 pinned by its published
                      known-answer vectors; mask layout pinned element by
                      element; keep rate, p = 0, the expectation of the
                      output, finite differences and the D identity pin the
                      forward and backward (tests/test_oracle_dropout.py).
  varlen (module)     packed variable-length sequences (the tip on PyTorch
                      calls under "What it doesn't solve", first page:
                      padded rows cost work): per-sequence plain attention,
                      pinned against one masked softmax over the whole packed
                      axis and its torch autograd (tests/test_oracle_varlen.py).
"""

from .attention import (
    attention_forward,
    attention_backward,
    attention_forward_bhnd,
    attention_backward_bhnd,
    tiled_forward,
    logsumexp_by_blocks,
    online_normalizer_trace,
)
from . import dropout, varlen

__all__ = [
    "attention_forward",
    "attention_backward",
    "attention_forward_bhnd",
    "attention_backward_bhnd",
    "tiled_forward",
    "logsumexp_by_blocks",
    "online_normalizer_trace",
    "dropout",
    "varlen",
]
