"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE, not part of the product.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never calls it and shares no code with it; the
two meet only on the seeded inputs.

Sources (the pages this follows):
  * everydayai.blog article "flash-attention-revolutionizing-transformer-efficiency"
    (no printed title; the text is synonym-spun, e.g. "Consideration" = Attention):
      - opening snippet ``standard_attention``: the definition
        softmax(Q K^T / sqrt(d_k)) V on (batch, seq, d) tensors;
      - "The Math Behind Flash Attention", formula 1 (softmax decomposition with
        the row maximum m) and formula 2 (softmax merger, garbled as printed);
      - "Enter Flash Attention": recomputation in the backward pass;
      - "The Impact of Flash Attention": exact computation, not an approximation.
  * scite.ai author page of Tri Dao, FlashAttention abstract: IO-aware *exact*
    attention; extension to block-sparse attention.

Parity status of each function (how it is pinned, in tests/test_oracle_*.py):
  forward / forward_rows      -- brute force, closed forms, torch fp64 SDPA, golden hand cases
  forward_blockwise / merge   -- equals the one-shot forward; the dropped-l mutation fails
  backward                    -- central finite differences, torch fp64 autograd, invariants
  backward_rows               -- equals `backward` on the sampled rows and keys (dense, causal,
                                 block-sparse, grouped heads) and torch fp64 autograd
  grouped-/multi-query heads  -- torch fp64 SDPA and autograd with enable_gqa, brute force and
                                 finite differences, K/V heads repeated == plain multi-head
  bf16_backward_bound         -- holds for a step-by-step simulation of a bf16 kernel's roundings,
                                 and is not vacuous (oracle/bounds.py)
  fp8 (oracle/fp8.py)         -- e4m3 rounding vs torch float8_e4m3fn; the Hadamard transform vs
                                 scipy (exact on integers); quantisation vs torch's conversion and
                                 exponent minimality; the P-rounding bound vs a simulation
"""

from .attention import (  # noqa: F401
    allowed,
    backward,
    backward_rows,
    forward,
    forward_blockwise,
    forward_rows,
    kv_head,
    merge_partials,
    probabilities,
)
from .brute import brute_backward_fd, brute_forward  # noqa: F401
from .bounds import bf16_backward_bound  # noqa: F401
from . import fp8  # noqa: F401
